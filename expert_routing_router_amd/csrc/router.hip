// Router of the DeepSeekMoE layer on gfx950: affinities, biased group-limited
// top-K and normalised gates (route_kernel, with a fused front end or fed by
// the tiled logits_kernel), and the per-expert loads (count_loads_kernel).
//
//   s_{i,t} = sigmoid(u_t . e_i)       -- DeepSeek-V3 Technical Report guides
//                                         (xyznot.com), "Metodo" section 2
//   top-K_r on s + b, gates from s      -- same section, gating equation; the
//                                         pwwt.cn note 1.1.2 (bias only routes)
//   groups ranked by the sum of their   -- pwwt.cn note 1.3 (node-limited
//   top K_r/M scores, at most M kept       routing; nodes = expert groups here)
//
// route_kernel: one workgroup (4 waves) owns 32 tokens and every expert (4
// tokens when the affinities are handed in). The front end
// writes the fp32 affinities of its tokens into LDS; the selection back end is
// one code path whatever the front end was (MFMA logits, fp64 logits, or
// affinities handed in by the caller), so the scores-in mode exercises exactly
// the production selection.
//
// Precision: the MFMA front end accumulates bf16 products (exact in fp32) in
// fp32 over 128-element chunks of d and sums the chunks in fp64; the sigmoid
// is evaluated in fp64 and rounded once to fp32. fp32 centroids are split into
// three bf16 terms (hi + mid + lo reproduces the fp32 value exactly), so the
// products stay exact on the bf16 MFMA path; the hi products and the much
// smaller mid+lo products go to separate accumulators so the small terms are
// not rounded against the large running sum.
#include "common.h"
#include "lds_dma.h"
#include "moe_internal.h"
#include <type_traits>

extern "C" __device__ unsigned int __ockl_wfred_max_u32(unsigned int);

namespace moe {

constexpr int RT_BT = 32;
constexpr int RT_BT_SEL = 4;
constexpr int RT_THREADS = 256;
constexpr int RT_NMAX = 256;
constexpr int RT_QMAX = 8;

template <int BT>
struct RouterLdsT {
  float s[BT][RT_NMAX];
  float b[RT_NMAX];
};
using RouterLds = RouterLdsT<RT_BT>;      // the fused front ends work on 32 tokens

__device__ __forceinline__ double sigmoid64(double z) {
  if (z >= 0.0) return 1.0 / (1.0 + exp(-z));
  double ez = exp(z);
  return ez / (1.0 + ez);
}

union V16 { i32x4 i; bf16x8 h; uint16_t s[8]; };

__device__ __forceinline__ void split3(const float* x, bf16x8& hi, bf16x8& mid, bf16x8& lo) {
  V16 a, b, c;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    float v = x[i];
    uint16_t h = f32_to_bf16(v);
    float r1 = v - bf16_to_f32(h);          // exact
    uint16_t m = f32_to_bf16(r1);
    float r2 = r1 - bf16_to_f32(m);         // exact
    a.s[i] = h; b.s[i] = m; c.s[i] = f32_to_bf16(r2);
  }
  hi = a.h; mid = b.h; lo = c.h;
}

// ---------------------------------------------------------------- front ends
// MFMA 16x16x32 bf16: lane l holds A row (l&15), B column (l&15), 8 k-values
// at k-group (l>>4); D element (4*(l>>4)+r, l&15) in register r.
// Wave w owns expert blocks w, w+4, ... (16 experts each) for all 32 tokens.
// Fragments are loaded straight from global memory three k-steps ahead of
// their MFMAs (four rotating register sets); every four k-steps (128 elements
// of d) the fp32 MFMA sums are flushed into fp64 accumulators.
template <bool SPLIT_E>
struct RouterFrag {
  bf16x8 a0, a1;
  typename std::conditional<SPLIT_E, f32x4, bf16x8>::type b[4][SPLIT_E ? 2 : 1];
};

template <bool SPLIT_E>
__device__ void front_mfma(const RouteArgs& a, RouterLds& sh, int t0) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, kg = lane >> 4;
  const int nblk = a.n_routed >> 4;
  const int nb = nblk > wave ? (nblk - wave + 3) >> 2 : 0;   // blocks wave, wave+4, ...
  const uint16_t* u = (const uint16_t*)a.u;
  const int ta0 = min(t0 + r16, a.T - 1), ta1 = min(t0 + 16 + r16, a.T - 1);
  const uint16_t* pa0 = u + (size_t)ta0 * a.d + kg * 8;
  const uint16_t* pa1 = u + (size_t)ta1 * a.d + kg * 8;
  // B rows of this wave's blocks; slots past nb (a wave with fewer blocks, or none when
  // N_r < 64) re-read block 0, which always exists, so every load stays inside E
  const uint16_t* pb16[4];
  const float* pb32[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int blk = j < nb ? wave + 4 * j : 0;
    const size_t row = (size_t)((blk << 4) + r16) * a.d + kg * 8;
    pb16[j] = (const uint16_t*)a.E + row;
    pb32[j] = (const float*)a.E + row;
  }
  const int nsteps = a.d >> 5;     // d % 128 == 0 on this path

  RouterFrag<SPLIT_E> f[4];
  auto load = [&](RouterFrag<SPLIT_E>& g, int step) __attribute__((always_inline)) {
    const int k = min(step, nsteps - 1) << 5;
    g.a0 = *(const bf16x8*)(pa0 + k);
    g.a1 = *(const bf16x8*)(pa1 + k);
#pragma unroll
    for (int j = 0; j < 4; j++) {
      if (!SPLIT_E) {
        *(bf16x8*)&g.b[j][0] = *(const bf16x8*)(pb16[j] + k);
      } else {
        *(f32x4*)&g.b[j][0] = *(const f32x4*)(pb32[j] + k);
        *(f32x4*)&g.b[j][1] = *(const f32x4*)(pb32[j] + k + 4);
      }
    }
  };

  double z64[2][4][4];
#pragma unroll
  for (int m = 0; m < 2; m++)
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int r = 0; r < 4; r++) z64[m][j][r] = 0.0;
  f32x4 acc[2][4], acs[2][4];
  auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < 2; m++)
#pragma unroll
      for (int j = 0; j < 4; j++) acc[m][j] = acs[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  };
  auto flush = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < 2; m++)
#pragma unroll
      for (int j = 0; j < 4; j++)
#pragma unroll
        for (int r = 0; r < 4; r++) {
          z64[m][j][r] += (double)acc[m][j][r];
          if (SPLIT_E) z64[m][j][r] += (double)acs[m][j][r];
        }
  };
  auto mfma = [&](const RouterFrag<SPLIT_E>& g) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 4; j++) {
      if (j < nb) {
        if (!SPLIT_E) {
          const bf16x8 B = *(const bf16x8*)&g.b[j][0];
          acc[0][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(g.a0, B, acc[0][j], 0, 0, 0);
          acc[1][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(g.a1, B, acc[1][j], 0, 0, 0);
        } else {
          float x[8];
          *(f32x4*)&x[0] = *(const f32x4*)&g.b[j][0];
          *(f32x4*)&x[4] = *(const f32x4*)&g.b[j][1];
          bf16x8 h, md, lo;
          split3(x, h, md, lo);
          acs[0][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(g.a0, lo, acs[0][j], 0, 0, 0);
          acs[1][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(g.a1, lo, acs[1][j], 0, 0, 0);
          acs[0][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(g.a0, md, acs[0][j], 0, 0, 0);
          acs[1][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(g.a1, md, acs[1][j], 0, 0, 0);
          acc[0][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(g.a0, h, acc[0][j], 0, 0, 0);
          acc[1][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(g.a1, h, acc[1][j], 0, 0, 0);
        }
      }
    }
  };

  load(f[0], 0);
  load(f[1], 1);
  load(f[2], 2);
  for (int s0 = 0; s0 < nsteps; s0 += 4) {      // nsteps % 4 == 0
    load(f[3], s0 + 3);
    zero_acc();
    mfma(f[0]);
    load(f[0], s0 + 4);
    mfma(f[1]);
    load(f[1], s0 + 5);
    mfma(f[2]);
    load(f[2], s0 + 6);
    mfma(f[3]);
    flush();
  }
#pragma unroll
  for (int m = 0; m < 2; m++)
#pragma unroll
    for (int j = 0; j < 4; j++)
      if (j < nb) {
        const int e = ((wave + 4 * j) << 4) + r16;
#pragma unroll
        for (int r = 0; r < 4; r++) sh.s[m * 16 + 4 * kg + r][e] = (float)sigmoid64(z64[m][j][r]);
      }
}

template <bool U_BF16, bool E_BF16>
__device__ void front_f64(const RouteArgs& a, RouterLds& sh, int t0, int nt) {
  for (int p = threadIdx.x; p < nt * a.n_routed; p += RT_THREADS) {
    const int t = p / a.n_routed, e = p - t * a.n_routed;
    double z = 0.0;
    for (int k = 0; k < a.d; k++) {
      const size_t iu = (size_t)(t0 + t) * a.d + k, ie = (size_t)e * a.d + k;
      const double x = U_BF16 ? bf16_to_f32(((const uint16_t*)a.u)[iu]) : ((const float*)a.u)[iu];
      const double w = E_BF16 ? bf16_to_f32(((const uint16_t*)a.E)[ie]) : ((const float*)a.E)[ie];
      z = fma(x, w, z);
    }
    sh.s[t][e] = (float)sigmoid64(z);
  }
}

// ---------------------------------------------------------------- selection
// v with lane l replaced by lane l ^ OFF's value
template <int OFF>
__device__ __forceinline__ float xor_lane(float v) {
  if constexpr (OFF < 32) return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1F | (OFF << 10)));
  else return __shfl_xor(v, 32, kWave);
}
// max over the aligned run of S lanes (S a power of two) that holds this lane
__device__ __forceinline__ float segment_max(float v, int S) {
  if (S > 1) v = fmaxf(v, xor_lane<1>(v));
  if (S > 2) v = fmaxf(v, xor_lane<2>(v));
  if (S > 4) v = fmaxf(v, xor_lane<4>(v));
  if (S > 8) v = fmaxf(v, xor_lane<8>(v));
  if (S > 16) v = fmaxf(v, xor_lane<16>(v));
  if (S > 32) v = fmaxf(v, xor_lane<32>(v));
  return v;
}

// Group scores when each group is an aligned run of S lanes of one expert slot
// (S a power of two, at most 64): every group's top-q scores are extracted at
// once by segmented max reductions, removing one holder of each maximum (the
// lowest lane) before the next; their fp32 sum is taken largest first, as in
// the per-lane loop it replaces. Returns lane g's group key (g < G), else 0.
__device__ __forceinline__ uint32_t group_keys_segmented(const RouteArgs& a, const float* b, const float* srow,
                                                         int lane, int S, int G, int q) {
  const int N = a.n_routed;
  const int segbase = lane & ~(S - 1);
  const uint64_t segmask = S == 64 ? ~0ull : ((1ull << S) - 1ull);
  float gsum[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    gsum[j] = -INFINITY;
    if (64 * j >= N) continue;
    const int e = lane + 64 * j;
    float v = -INFINITY;
    if (e < N) {
      v = a.group_score_biased ? srow[e] + b[e] : srow[e];
      if (v != v) v = -INFINITY;               // a NaN score never ranks
    }
    float acc = 0.f;
    for (int r = 0; r < q; r++) {
      const float m = segment_max(v, S);
      acc = r == 0 ? m : acc + m;
      if (r + 1 < q) {
        const uint64_t hit = (__ballot(v == m) >> segbase) & segmask;
        if (lane == segbase + __ffsll((unsigned long long)hit) - 1) v = -INFINITY;
      }
    }
    gsum[j] = acc;
  }
  // lane g < G takes group g's sum from slot (g*S)/64, lane (g*S)%64
  const int src = (lane * S) & 63, slot = (lane * S) >> 6;
  float mine = -INFINITY;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const float x = __shfl(gsum[j], src, kWave);
    if (slot == j) mine = x;
  }
  return lane < G ? max(ordered_f32(mine), 1u) : 0u;
}

// One wave per token. Expert e lives in lane (e & 63), slot (e >> 6). Each
// selection round is one wave reduction (device library, DPP based) for the
// largest ordered key and one ballot per slot for the lowest expert index
// holding it -- the total order (key desc, index asc); -0 and +0 share one
// ordered key.
template <int BT>
__device__ void select_tokens(const RouteArgs& a, RouterLdsT<BT>& sh, int t0, int nt) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int N = a.n_routed, K = a.top_k, G = a.n_groups, M = a.topk_groups, q = a.group_topk;
  const int S = N / G;
  const bool seg_groups = (S & (S - 1)) == 0 && S <= 64;
  for (int t = wave; t < nt; t += RT_THREADS / kWave) {
    const float* srow = sh.s[t];
    // ordered keys; 0 = not a candidate. A candidate's key is at least 1, so K rounds
    // always find K distinct experts in range. A NaN key takes 1, the lowest
    // candidate key: it ranks after every number (-inf included), as a NaN score
    // never ranks in the group scores either.
    uint32_t ok[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int e = lane + 64 * j;
      const float kv = e < N ? srow[e] + sh.b[e] : 0.f;
      ok[j] = e < N ? (kv != kv ? 1u : max(ordered_f32(kv), 1u)) : 0u;
    }
    if (G > 1) {
      uint32_t gk = 0u;
      if (seg_groups) {
        gk = group_keys_segmented(a, sh.b, srow, lane, S, G, q);
      } else if (lane < G) {
        float top[RT_QMAX];
#pragma unroll
        for (int i = 0; i < RT_QMAX; i++) top[i] = -INFINITY;
        for (int i = 0; i < S; i++) {
          const int e = lane * S + i;
          float v = a.group_score_biased ? srow[e] + sh.b[e] : srow[e];
#pragma unroll
          for (int j = 0; j < RT_QMAX; j++) {
            if (j < q && v > top[j]) { const float tmp = top[j]; top[j] = v; v = tmp; }
          }
        }
        float acc = top[0];
#pragma unroll
        for (int j = 1; j < RT_QMAX; j++)
          if (j < q) acc = acc + top[j];                    // fp32, largest first
        gk = max(ordered_f32(acc), 1u);
      }
      uint64_t chosen = 0ull;
      for (int m = 0; m < M; m++) {
        const uint32_t gmax = __ockl_wfred_max_u32(gk);
        const uint64_t holders = __ballot(lane < G && gk == gmax);     // lowest group index first
        if (gmax && holders) {
          const int g = (int)__builtin_ctzll(holders);
          chosen |= 1ull << g;
          if (lane == g) gk = 0u;
        }
      }
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int e = lane + 64 * j;
        if (e < N && !((chosen >> (e / S)) & 1ull)) ok[j] = 0u;
      }
    }
    // Round k: the largest key is one wave reduction; the lowest expert index
    // holding it comes from one ballot per slot (expert lane + 64 j, so the
    // first slot with a holder, then its lowest lane); it is wave-uniform, so
    // only one slot is touched to remove it.
    int my_e = 0;
    for (int k = 0; k < K; k++) {
      const uint32_t lmax = max(max(ok[0], ok[1]), max(ok[2], ok[3]));
      const uint32_t kmax = __ockl_wfred_max_u32(lmax);
      int e = -1;
      if (kmax) {
#pragma unroll
        for (int j = 3; j >= 0; j--) {
          const uint64_t m = __ballot(ok[j] == kmax);
          if (m) e = 64 * j + (int)__builtin_ctzll(m);
        }
#pragma unroll
        for (int j = 0; j < 4; j++)
          if ((e >> 6) == j && lane == (e & 63)) ok[j] = 0u;
      }
      if (lane == k) my_e = e;
    }
    // gate denominator: the selected scores in selection order, summed in fp64
    const float my_s = lane < K && my_e >= 0 ? srow[my_e] : 0.f;
    double sum = 0.0;
    for (int k = 0; k < K; k++) sum += (double)__int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_s), k));
    if (lane < K) {
      const float g = sum > 0.0 ? (float)((double)my_s / sum) : 1.0f / (float)K;
      const size_t o = (size_t)(t0 + t) * K + lane;
      a.idx[o] = my_e;
      a.gate[o] = g;
    }
  }
}

template <int FRONT, bool U_BF16, bool E_BF16, int BT = RT_BT>
__global__ __launch_bounds__(RT_THREADS) void route_kernel(RouteArgs a) {
  static_assert(FRONT == kFrontScoresIn || BT == RT_BT, "the fused front ends work on 32 tokens");
  __shared__ RouterLdsT<BT> sh;
  const int t0 = blockIdx.x * BT;
  const int nt = min(BT, a.T - t0);
  for (int e = threadIdx.x; e < a.n_routed; e += RT_THREADS) {
    sh.b[e] = a.b[e];
  }
  if constexpr (FRONT == kFrontScoresIn) {
    for (int p = threadIdx.x; p < nt * a.n_routed; p += RT_THREADS) {
      const int t = p / a.n_routed, e = p - t * a.n_routed;
      sh.s[t][e] = a.scores_in[(size_t)(t0 + t) * a.n_routed + e];
    }
  } else if constexpr (FRONT == kFrontMfma) {
    front_mfma<false>(a, sh, t0);
  } else if constexpr (FRONT == kFrontMfmaSplitE) {
    front_mfma<true>(a, sh, t0);
  } else {
    front_f64<U_BF16, E_BF16>(a, sh, t0, nt);
  }
  __syncthreads();
  if (a.scores_out) {
    for (int p = threadIdx.x; p < nt * a.n_routed; p += RT_THREADS) {
      const int t = p / a.n_routed, e = p - t * a.n_routed;
      a.scores_out[(size_t)(t0 + t) * a.n_routed + e] = sh.s[t][e];
    }
  }
  select_tokens(a, sh, t0, nt);
}

// ---------------------------------------------------------------- two-phase router
// For large batches the logits are better tiled over (tokens x experts) than
// one workgroup per 32 tokens x all experts (which streams the whole centroid
// matrix through every CU). Phase 1 (logits_kernel) computes the affinities
// of a 128-token x 64-expert tile and writes them to a scores buffer; phase 2
// is route_kernel in scores-in mode (the same selection code). Phase 1 does
// the same arithmetic as front_mfma -- the same 16x16x32 MFMAs on the same
// operands, fp32 partials over 128-element chunks of d summed in fp64 in chunk
// order, the split of fp32 centroids into hi/mid/lo bf16 planes, the same
// sigmoid -- so both routers give bit-identical affinities.
constexpr int LG_BT = 128;          // tokens per workgroup
constexpr int LG_BE = 64;           // experts per workgroup
constexpr int LG_BK = 64;           // bf16 elements per stage row (128 bytes)

template <int NPLANES>
struct LogitsCfg {
  static constexpr int U_BYTES = LG_BT * LG_BK * 2;       // 16 KB
  static constexpr int E_BYTES = LG_BE * LG_BK * 2;       // 8 KB per plane
  static constexpr int STAGE = U_BYTES + NPLANES * E_BYTES;
  static constexpr int STAGES = NPLANES == 1 ? 6 : 3;
  static constexpr int BYTES = STAGES * STAGE;
  static constexpr int U_PER_WAVE = LG_BT / 8 / 4;         // 1 KB blocks of 8 rows, 4 waves
  static constexpr int E_PER_WAVE = LG_BE / 8 / 4;
  static constexpr int LOADS = U_PER_WAVE + NPLANES * E_PER_WAVE;
  static_assert(BYTES <= 160 * 1024, "LDS budget");
};

// fp32 centroids -> three bf16 planes [3][N][d] with hi + mid + lo == value exactly
__global__ void split_planes_kernel(const float* E, uint16_t* planes, long n) {
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) {
    const float v = E[i];
    const uint16_t h = f32_to_bf16(v);
    const float r1 = v - bf16_to_f32(h);
    const uint16_t m = f32_to_bf16(r1);
    const float r2 = r1 - bf16_to_f32(m);
    planes[i] = h;
    planes[n + i] = m;
    planes[2 * n + i] = f32_to_bf16(r2);
  }
}

template <int NPLANES>
__global__ __launch_bounds__(256, 1) void logits_kernel(const uint16_t* __restrict__ u,
                                                        const uint16_t* __restrict__ planes, float* scores,
                                                        int T, int d, int N) {
  using C = LogitsCfg<NPLANES>;
  extern __shared__ __align__(16) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t0 = blockIdx.x * LG_BT, e0 = blockIdx.y * LG_BE;

  // ---- loads: one instruction fills 8 rows x 128 bytes; lane l writes row
  // l>>3, slot l&7 and fetches chunk slot ^ ((row >> 1) & 7)
  const int brow = lane >> 3;
  const int bchunk = (lane & 7) ^ ((((wave & 1) << 2) + (lane >> 4)) & 7);   // block parity = wave parity
  const i32x4 ur = rsrc_words(u, (long)T * d * 2);
  const i32x4 er = rsrc_words(planes, (long)NPLANES * N * d * 2);
  int uoff[C::U_PER_WAVE], eoff[NPLANES][C::E_PER_WAVE];
#pragma unroll
  for (int i = 0; i < C::U_PER_WAVE; i++) {
    const int t = t0 + (wave + 4 * i) * 8 + brow;
    uoff[i] = t < T ? (t * d + bchunk * 8) * 2 : kOutOfRange;
  }
#pragma unroll
  for (int p = 0; p < NPLANES; p++)
#pragma unroll
    for (int i = 0; i < C::E_PER_WAVE; i++) {
      const int e = e0 + (wave + 4 * i) * 8 + brow;
      eoff[p][i] = ((p * N + e) * d + bchunk * 8) * 2;
    }
  const uint32_t lds0 = lds_addr(lds);
  auto issue = [&](int kt, int buf) __attribute__((always_inline)) {
    const int koff = kt * LG_BK * 2;
    const uint32_t sb = lds0 + buf * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::U_PER_WAVE; i++) dma_b128(ur, uoff[i], koff, sb + (wave + 4 * i) * 1024);
#pragma unroll
    for (int p = 0; p < NPLANES; p++)
#pragma unroll
      for (int i = 0; i < C::E_PER_WAVE; i++)
        dma_b128(er, eoff[p][i], koff, sb + C::U_BYTES + p * C::E_BYTES + (wave + 4 * i) * 1024);
  };

  // ---- wave w: tokens 32w .. 32w+31 (two 16-row blocks) x the 64 experts (four blocks)
  const int r16 = lane & 15, kg = lane >> 4;
  const int sw = (r16 >> 1) & 7;
  int roff[2];
#pragma unroll
  for (int ks = 0; ks < 2; ks++) roff[ks] = r16 * 128 + (((ks * 4 + kg) ^ sw) << 4);
  double z64[2][4][4];
#pragma unroll
  for (int m = 0; m < 2; m++)
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int r = 0; r < 4; r++) z64[m][j][r] = 0.0;

  // operand fragments of one step: a[ks][m] (token blocks), b[ks][j][plane] (expert blocks)
  struct Frag { bf16x8 a[2][2]; bf16x8 b[2][4][NPLANES]; };
  // fp32 sums of one 128-element chunk: h from the hi plane, l from mid + lo
  struct Acc { f32x4 h[2][4]; f32x4 l[2][4]; };
  auto read_frags = [&](Frag& f, int buf) __attribute__((always_inline)) {
    const uint8_t* U = lds + buf * C::STAGE;
    const uint8_t* Ep = U + C::U_BYTES;
#pragma unroll
    for (int ks = 0; ks < 2; ks++) {
      f.a[ks][0] = *(const bf16x8*)(U + (wave * 32) * 128 + roff[ks]);
      f.a[ks][1] = *(const bf16x8*)(U + (wave * 32 + 16) * 128 + roff[ks]);
#pragma unroll
      for (int j = 0; j < 4; j++)
#pragma unroll
        for (int p = 0; p < NPLANES; p++)
          f.b[ks][j][p] = *(const bf16x8*)(Ep + p * C::E_BYTES + (j * 16) * 128 + roff[ks]);
    }
  };
  // one step's MFMAs; FIRST starts a chunk (the accumulators restart from zero)
  auto mma = [&](auto first_tag, Acc& A, const Frag& f) __attribute__((always_inline)) {
    constexpr bool FIRST = decltype(first_tag)::value;
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ks++)
#pragma unroll
      for (int j = 0; j < 4; j++)
#pragma unroll
        for (int m = 0; m < 2; m++) {
          const bool z = FIRST && ks == 0;
          if constexpr (NPLANES > 1) {
            A.l[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[ks][m], f.b[ks][j][2], z ? zero : A.l[m][j], 0, 0, 0);
            A.l[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[ks][m], f.b[ks][j][1], A.l[m][j], 0, 0, 0);
          }
          A.h[m][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[ks][m], f.b[ks][j][0], z ? zero : A.h[m][j], 0, 0, 0);
        }
  };
  auto fold = [&](const Acc& A) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < 2; m++)
#pragma unroll
      for (int j = 0; j < 4; j++)
#pragma unroll
        for (int r = 0; r < 4; r++) {
          z64[m][j][r] += (double)A.h[m][j][r];
          if (NPLANES > 1) z64[m][j][r] += (double)A.l[m][j][r];
        }
  };

  // Ring of S stage buffers, software-pipelined: step kt waits for stage kt+1
  // (S-2 younger stages may stay in flight) and for its own LDS reads of stage
  // kt, then a barrier (every wave holds stage kt in registers and sees stage
  // kt+1 in LDS); it refills stage kt's buffer with step kt+S, reads stage
  // kt+1's fragments (after the last step: the re-read copy, unused) and runs
  // stage kt's MFMAs. Chunks of 128 elements (two
  // steps) alternate between two accumulator sets, and a chunk's fp32 sums are
  // folded into fp64 (in chunk order) during the first step of the next chunk,
  // so LDS reads, MFMAs and the fp64 work of different steps overlap. Loads
  // past the last step re-read it into buffers that are never read again, so
  // the count per step is fixed.
  constexpr int S = C::STAGES;
  // three planes: the next fragments are read after this step's MFMAs, and one
  // accumulator set is used, so the registers of one fragment set and one
  // accumulator set suffice
  constexpr bool kEarlyReads = NPLANES == 1;
  const int nk = d / LG_BK;                    // even: d % 128 == 0
  Frag F0, F1;
  Acc A0, A1;
#pragma unroll
  for (int m = 0; m < 2; m++)
#pragma unroll
    for (int j = 0; j < 4; j++) A1.h[m][j] = A1.l[m][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < S; p++) issue(min(p, nk - 1), p);
  wait_vmcnt<(S - 1) * C::LOADS>();
  __syncthreads();
  read_frags(F0, 0);
  auto step = [&](auto first_tag, auto fold_tag, Acc& acc, const Acc& prev, const Frag& cur, Frag& nxt, int kt)
      __attribute__((always_inline)) {
    wait_vmcnt_lgkm0<(S - 2) * C::LOADS>();
    __syncthreads();
    issue(min(kt + S, nk - 1), kt % S);
    if (kEarlyReads) {
      read_frags(nxt, (kt + 1) % S);
      __builtin_amdgcn_sched_barrier(0);     // the reads go out before the MFMAs
    }
    mma(first_tag, acc, cur);
    if constexpr (decltype(fold_tag)::value) fold(prev);
    if (!kEarlyReads) {
      __builtin_amdgcn_sched_barrier(0);
      read_frags(nxt, (kt + 1) % S);
    }
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  int kt = 0;
  if constexpr (kEarlyReads) {
    for (; kt + 4 <= nk; kt += 4) {
      step(T_{}, T_{}, A0, A1, F0, F1, kt);
      step(F_{}, F_{}, A0, A1, F1, F0, kt + 1);
      step(T_{}, T_{}, A1, A0, F0, F1, kt + 2);
      step(F_{}, F_{}, A1, A0, F1, F0, kt + 3);
    }
    if (kt < nk) {                             // nk % 4 == 2: one more chunk
      step(T_{}, T_{}, A0, A1, F0, F1, kt);
      step(F_{}, F_{}, A0, A1, F1, F0, kt + 1);
      fold(A0);
    } else {
      fold(A1);
    }
  } else {
    // three planes: one accumulator set, each chunk folded right after its second step
    for (; kt < nk; kt += 2) {
      step(T_{}, F_{}, A0, A0, F0, F1, kt);
      step(F_{}, F_{}, A0, A0, F1, F0, kt + 1);
      fold(A0);
    }
  }
  wait_vmcnt<0>();   // no LDS write may land after the workgroup ends

  // D element (4*(lane>>4) + r, lane&15) of each 16x16 block
#pragma unroll
  for (int m = 0; m < 2; m++)
#pragma unroll
    for (int r = 0; r < 4; r++) {
      const int t = t0 + wave * 32 + m * 16 + 4 * kg + r;
      if (t < T) {
#pragma unroll
        for (int j = 0; j < 4; j++) scores[(size_t)t * N + e0 + 16 * j + r16] = (float)sigmoid64(z64[m][j][r]);
      }
    }
}

bool route_two_phase_ok(const RouteArgs& a) {
  return a.in_dtype == MOE_BF16 && (a.router_dtype == MOE_BF16 || a.router_dtype == MOE_F32) &&
         a.n_routed % LG_BE == 0 && a.d % 128 == 0 && a.T > 0;
}

size_t route_two_phase_bytes(int T, int N, int d, int router_dtype) {
  const size_t sc = (((size_t)T * N * 4) + 255) / 256 * 256;
  const size_t pl = router_dtype == MOE_F32 ? (((size_t)3 * N * d * 2) + 255) / 256 * 256 : 0;
  return sc + pl;
}

hipError_t launch_route(const RouteArgs& a, int front, hipStream_t s);

// Phase 1 into `scratch` (scores, then the bf16 planes of fp32 centroids), phase 2 from there.
hipError_t launch_route_two_phase(const RouteArgs& a, void* scratch, hipStream_t s) {
  float* scores = (float*)scratch;
  const size_t sc = (((size_t)a.T * a.n_routed * 4) + 255) / 256 * 256;
  const dim3 grid(cdiv(a.T, LG_BT), a.n_routed / LG_BE);
  hipError_t e;
  if (a.router_dtype == MOE_F32) {
    uint16_t* planes = (uint16_t*)((uint8_t*)scratch + sc);
    const long n = (long)a.n_routed * a.d;
    split_planes_kernel<<<(int)std::min<long>(cdiv<long>(n, 256), 2048), 256, 0, s>>>((const float*)a.E, planes, n);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    auto k = logits_kernel<3>;
    if ((e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                 LogitsCfg<3>::BYTES)) != hipSuccess) return e;
    k<<<grid, 256, LogitsCfg<3>::BYTES, s>>>((const uint16_t*)a.u, planes, scores, a.T, a.d, a.n_routed);
  } else {
    auto k = logits_kernel<1>;
    if ((e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                 LogitsCfg<1>::BYTES)) != hipSuccess) return e;
    k<<<grid, 256, LogitsCfg<1>::BYTES, s>>>((const uint16_t*)a.u, (const uint16_t*)a.E, scores, a.T, a.d,
                                             a.n_routed);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  RouteArgs b = a;
  b.scores_in = scores;
  b.scores_out = nullptr;
  return launch_route(b, kFrontScoresIn, s);
}

// Per-expert loads from the selections. The router kernels add no counts
// themselves: thousands of workgroups adding into the same N counters
// serialise on those addresses. Here each of a few workgroups histograms a
// contiguous slice of idx in LDS and adds its nonzero bins, so each counter
// takes at most gridDim.x global atomics.
__global__ __launch_bounds__(256) void count_loads_kernel(const int32_t* __restrict__ idx, long n, int N,
                                                          int32_t* __restrict__ counts) {
  __shared__ int h[RT_NMAX];
  for (int e = threadIdx.x; e < N; e += 256) h[e] = 0;
  __syncthreads();
  const long per = (n + gridDim.x - 1) / gridDim.x;
  const long lo = (long)blockIdx.x * per, hi = lo + per < n ? lo + per : n;
  for (long i = lo + threadIdx.x; i < hi; i += 256) {
    const int e = idx[i];
    if ((unsigned)e < (unsigned)N) atomicAdd(&h[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < N; e += 256)
    if (h[e]) atomicAdd(&counts[e], h[e]);
}

hipError_t launch_count_loads(const int32_t* idx, long n, int N, int32_t* counts, hipStream_t s) {
  hipError_t e = launch_fill_i32(counts, 0, N, s);
  if (e != hipSuccess || n <= 0) return e;
  const int blocks = (int)std::min<long>(cdiv<long>(n, 2048), 32);
  count_loads_kernel<<<blocks, 256, 0, s>>>(idx, n, N, counts);
  return hipGetLastError();
}

__global__ void fill_i32_kernel(int32_t* p, int32_t v, long n) {
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x)
    p[i] = v;
}

hipError_t launch_fill_i32(int32_t* p, int32_t v, long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int blocks = (int)std::min<long>(cdiv<long>(n, 256), 1024);
  fill_i32_kernel<<<blocks, 256, 0, s>>>(p, v, n);
  return hipGetLastError();
}

hipError_t launch_route(const RouteArgs& a, int front, hipStream_t s) {
  const dim3 grid(cdiv(a.T, RT_BT));
  const bool ub = a.in_dtype == MOE_BF16;
  switch (front) {
    case kFrontScoresIn:
      // selection only: 4 tokens per workgroup (one per wave) for more waves in flight
      route_kernel<kFrontScoresIn, false, false, RT_BT_SEL><<<dim3(cdiv(a.T, RT_BT_SEL)), RT_THREADS, 0, s>>>(a);
      break;
    case kFrontMfma: route_kernel<kFrontMfma, true, true><<<grid, RT_THREADS, 0, s>>>(a); break;
    case kFrontMfmaSplitE: route_kernel<kFrontMfmaSplitE, true, false><<<grid, RT_THREADS, 0, s>>>(a); break;
    default: {
      // fp64 VALU logits, any dtype combination
      const bool eb = a.router_dtype == MOE_BF16;
      if (ub && eb) route_kernel<kFrontF64, true, true><<<grid, RT_THREADS, 0, s>>>(a);
      else if (ub) route_kernel<kFrontF64, true, false><<<grid, RT_THREADS, 0, s>>>(a);
      else if (eb) route_kernel<kFrontF64, false, true><<<grid, RT_THREADS, 0, s>>>(a);
      else route_kernel<kFrontF64, false, false><<<grid, RT_THREADS, 0, s>>>(a);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !a.counts) return e;
  return launch_count_loads(a.idx, (long)a.T * a.top_k, a.n_routed, a.counts, s);
}

}  // namespace moe
