// Router of the DeepSeekMoE layer on gfx950: affinities, biased group-limited
// top-K and normalised gates (route_kernel, fed by a logits kernel or with an
// fp64 front end of its own), and the per-expert loads (count_loads_kernel).
//
//   s_{i,t} = sigmoid(u_t . e_i)       -- DeepSeek-V3 Technical Report guides
//                                         (xyznot.com), "Metodo" section 2
//   top-K_r on s + b, gates from s      -- same section, gating equation; the
//                                         pwwt.cn note 1.1.2 (bias only routes)
//   groups ranked by the sum of their   -- pwwt.cn note 1.3 (node-limited
//   top K_r/M scores, at most M kept       routing; nodes = expert groups here)
//
// Paths, by shape (run_router picks one):
//  * split-K router (bf16 u and centroids, N_r = 256): logits_splitk_kernel
//    computes 128 tokens x 256 experts over one of S slices of d per
//    workgroup, writes each slice's sum as fp32, and route_kernel in partials mode adds
//    the S slices, applies the sigmoid and selects;
//  * tiled two-phase router (N_r % 64 == 0, bf16 u, bf16 or fp32 centroids):
//    logits_kernel writes fp32 affinities, route_kernel selects from them;
//  * any other shape: route_kernel with fp64 VALU logits.
// The selection back end is one code path whatever the front end was
// (affinities handed in by the caller included), so the scores-in mode
// exercises exactly the production selection.
//
// Precision: bf16 products (exact in fp32) are summed by the MFMAs in fp32
// over chunks of d of at most 128 elements, the chunks in fp64; the sigmoid is evaluated
// in fp64 and rounded once to fp32. The split-K router rounds each slice's
// fp64 sum to fp32 once before the S slices are added in fp64, in slice order.
// fp32 centroids are split into three bf16 terms (hi + mid + lo reproduces the
// fp32 value exactly), so the products stay exact on the bf16 MFMA path; the
// hi products and the much smaller mid+lo products go to separate accumulators
// so the small terms are not rounded against the large running sum.
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
using RouterLds = RouterLdsT<RT_BT>;      // the fp64 front end works on 32 tokens

// One formula for every z (no divergent branches across a wave): for z < 0,
// exp(-z) is large and 1 / (1 + exp(-z)) keeps full fp64 relative accuracy
// (it underflows to 0 only below z = -709, far under fp32's smallest affinity).
__device__ __forceinline__ double sigmoid64(double z) {
  return 1.0 / (1.0 + exp(-z));
}

// ---------------------------------------------------------------- front ends
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

// ---------------------------------------------------------------- lane-major selection (N_r = 256)
// The same selection for 256 experts with lane l holding experts 4l..4l+3, so a
// group of 32 contiguous experts is 8 adjacent lanes: its top-2 come from a
// sorting network on each lane's 4 values and three cross-lane merges (DPP), the
// group ranking from 8 lane reads, and each top-K round is a row-wise DPP max,
// 4 lane reads and one ballot (the lowest lane, then the lowest of its 4 slots,
// is the lowest expert index holding the maximum). About 400 instructions per
// token instead of thousands. Same total orders, same NaN and -0 handling, same
// fp64 gate sums in selection order as select_tokens.
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_ROW_HALF_MIRROR = 0x141, DPP_ROW_MIRROR = 0x140;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// maximum over the wave (the same value in every lane)
__device__ __forceinline__ uint32_t wave_max_lm(uint32_t v) {
  v = max(v, dpp_u32<DPP_XOR1>(v));
  v = max(v, dpp_u32<DPP_XOR2>(v));
  v = max(v, dpp_u32<DPP_ROW_HALF_MIRROR>(v));
  v = max(v, dpp_u32<DPP_ROW_MIRROR>(v));                 // each 16-lane row holds its maximum
  const uint32_t r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return max(max(r0, r1), max(r2, r3));
}
// the two largest of a multiset, merged with another lane's pair
__device__ __forceinline__ void top2_merge(float& t1, float& t2, float p1, float p2) {
  const float n1 = fmaxf(t1, p1);
  t2 = fmaxf(fminf(t1, p1), fmaxf(t2, p2));
  t1 = n1;
}

bool route_lm_ok(const RouteArgs& a) {
  const int S = a.n_groups > 0 ? a.n_routed / a.n_groups : 0;
  return a.n_routed == RT_NMAX && (a.n_groups == 1 || (S == 32 && a.group_topk <= 2));
}

// one wave per token; s4: this lane's 4 affinities (experts 4 lane ..), b4: their biases
__device__ __forceinline__ void select_lane_major(const RouteArgs& a, const float s4[4], const float b4[4], int t) {
  const int lane = threadIdx.x & 63;
  const int K = a.top_k, G = a.n_groups, M = a.topk_groups, q = a.group_topk;
  uint32_t k4[4];
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const float kv = s4[i] + b4[i];
    k4[i] = kv != kv ? 1u : max(ordered_f32(kv), 1u);     // NaN ranks after every number
  }
  if (G > 1) {
    // each group's q largest (q <= 2) values of s + b (or s), NaN as -inf; fp32 sum, largest first
    float g[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const float v = a.group_score_biased ? s4[i] + b4[i] : s4[i];
      g[i] = v != v ? -INFINITY : v;
    }
    const float h1 = fmaxf(g[0], g[1]), l1 = fminf(g[0], g[1]);
    const float h2 = fmaxf(g[2], g[3]), l2 = fminf(g[2], g[3]);
    float t1 = fmaxf(h1, h2), t2 = fmaxf(fminf(h1, h2), fmaxf(l1, l2));
    top2_merge(t1, t2, dpp_f32<DPP_XOR1>(t1), dpp_f32<DPP_XOR1>(t2));
    top2_merge(t1, t2, dpp_f32<DPP_XOR2>(t1), dpp_f32<DPP_XOR2>(t2));
    top2_merge(t1, t2, dpp_f32<DPP_ROW_HALF_MIRROR>(t1), dpp_f32<DPP_ROW_HALF_MIRROR>(t2));
    const float gs = q >= 2 ? t1 + t2 : t1;
    const uint32_t mine = max(ordered_f32(gs), 1u);
    // rank of this lane's group g = lane / 8 among the 8: (score desc, group index asc)
    const int gi = lane >> 3;
    int rank = 0;
#pragma unroll
    for (int h = 0; h < 8; h++) {
      const uint32_t o = __builtin_amdgcn_readlane(mine, 8 * h);
      rank += (o > mine || (o == mine && h < gi)) ? 1 : 0;
    }
    if (rank >= M) k4[0] = k4[1] = k4[2] = k4[3] = 0u;
  }
  // K rounds: the largest key, then the lowest expert index holding it
  int my_e = 0;
  float my_s = 0.f;
  for (int k = 0; k < K; k++) {
    const uint32_t lmax = max(max(k4[0], k4[1]), max(k4[2], k4[3]));
    const uint32_t kmax = wave_max_lm(lmax);
    const uint64_t hold = __ballot(lmax == kmax);
    const int L = (int)__builtin_ctzll(hold);
    int fs = 3;                                             // this lane's lowest slot holding kmax
    fs = k4[2] == kmax ? 2 : fs;
    fs = k4[1] == kmax ? 1 : fs;
    fs = k4[0] == kmax ? 0 : fs;
    const int slot = __builtin_amdgcn_readlane(fs, L);
    // lane L's four affinities as wave-uniform values, then a scalar pick (indexing s4
    // by slot would send the array through LDS)
    const int c0 = __builtin_amdgcn_readlane(__float_as_int(s4[0]), L);
    const int c1 = __builtin_amdgcn_readlane(__float_as_int(s4[1]), L);
    const int c2 = __builtin_amdgcn_readlane(__float_as_int(s4[2]), L);
    const int c3 = __builtin_amdgcn_readlane(__float_as_int(s4[3]), L);
    const float sel = __int_as_float(slot == 0 ? c0 : slot == 1 ? c1 : slot == 2 ? c2 : c3);
    const bool owner = lane == L;
#pragma unroll
    for (int i = 0; i < 4; i++) k4[i] = owner && slot == i ? 0u : k4[i];
    my_e = lane == k ? 4 * L + slot : my_e;
    my_s = lane == k ? sel : my_s;
  }
  // gate denominator: the selected scores in selection order, summed in fp64
  double sum = 0.0;
  for (int k = 0; k < K; k++) sum += (double)__int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_s), k));
  if (lane < K) {
    const float gte = sum > 0.0 ? (float)((double)my_s / sum) : 1.0f / (float)K;
    const size_t o = (size_t)t * K + lane;
    a.idx[o] = my_e;
    a.gate[o] = gte;
  }
}

// selection of 4 tokens per workgroup (one per wave) from given affinities or from
// the split-K partial logits
template <int FRONT>
__global__ __launch_bounds__(RT_THREADS) void route_lm_kernel(RouteArgs a) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (RT_THREADS / kWave) + (threadIdx.x >> 6);
  if (t >= a.T) return;
  float s4[4], b4[4];
  const f32x4 bv = *(const f32x4*)(a.b + 4 * lane);
#pragma unroll
  for (int i = 0; i < 4; i++) b4[i] = bv[i];
  if constexpr (FRONT == kFrontScoresIn) {
    const f32x4 v = *(const f32x4*)(a.scores_in + (size_t)t * RT_NMAX + 4 * lane);
#pragma unroll
    for (int i = 0; i < 4; i++) s4[i] = v[i];
  } else {
    // the S fp32 slice sums, added in fp64 in slice order; 4 slices' loads in flight at a time
    const size_t slice = (size_t)a.T * RT_NMAX;
    const float* src = a.partials + (size_t)t * RT_NMAX + 4 * lane;
    double z[4] = {0.0, 0.0, 0.0, 0.0};
    int sl = 0;
    for (; sl + 4 <= a.n_slices; sl += 4) {
      f32x4 v[4];
#pragma unroll
      for (int j = 0; j < 4; j++) v[j] = *(const f32x4*)(src + (sl + j) * slice);
#pragma unroll
      for (int j = 0; j < 4; j++)
#pragma unroll
        for (int i = 0; i < 4; i++) z[i] += (double)v[j][i];
    }
    for (; sl < a.n_slices; sl++) {
      const f32x4 v = *(const f32x4*)(src + sl * slice);
#pragma unroll
      for (int i = 0; i < 4; i++) z[i] += (double)v[i];
    }
#pragma unroll
    for (int i = 0; i < 4; i++) s4[i] = (float)sigmoid64(z[i]);
  }
  if (a.scores_out)
    *(f32x4*)(a.scores_out + (size_t)t * RT_NMAX + 4 * lane) = f32x4{s4[0], s4[1], s4[2], s4[3]};
  select_lane_major(a, s4, b4, t);
}

template <int FRONT, bool U_BF16, bool E_BF16, int BT = RT_BT>
__global__ __launch_bounds__(RT_THREADS) void route_kernel(RouteArgs a) {
  static_assert(FRONT == kFrontF64 ? BT == RT_BT : BT == RT_THREADS / kWave,
                "the fp64 front end works on 32 tokens, the others on one token per wave");
  __shared__ RouterLdsT<BT> sh;
  const int t0 = blockIdx.x * BT;
  const int nt = min(BT, a.T - t0);
  for (int e = threadIdx.x; e < a.n_routed; e += RT_THREADS) {
    sh.b[e] = a.b[e];
  }
  if constexpr (FRONT == kFrontScoresIn) {
    // wave w fills token w's row (one token per wave); every load is issued before any store
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (w < nt) {
      const float* src = a.scores_in + (size_t)(t0 + w) * a.n_routed;
      float v[RT_NMAX / 64];
#pragma unroll
      for (int j = 0; j < RT_NMAX / 64; j++) {
        const int e = lane + 64 * j;
        v[j] = e < a.n_routed ? src[e] : 0.f;
      }
#pragma unroll
      for (int j = 0; j < RT_NMAX / 64; j++)
        if (lane + 64 * j < a.n_routed) sh.s[w][lane + 64 * j] = v[j];
    }
  } else if constexpr (FRONT == kFrontPartials) {
    // the split-K logits: S fp32 slice sums per (token, expert), added in fp64 in slice order
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (w < nt) {
      const size_t slice = (size_t)a.T * a.n_routed;
      const float* src = a.partials + (size_t)(t0 + w) * a.n_routed;
      double z[RT_NMAX / 64];
#pragma unroll
      for (int j = 0; j < RT_NMAX / 64; j++) z[j] = 0.0;
      int sl = 0;
      for (; sl + 4 <= a.n_slices; sl += 4) {          // 4 slices' loads in flight at a time
        float v[4][RT_NMAX / 64];
#pragma unroll
        for (int q = 0; q < 4; q++)
#pragma unroll
          for (int j = 0; j < RT_NMAX / 64; j++) {
            const int e = lane + 64 * j;
            v[q][j] = e < a.n_routed ? src[(sl + q) * slice + e] : 0.f;
          }
#pragma unroll
        for (int q = 0; q < 4; q++)
#pragma unroll
          for (int j = 0; j < RT_NMAX / 64; j++) z[j] += (double)v[q][j];
      }
      for (; sl < a.n_slices; sl++)
#pragma unroll
        for (int j = 0; j < RT_NMAX / 64; j++) {
          const int e = lane + 64 * j;
          z[j] += (double)(e < a.n_routed ? src[sl * slice + e] : 0.f);
        }
#pragma unroll
      for (int j = 0; j < RT_NMAX / 64; j++)
        if (lane + 64 * j < a.n_routed) sh.s[w][lane + 64 * j] = (float)sigmoid64(z[j]);
    }
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
// of a 128-token x 64-expert tile and writes them to a scores buffer: 16x16x32
// MFMAs, fp32 partials over 128-element chunks of d summed in fp64 in chunk
// order, fp32 centroids split into hi/mid/lo bf16 planes. Phase 2 is
// route_kernel in scores-in mode (the same selection code).
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

// ---------------------------------------------------------------- split-K router
// For N_r = 256 experts with bf16 u and centroids. A workgroup (8 waves) owns
// 128 tokens x all 256 experts over one slice of d (S slices of d/S elements,
// each a whole number of 128-element chunks), so each u element is read once
// and each centroid slice once per 128 tokens. u and the centroids are read
// in place: a load instruction takes 128 bytes (one cache line) of each of 8
// rows, and each lane picks the 16-byte chunk that its LDS slot holds under
// the XOR swizzle of the MFMA operand reads. Wave (wm, wn) computes tokens
// 64 wm.. x experts 64 wn.. with v_mfma_f32_32x32x16_bf16 (2 x 2 blocks); its
// fp32 sums over chunks of at most 128 elements are added into fp64 in chunk
// order, and the slice's fp64 sum is written once as fp32 to
// partials[slice][t][e].
// route_kernel in partials mode adds the S slices in fp64, in slice order.
constexpr int SK_BT = 128;                 // tokens per workgroup
constexpr int SK_NE = 256;                 // experts per workgroup (all of them)
constexpr int SK_BK = 64;                  // elements per stage row (128 bytes)
constexpr int SK_U_BYTES = SK_BT * SK_BK * 2;                 // 16 KB
constexpr int SK_STAGE = (SK_BT + SK_NE) * SK_BK * 2;         // 48 KB
constexpr int SK_STAGES = 3;
constexpr int SK_U_PER_WAVE = SK_BT / 8 / 8;                  // 1 KB blocks of 8 rows over 8 waves
constexpr int SK_E_PER_WAVE = SK_NE / 8 / 8;
constexpr int SK_LOADS = SK_U_PER_WAVE + SK_E_PER_WAVE;
static_assert(SK_STAGES * SK_STAGE <= 160 * 1024, "LDS budget");

__global__ __launch_bounds__(512, 1) void logits_splitk_kernel(const uint16_t* __restrict__ u,
                                                               const uint16_t* __restrict__ E,
                                                               float* __restrict__ partials, int T, int d,
                                                               int n_slices) {
  extern __shared__ __align__(16) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int t0 = blockIdx.x * SK_BT, sl = blockIdx.y;
  const int L = d / n_slices;                  // elements per slice, a multiple of 128
  const int k_begin = sl * L;
  const int nk = L / SK_BK;                    // stages, even

  // ---- loads: block i of a stage is 8 rows x 128 bytes; lane l writes row l >> 3, slot l & 7
  const int brow = lane >> 3;
  const int bchunk = (lane & 7) ^ brow;        // block rows start at multiples of 8
  const i32x4 ur = rsrc_words(u, (long)T * d * 2);
  const i32x4 er = rsrc_words(E, (long)SK_NE * d * 2);
  int eoff[SK_E_PER_WAVE];
#pragma unroll
  for (int i = 0; i < SK_E_PER_WAVE; i++) eoff[i] = (((wave + 8 * i) * 8 + brow) * d + k_begin + bchunk * 8) * 2;
  int uoff[SK_U_PER_WAVE];
#pragma unroll
  for (int i = 0; i < SK_U_PER_WAVE; i++) {
    const int t = t0 + (wave + 8 * i) * 8 + brow;
    uoff[i] = t < T ? (t * d + k_begin + bchunk * 8) * 2 : kOutOfRange;
  }
  const uint32_t lds0 = lds_addr(lds);
  auto issue_part = [&](auto p_tag, int kt, int buf) __attribute__((always_inline)) {
    constexpr int P = decltype(p_tag)::value;
    const uint32_t sb = lds0 + buf * SK_STAGE;
    if constexpr (P < SK_U_PER_WAVE) {
      dma_b128(ur, uoff[P], kt * SK_BK * 2, sb + (wave + 8 * P) * 1024);
    } else {
      constexpr int Q = P - SK_U_PER_WAVE;
      dma_b128(er, eoff[Q], kt * SK_BK * 2, sb + SK_U_BYTES + (wave + 8 * Q) * 1024);
    }
  };
  auto issue = [&](int kt, int buf) __attribute__((always_inline)) {
    static_for<SK_LOADS>([&](auto p) __attribute__((always_inline)) { issue_part(p, kt, buf); });
  };

  // ---- operand reads: lane l takes row l & 31, 16-byte chunk 2 ks + (l >> 5) of k-substep ks
  const int l32 = lane & 31, khalf = lane >> 5;
  int roff[4];
#pragma unroll
  for (int ks = 0; ks < 4; ks++) roff[ks] = l32 * 128 + (((2 * ks + khalf) ^ (l32 & 7)) << 4);
  const int arow = wm * 64 * 128, brow0 = wn * 64 * 128;

  f32x16 acc[2][2];
  double z64[2][2][16];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) { acc[i][j][r] = 0.f; z64[i][j][r] = 0.0; }

  // The fp32 sums of token block i go into fp64 when one of its chunks ends:
  // block 0's chunks are the 128-element chunks [128 c, 128 c + 128), block 1's
  // are shifted by 64 (64 elements first and last), so every stage ends exactly
  // one block's chunk and its fold (cvt + fp64 add of 32 sums) is interleaved
  // with the MFMAs of the other block instead of stalling the matrix core.
  auto fold_piece = [&](auto x_tag, auto p_tag) __attribute__((always_inline)) {
    constexpr int X = decltype(x_tag)::value, P = decltype(p_tag)::value;
    constexpr int j = P >> 1, r0 = (P & 1) * 8;
#pragma unroll
    for (int r = r0; r < r0 + 8; r++) {
      z64[X][j][r] += (double)acc[X][j][r];
      acc[X][j][r] = 0.f;
    }
  };
  // two k-substeps of stage `buf`: their operand reads, then their MFMAs (token
  // block X first) with loads P0..P1-1 (of step kti into buffer bufi) spread
  // between them; FOLD: block X's chunk ends with these substeps, and its fold
  // pieces go between block 1-X's MFMAs
  auto half = [&](auto h_tag, auto p0_tag, auto p1_tag, auto x_tag, auto fold_tag, int buf, int kti, int bufi)
      __attribute__((always_inline)) {
    constexpr int H = decltype(h_tag)::value;
    constexpr int P0 = decltype(p0_tag)::value, P1 = decltype(p1_tag)::value;
    constexpr int X = decltype(x_tag)::value;
    constexpr bool FOLD = decltype(fold_tag)::value;
    const uint8_t* U = lds + buf * SK_STAGE;
    const uint8_t* Ep = U + SK_U_BYTES;
    bf16x8 af[2][2], bf[2][2];
#pragma unroll
    for (int q = 0; q < 2; q++)
#pragma unroll
      for (int i = 0; i < 2; i++) {
        af[q][i] = *(const bf16x8*)(U + arow + i * 32 * 128 + roff[H + q]);
        bf[q][i] = *(const bf16x8*)(Ep + brow0 + i * 32 * 128 + roff[H + q]);
      }
    static_for<8>([&](auto m_tag) __attribute__((always_inline)) {
      constexpr int m = decltype(m_tag)::value;
      constexpr int i = m < 4 ? X : 1 - X, q = (m >> 1) & 1, j = m & 1;
      if constexpr (m % 2 == 0 && P0 + m / 2 < P1) {
        __builtin_amdgcn_sched_barrier(0);
        issue_part(std::integral_constant<int, P0 + m / 2>{}, kti, bufi);
        __builtin_amdgcn_sched_barrier(0);
      }
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[q][i], bf[q][j], acc[i][j], 0, 0, 0);
      if constexpr (FOLD && m >= 4) {
        __builtin_amdgcn_sched_barrier(0);
        fold_piece(x_tag, std::integral_constant<int, m - 4>{});
        __builtin_amdgcn_sched_barrier(0);
      }
    });
  };
  // one stage; X: the token block whose chunk ends with it
  auto stage = [&](auto x_tag, int buf, int kti, int bufi) __attribute__((always_inline)) {
    half(std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{},
         std::integral_constant<int, SK_LOADS / 2>{}, x_tag, std::false_type{}, buf, kti, bufi);
    half(std::integral_constant<int, 2>{}, std::integral_constant<int, SK_LOADS / 2>{},
         std::integral_constant<int, SK_LOADS>{}, x_tag, std::true_type{}, buf, kti, bufi);
  };

  // ring of SK_STAGES buffers, as in the grouped GEMM: wait for this wave's loads of
  // step kt, barrier, multiply stage kt while refilling the buffer of step kt-1 with
  // step kt+STAGES-1 (past the last step: re-reads of it, never used). Even stages end
  // a chunk of token block 1, odd stages one of block 0 (nk is even).
  constexpr int S = SK_STAGES;
#pragma unroll
  for (int p = 0; p < S - 1; p++) issue(min(p, nk - 1), p);
  for (int kt = 0; kt < nk; kt += 2) {
#pragma unroll
    for (int e = 0; e < 2; e++) {
      const int k = kt + e;
      wait_vmcnt<(S - 2) * SK_LOADS>();
      __syncthreads();
      const int kti = min(k + S - 1, nk - 1), bufi = (k + S - 1) % S;
      if (e == 0) stage(std::integral_constant<int, 1>{}, k % S, kti, bufi);
      else stage(std::integral_constant<int, 0>{}, k % S, kti, bufi);
    }
  }
  // block 1's last chunk: the final stage
  static_for<4>([&](auto p) __attribute__((always_inline)) { fold_piece(std::integral_constant<int, 1>{}, p); });
  wait_vmcnt<0>();   // no LDS write may land after the workgroup ends

  // D element (8*(r>>2) + 4*(lane>>5) + (r&3), lane&31) of each 32x32 block
  float* out = partials + (size_t)sl * T * SK_NE;
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int t = t0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
      if (t < T) {
#pragma unroll
        for (int j = 0; j < 2; j++) out[(size_t)t * SK_NE + wn * 64 + j * 32 + l32] = (float)z64[i][j][r];
      }
    }
}

// slices of d (each a whole number of 128-element chunks) so that the grid has
// enough workgroups to fill the chip
static int splitk_slices(int T, int d) {
  const int tiles = (T + SK_BT - 1) / SK_BT, chunks = d / 128;
  int best = chunks;
  for (int sdiv = 1; sdiv <= chunks; sdiv++)
    if (chunks % sdiv == 0 && (long)tiles * sdiv >= 224) { best = sdiv; break; }
  return best;
}

bool route_splitk_ok(const RouteArgs& a) {
  return a.in_dtype == MOE_BF16 && a.router_dtype == MOE_BF16 && a.n_routed == SK_NE && a.d % 128 == 0 &&
         a.T > 0;
}

size_t route_splitk_bytes(int T, int d) {
  return (size_t)splitk_slices(T, d) * T * SK_NE * 4;
}

hipError_t launch_route_splitk(const RouteArgs& a, void* scratch, hipStream_t s) {
  float* partials = (float*)scratch;
  const int S = splitk_slices(a.T, a.d);
  hipError_t e;
  auto k = logits_splitk_kernel;
  if ((e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize,
                               SK_STAGES * SK_STAGE)) != hipSuccess) return e;
  k<<<dim3(cdiv(a.T, SK_BT), S), 512, SK_STAGES * SK_STAGE, s>>>((const uint16_t*)a.u, (const uint16_t*)a.E, partials, a.T, a.d, S);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  RouteArgs b = a;
  b.partials = partials;
  b.n_slices = S;
  return launch_route(b, kFrontPartials, s);
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
      if (route_lm_ok(a))
        route_lm_kernel<kFrontScoresIn><<<dim3(cdiv(a.T, RT_BT_SEL)), RT_THREADS, 0, s>>>(a);
      else
        route_kernel<kFrontScoresIn, false, false, RT_BT_SEL><<<dim3(cdiv(a.T, RT_BT_SEL)), RT_THREADS, 0, s>>>(a);
      break;
    case kFrontPartials:
      if (route_lm_ok(a))
        route_lm_kernel<kFrontPartials><<<dim3(cdiv(a.T, RT_BT_SEL)), RT_THREADS, 0, s>>>(a);
      else
        route_kernel<kFrontPartials, false, false, RT_BT_SEL><<<dim3(cdiv(a.T, RT_BT_SEL)), RT_THREADS, 0, s>>>(a);
      break;
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

// ---------------------------------------------------------------- one router for every entry point
size_t router_scratch_bytes(const RouteArgs& a) {
  if (route_splitk_ok(a)) return route_splitk_bytes(a.T, a.d);
  if (route_two_phase_ok(a)) return route_two_phase_bytes(a.T, a.n_routed, a.d, a.router_dtype);
  return 0;
}

hipError_t run_router(const RouteArgs& a, void* scratch, hipStream_t s) {
  if (a.scores_in) return launch_route(a, kFrontScoresIn, s);
  if (route_splitk_ok(a)) return launch_route_splitk(a, scratch, s);
  if (route_two_phase_ok(a)) return launch_route_two_phase(a, scratch, s);
  return launch_route(a, kFrontF64, s);
}

}  // namespace moe
