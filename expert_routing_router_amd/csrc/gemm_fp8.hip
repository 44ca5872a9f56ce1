// Grouped expert GEMMs with E4M3 operands and fine-grained fp32 scales.
//
// The pages' FP8 recipe (DeepSeek-V3 guides on xyznot.com, FP8 key idea;
// pwwt.cn note section 3): E4M3 inputs, one scale per 1x128 activation tile
// and per 128x128 weight block, partial sums promoted to fp32 every 128
// K-elements. On gfx950 the MFMA already accumulates in fp32, so the promotion
// becomes a scale applied once per 128-wide K block of
// acc = sum_kb partial_kb * (s_act[row, kb] * s_w[nblock, kb]): the register-staged
// kernel below folds each block's fresh fp32 partial (two v_mfma 32x32x64
// f8f6f4) into the accumulator; the LDS-DMA kernel keeps the accumulator in
// units of the current block's scale and rescales it at each block.
// The per-row activation scales of the tile are staged in LDS beside A.
// Tiling, ragged segments and the SwiGLU epilogue follow the bf16 kernel.
#include "common.h"
#include "fp8_codec.h"
#include "lds_dma.h"
#include "tile_order.h"
#include "moe_internal.h"
#include <type_traits>

namespace moe {

constexpr int GF_BK = 128;        // fp8 elements (bytes) per K step = one scale block
constexpr int GF_BN = 128;
constexpr int GF_THREADS = 256;

template <int MB>
struct Fp8Lds {
  static constexpr int BM = 64 * MB;
  static constexpr int A_BYTES = BM * GF_BK;
  static constexpr int B_BYTES = GF_BN * GF_BK;
  static constexpr int SA_BYTES = BM * 4;
  static constexpr int STAGE = A_BYTES + B_BYTES + SA_BYTES;
  static constexpr int BYTES = 2 * STAGE;
};

__device__ __forceinline__ int swz8(int row, int chunk) { return row * 128 + ((chunk ^ (row & 7)) << 4); }

template <int MB, bool SWIGLU>
__global__ __launch_bounds__(GF_THREADS, 1) void gemm_fp8_kernel(GemmArgs a) {
  using L = Fp8Lds<MB>;
  constexpr int BM = L::BM;
  constexpr int ACH = BM * 8 / GF_THREADS;
  constexpr int BCH = GF_BN * 8 / GF_THREADS;
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ int32_t sprefix[512];
  __shared__ int32_t srow[BM];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  for (int i = tid; i <= a.n_seg; i += GF_THREADS) sprefix[i] = a.mtile_prefix[i];
  __syncthreads();
  const int n_tiles = SWIGLU ? a.N / 64 : a.N / GF_BN;
  int seg, ntile, mtile;
  // Workgroup i runs on XCD i % 8, and each XCD starts its workgroups in order of i.
  // Give XCD x the contiguous logical range [x*per, (x+1)*per): the tiles of one
  // expert (all its n-tiles) then run side by side on one XCD and share the
  // expert's gathered rows in that XCD's L2.
  const int total_tiles = sprefix[a.n_seg] * n_tiles;
  const int per_xcd = (total_tiles + 7) >> 3;
  const int lt = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if ((int)(blockIdx.x >> 3) >= per_xcd) return;
  if (!decode_tile(sprefix, a.n_seg, n_tiles, lt, seg, ntile, mtile)) return;

  const int row0 = a.offsets[seg] + mtile * BM;
  const int mvalid = min(BM, a.offsets[seg + 1] - row0);
  const int K = a.K, KB = K / 128;
  const bool first = seg < a.n_first;
  const uint8_t* wbase = first ? (const uint8_t*)a.w0 + (size_t)seg * a.wstride0
                               : (const uint8_t*)a.w1 + (size_t)(seg - a.n_first) * a.wstride1;
  const float* wsc = first ? a.ws0 + (size_t)seg * a.sstride0 : a.ws1 + (size_t)(seg - a.n_first) * a.sstride1;

  for (int r = tid; r < BM; r += GF_THREADS)
    srow[r] = r < mvalid && (unsigned)(row0 + r) < (unsigned)a.rows_bound
                  ? (a.row_index ? a.row_index[row0 + r] : row0 + r) : -1;
  __syncthreads();

  const int cch = tid & 7, rbase = tid >> 3;
  // rows past the segment (and scale slots past BM) load zeros through out-of-range offsets
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, a.x_rows * (long)K);
  const __amdgpu_buffer_rsrc_t sr = make_rsrc(a.x_scale, a.x_rows * (long)KB * 4);
  int aoff[ACH];
#pragma unroll
  for (int i = 0; i < ACH; i++) {
    const int src = srow[rbase + 32 * i];
    aoff[i] = src >= 0 ? src * K + cch * 16 : kOutOfRange;
  }
  int soff[2];
#pragma unroll
  for (int i = 0; i < 2; i++) {
    const int r = tid + i * GF_THREADS;
    const int src = r < BM ? srow[r] : -1;
    soff[i] = src >= 0 ? src * KB * 4 : kOutOfRange;
  }
  int boff[BCH];
#pragma unroll
  for (int i = 0; i < BCH; i++) {
    const int br = rbase + 32 * i;
    const int wrow = SWIGLU ? (br < 64 ? ntile * 64 + br : a.N + ntile * 64 + (br - 64)) : ntile * GF_BN + br;
    boff[i] = wrow * K + cch * 16;
  }
  // weight block-row of each of this wave's two 32-row n-blocks
  int wblk[2];
#pragma unroll
  for (int j = 0; j < 2; j++) {
    const int wrow = SWIGLU ? (j == 0 ? ntile * 64 + wn * 32 : a.N + ntile * 64 + wn * 32)
                            : ntile * GF_BN + wn * 64 + j * 32;
    wblk[j] = wrow / 128;
  }

  // One register set for the next K block (the accumulators live in VGPRs
  // here because the scale fold is VALU work, which leaves no room for two).
  i32x4 ra[ACH], rb[BCH];
  float rs[2];
  auto gload = [&](int kb) __attribute__((always_inline)) {
    const int k0 = kb * GF_BK;
#pragma unroll
    for (int i = 0; i < ACH; i++) ra[i] = __builtin_amdgcn_raw_buffer_load_b128(xr, aoff[i] + k0, 0, 0);
#pragma unroll
    for (int i = 0; i < BCH; i++) rb[i] = __builtin_nontemporal_load((const i32x4*)(wbase + boff[i] + k0));
#pragma unroll
    for (int i = 0; i < 2; i++)
      rs[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(sr, soff[i] + kb * 4, 0, 0));
  };
  auto sstore = [&](int buf) __attribute__((always_inline)) {
    uint8_t* A = lds + buf * L::STAGE;
    uint8_t* B = A + L::A_BYTES;
    float* SA = (float*)(B + L::B_BYTES);
#pragma unroll
    for (int i = 0; i < ACH; i++) *(i32x4*)(A + swz8(rbase + 32 * i, cch)) = ra[i];
#pragma unroll
    for (int i = 0; i < BCH; i++) *(i32x4*)(B + swz8(rbase + 32 * i, cch)) = rb[i];
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const int r = tid + i * GF_THREADS;
      if (r < BM) SA[r] = rs[i];
    }
  };

  f32x16 acc[MB][2];
#pragma unroll
  for (int i = 0; i < MB; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;
  int mb_active = 0;
#pragma unroll
  for (int i = 0; i < MB; i++)
    if ((2 * i + wm) * 32 < mvalid) mb_active = i + 1;

  const int l32 = lane & 31, khalf = lane >> 5;
  // One 128-wide K block from LDS buffer `buf` with NA active m-blocks: for
  // each 32x32 block, two MFMAs into a fresh fp32 partial, then the scale fold.
  auto compute_na = [&](auto na_tag, int buf, int kb) __attribute__((always_inline)) {
    constexpr int NA = decltype(na_tag)::value;
    const uint8_t* A = lds + buf * L::STAGE;
    const uint8_t* B = A + L::A_BYTES;
    const float* SA = (const float*)(B + L::B_BYTES);
#pragma unroll
    for (int j = 0; j < 2; j++) {
      const float sw = wsc[(size_t)wblk[j] * KB + kb];
      const int brow = (SWIGLU ? j * 64 + wn * 32 : wn * 64 + j * 32) + l32;
      i32x8 bfr[2];
#pragma unroll
      for (int h = 0; h < 2; h++) {
        const int c0 = h * 4 + khalf * 2;
        const i32x4 lo = *(const i32x4*)(B + swz8(brow, c0));
        const i32x4 hi = *(const i32x4*)(B + swz8(brow, c0 + 1));
        bfr[h] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
      for (int i = 0; i < NA; i++) {
        const int arow = (2 * i + wm) * 32 + l32;
        f32x16 p;
#pragma unroll
        for (int r = 0; r < 16; r++) p[r] = 0.f;
#pragma unroll
        for (int h = 0; h < 2; h++) {
          const int c0 = h * 4 + khalf * 2;
          const i32x4 lo = *(const i32x4*)(A + swz8(arow, c0));
          const i32x4 hi = *(const i32x4*)(A + swz8(arow, c0 + 1));
          const i32x8 afr = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          // cbsz = blgp = 0: both operands E4M3; scale exponents 127 = 2^0
          p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(afr, bfr[h], p, 0, 0, 0, 127, 0, 127);
        }
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int row = (2 * i + wm) * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
          acc[i][j][r] += p[r] * (SA[row] * sw);
        }
        // one partial live at a time
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  auto k_loop = [&](auto na_tag) __attribute__((always_inline)) {
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kb = 0; kb < KB; kb++) {
      gload(min(kb + 1, KB - 1));        // unconditional: in-order wait counting
      compute_na(na_tag, kb & 1, kb);
      sstore((kb + 1) & 1);
      __syncthreads();
    }
  };
  // A wave with no active m-block still runs the loop: it loads its share of
  // every LDS tile and takes part in every barrier.
  switch (__builtin_amdgcn_readfirstlane(mb_active)) {
    case 0: k_loop(std::integral_constant<int, 0>{}); break;
    case 1: k_loop(std::integral_constant<int, 1>{}); break;
    case 2: k_loop(std::integral_constant<int, 2>{}); break;
    default: k_loop(std::integral_constant<int, MB>{}); break;
  }

  // GEMM1 writes H in fp32 (it is re-quantised to E4M3 per 1x128 tile next);
  // GEMM2 writes Y in bf16.
#pragma unroll
  for (int i = 0; i < MB; i++) {
    if (i < mb_active) {
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int row = (2 * i + wm) * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
        if (row < mvalid && (unsigned)(row0 + row) < (unsigned)a.rows_bound) {
          if (SWIGLU) {
            float* orow = (float*)a.out + (size_t)(row0 + row) * a.N;
            orow[ntile * 64 + wn * 32 + l32] = silu_mul(acc[i][0][r], acc[i][1][r]);
          } else {
            uint16_t* orow = (uint16_t*)a.out + (size_t)(row0 + row) * a.N;
            const int col = ntile * GF_BN + wn * 64 + l32;
            orow[col] = f32_to_bf16(acc[i][0][r]);
            orow[col + 32] = f32_to_bf16(acc[i][1][r]);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------- LDS-DMA path
// 8 waves (2 along M x 4 along N), tile 64*MB rows x 256 weight rows. A stage
// holds 64 elements of K (half a scale block) of both operands and, at the
// first stage of each 128-element block, the tile rows' activation scales of
// that block; four stages in a ring, three in flight while one is multiplied. Buffer loads write the E4M3
// rows and the row scales straight into LDS. The two weight-block scales a
// workgroup needs per K block (gate and up rows for SwiGLU, the two 128-row
// halves of the tile for the down GEMM) are staged in LDS once, for all K.
//
// The MFMA takes the weight rows as its first operand and the activation rows
// as its second, so each lane's 16 results belong to one activation row (its
// column) and 16 rows of one 32-row weight block, which share one scale
// s = s_act * s_w per 128-element block. The accumulator is kept in units of
// the current block's s: at each block's first stage it is multiplied by
// s_prev / s, and the MFMAs of both 64-element stages accumulate into it
// directly. The sum is the pages' promotion every 128 elements,
// sum_kb s_kb * p_kb, up to fp32 rounding of the ratios.
//
// A stage row is 64 bytes = 4 chunks of 16; one load instruction of a wave
// fills 16 rows (1 KB): lane l writes row l>>2, slot l&3 and fetches chunk
// slot ^ ((row >> 2) & 3), so the MFMA operand reads (16 lanes = 16
// consecutive rows, one chunk) hit 16 distinct 4-bank groups.
constexpr int F8_BK = 128;              // scale block along K
constexpr int F8_SK = 64;               // K elements per stage
constexpr int F8_STAGES = 4;
constexpr int F8_MAX_KB = 256;          // K <= 32768

template <int MB>
struct F8DmaCfg {
  static constexpr int THREADS = 512;
  static constexpr int BM = 64 * MB;
  static constexpr int BN = 256;
  static constexpr int A_LOADS = BM / 16;            // 1 KB loads per stage
  static constexpr int B_LOADS = BN / 16;
  static constexpr int A_BYTES = BM * F8_SK;
  static constexpr int B_BYTES = BN * F8_SK;
  static constexpr int SA_BYTES = BM * 4;
  static constexpr int STAGE = A_BYTES + B_BYTES + SA_BYTES;
  static constexpr int BYTES = F8_STAGES * STAGE;
  static constexpr int A_MAX = (A_LOADS + 7) / 8;    // A loads of waves 0 .. (A_LOADS % 8) - 1 (or all)
  static constexpr int A_MIN = A_LOADS / 8;
  static constexpr int B_PER_WAVE = B_LOADS / 8;
  static constexpr int SA_WAVES = BM / 64;           // waves that load 64 row scales each
  static_assert(B_LOADS % 8 == 0 && SA_WAVES <= 8, "loads split over 8 waves");
  static_assert(STAGE % 16 == 0, "stage alignment");
  static_assert(BYTES + 2 * F8_MAX_KB * 4 + 2048 + 4 * BM * 4 <= 160 * 1024, "LDS budget");
};

template <int MB, bool SWIGLU>
__global__ __launch_bounds__(512, 1) void gemm_fp8_dma_kernel(GemmArgs a) {
  using C = F8DmaCfg<MB>;
  constexpr int BM = C::BM, BN = C::BN, HN = BN / 2;
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ int32_t sprefix[512];
  __shared__ float ssw[2][F8_MAX_KB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;

  for (int i = tid; i <= a.n_seg; i += C::THREADS) sprefix[i] = a.mtile_prefix[i];
  __syncthreads();
  const int n_tiles = SWIGLU ? a.N / HN : a.N / BN;
  int seg, ntile, mtile;
  // XCD-contiguous logical ranges, as in the bf16 kernels
  const int total_tiles = sprefix[a.n_seg] * n_tiles;
  const int per_xcd = (total_tiles + 7) >> 3;
  const int lt = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if ((int)(blockIdx.x >> 3) >= per_xcd) return;
  if (!decode_tile(sprefix, a.n_seg, n_tiles, lt, seg, ntile, mtile)) return;

  const int row0 = a.offsets[seg] + mtile * BM;
  const int mvalid = min(BM, a.offsets[seg + 1] - row0);
  const int K = a.K, KB = K / F8_BK, KS = K / F8_SK;
  const bool first = seg < a.n_first;
  const uint8_t* wbase = first ? (const uint8_t*)a.w0 + (size_t)seg * a.wstride0
                               : (const uint8_t*)a.w1 + (size_t)(seg - a.n_first) * a.wstride1;
  const float* wsc = first ? a.ws0 + (size_t)seg * a.sstride0 : a.ws1 + (size_t)(seg - a.n_first) * a.sstride1;

  // weight-block rows of the tile: SwiGLU gate rows / up rows; down: the two 128-row halves
  const int blk0 = SWIGLU ? ntile : 2 * ntile;
  const int blk1 = SWIGLU ? a.N / 128 + ntile : 2 * ntile + 1;
  for (int i = tid; i < KB; i += C::THREADS) {
    ssw[0][i] = wsc[(size_t)blk0 * KB + i];
    ssw[1][i] = wsc[(size_t)blk1 * KB + i];
  }

  // ---- per-lane global offsets of this wave's loads (fixed over K)
  const int lrow = lane >> 2;                                  // row within a 16-row load
  const int lchunk = (lane & 3) ^ ((lane >> 4) & 3);           // chunk its slot holds
  // K-blocked activation codes (the down GEMM's H, written so by the gate/up GEMM's epilogue):
  // per m-tile, per 64-element step, the tile's BM rows with the chunk swizzle applied, so
  // load i of a stage reads its kilobyte i; rows past mvalid hold padding, whose products
  // only reach output rows that are not stored
  const bool xblk = a.x_blocked;
  const int mt = sprefix[seg] + mtile;
  const i32x4 xr = xblk ? rsrc_words((const uint8_t*)a.x + (size_t)mt * BM * K, (long)BM * K)
                        : rsrc_words(a.x, a.x_rows * (long)K);
  const int astep = xblk ? BM * F8_SK : F8_SK;
  const i32x4 sr = rsrc_words(a.x_scale, a.x_rows * (long)KB * 4);
  // K-blocked weights (moe_pack_expert_weights): the tile's 256 rows per 64-element step are
  // one contiguous 16 KB with this kernel's chunk swizzle applied, so load i of a stage reads
  // its kilobyte i
  const bool wblk = a.w_blocked;
  const i32x4 wr = wblk ? rsrc_words(wbase + (size_t)ntile * BN * K, (long)BN * K)
                        : rsrc_words(wbase, (long)(SWIGLU ? 2 * a.N : a.N) * K);
  const int bstep = wblk ? BN * F8_SK : F8_SK;
  // wave w loads A blocks w, w + 8, ...: waves below A_LOADS % 8 take one more
  const int n_a = (C::A_LOADS % 8 == 0 || wave < C::A_LOADS % 8) ? C::A_MAX : C::A_MIN;
  int aoff[C::A_MAX];
#pragma unroll
  for (int i = 0; i < C::A_MAX; i++) {
    const int r = (wave + 8 * i) * 16 + lrow;
    const int rr = min(max(row0 + min(r, mvalid - 1), 0), a.rows_bound - 1);   // in range for any offsets
    const int src = a.row_index ? a.row_index[rr] : rr;
    aoff[i] = xblk ? (wave + 8 * i) * 1024 + lane * 16 : r < mvalid ? src * K + lchunk * 16 : kOutOfRange;
  }
  int soff_row;
  {
    const int r = (wave < C::SA_WAVES ? wave : 0) * 64 + lane;
    const int rr = min(max(row0 + min(r, mvalid - 1), 0), a.rows_bound - 1);   // in range for any offsets
    const int src = a.row_index ? a.row_index[rr] : rr;
    soff_row = r < mvalid ? src * KB * 4 : kOutOfRange;
  }
  int boff[C::B_PER_WAVE];
#pragma unroll
  for (int i = 0; i < C::B_PER_WAVE; i++) {
    const int r = (wave + 8 * i) * 16 + lrow;
    const int wrow = SWIGLU ? (r < HN ? ntile * HN + r : a.N + ntile * HN + (r - HN)) : ntile * BN + r;
    boff[i] = wblk ? (wave + 8 * i) * 1024 + lane * 16 : wrow * K + lchunk * 16;
  }
  const uint32_t lds0 = lds_addr(lds);
  const bool sa_wave = wave < C::SA_WAVES;
  // Load P of this wave's share of stage ks into buffer buf: its B blocks (the weight
  // codes, read from HBM, so issued first: measured at V3, the gate/up GEMM 2.98 -> 2.91 ms
  // against A first), then its A blocks, then (waves below SA_WAVES) the row scales of
  // the stage's 128-block.
  // Only the first stage of a 128-block reads the row scales (it rescales the
  // accumulators), so only stages of even index load them: each of those loads
  // gathers 64 separate 4-byte values. Of any two consecutive stages exactly one
  // is even, which keeps the waits' counts the same for every stage.
  constexpr int NPARTS = C::A_MAX + C::B_PER_WAVE + 1;
  auto issue_part = [&](auto p_tag, auto sa_tag, int ks, int buf) __attribute__((always_inline)) {
    constexpr int P = decltype(p_tag)::value;
    constexpr bool SA = decltype(sa_tag)::value;
    const uint32_t sbase = lds0 + buf * C::STAGE;
    if constexpr (P >= C::B_PER_WAVE && P < C::A_MAX + C::B_PER_WAVE) {
      constexpr int Q = P - C::B_PER_WAVE;
      if (Q < C::A_MIN || n_a == C::A_MAX) dma_b128(xr, aoff[Q], ks * astep, sbase + (wave + 8 * Q) * 1024);
    } else if constexpr (P < C::B_PER_WAVE) {
      constexpr int Q = P;
      // K-blocked gate/up weights are read with the non-temporal hint (measured: it helps the
      // gate/up GEMM and slows the down GEMM, whose H rows are re-read by its 28 n-tiles)
      if (SWIGLU && wblk) dma_b128_nt(wr, boff[Q], ks * bstep, sbase + C::A_BYTES + (wave + 8 * Q) * 1024);
      else dma_b128(wr, boff[Q], ks * bstep, sbase + C::A_BYTES + (wave + 8 * Q) * 1024);
    } else {
      if (SA && sa_wave) dma_b32(sr, soff_row, (ks >> 1) * 4, sbase + C::A_BYTES + C::B_BYTES + wave * 256);
    }
  };
  auto issue = [&](auto sa_tag, int ks, int buf) __attribute__((always_inline)) {
    static_for<NPARTS>([&](auto p) __attribute__((always_inline)) { issue_part(p, sa_tag, ks, buf); });
  };
  // this wave's loads of stage ks are done when at most those of the two later stages are
  // pending: its A and B loads of both and one row-scale load (waves below SA_WAVES)
  const int n_pend = 2 * (n_a + C::B_PER_WAVE) + (sa_wave ? 1 : 0);
  auto wait_stage = [&]() __attribute__((always_inline)) {
    if (n_pend == 11) wait_vmcnt<11>();
    else if (n_pend == 10) wait_vmcnt<10>();
    else if (n_pend == 9) wait_vmcnt<9>();
    else if (n_pend == 8) wait_vmcnt<8>();
    else wait_vmcnt<0>();
  };

  f32x16 acc[MB][2];
#pragma unroll
  for (int i = 0; i < MB; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;
  int mb_active = 0;
#pragma unroll
  for (int i = 0; i < MB; i++)
    if ((2 * i + wm) * 32 < mvalid) mb_active = i + 1;

  // operand reads: lane l32 reads row block*32 + l32 (whose (row >> 2) & 3 is (l32 >> 2) & 3),
  // the 32 bytes of K half khalf: chunks 2*khalf and 2*khalf + 1
  const int l32 = lane & 31, khalf = lane >> 5;
  const int sw = (l32 >> 2) & 3;
  const int roff0 = l32 * F8_SK + (((2 * khalf) ^ sw) << 4);
  const int roff1 = l32 * F8_SK + (((2 * khalf + 1) ^ sw) << 4);
  const int bro[2] = {(SWIGLU ? wn * 32 : wn * 64) * F8_SK, (SWIGLU ? HN + wn * 32 : wn * 64 + 32) * F8_SK};
  // which staged weight-scale row each of this wave's two weight blocks uses
  const int wsel0 = SWIGLU ? 0 : (wn >> 1), wsel1 = SWIGLU ? 1 : (wn >> 1);

  // Each accumulator holds its block's sum in units of the current 128-block's
  // scale s = s_act[this lane's row] * s_w[block]: acc = sum_kb p_kb * s_kb / s_cur.
  // At the first 64-element stage of a 128-block it is rescaled by s_prev / s_cur
  // (one reciprocal and 16 multiplies per lane and block); then both stages'
  // MFMAs accumulate into it directly, and the epilogue multiplies by the last
  // block's s. This is the pages' fp32 promotion, sum_kb s_kb * p_kb, with the
  // scale applied once per 128 elements instead of once per 64-element partial,
  // and no partial registers. A zero scale (no such tile comes out of the
  // quantisers; rows past the segment read zero scales) keeps the previous one.
  float sprev[MB][2];
#pragma unroll
  for (int i = 0; i < MB; i++) sprev[i][0] = sprev[i][1] = 1.0f;
  // The loads of stage ksl into buffer bufl. The gate/up GEMM spreads them
  // between the blocks' MFMAs (one before the first block, one after each
  // block, the rest at the end), so the texture unit's queues do not fill with
  // a burst after every barrier; the down GEMM issues them in one burst before
  // its MFMAs (measured at V3: spreading took the gate/up GEMM from 3.10 to
  // 3.04 ms and the down GEMM from 1.69 to 1.71 ms).
  constexpr bool SPREAD = SWIGLU;
  auto compute_na = [&](auto na_tag, auto first_tag, int buf, int ks, int ksl, int bufl)
                        __attribute__((always_inline)) {
    constexpr int NA = decltype(na_tag)::value;
    constexpr bool FIRST = decltype(first_tag)::value;
    // the loads go 3 stages ahead: the first stage of a pair loads an odd stage, the second an even
    using SAL = std::integral_constant<bool, !FIRST>;
    if constexpr (SPREAD) issue_part(std::integral_constant<int, 0>{}, SAL{}, ksl, bufl);
    else issue(SAL{}, ksl, bufl);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NA > 0) {
      const uint8_t* A = lds + buf * C::STAGE;
      const uint8_t* B = A + C::A_BYTES;
      const float* SA = (const float*)(B + C::B_BYTES);
      float swj[2] = {1.0f, 1.0f};
      if constexpr (FIRST) {
        swj[0] = ssw[wsel0][ks >> 1];
        swj[1] = ssw[wsel1][ks >> 1];
      }
      i32x8 bfr[2];
#pragma unroll
      for (int j = 0; j < 2; j++) {
        const i32x4 lo = *(const i32x4*)(B + bro[j] + roff0);
        const i32x4 hi = *(const i32x4*)(B + bro[j] + roff1);
        bfr[j] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
      static_for<NA>([&](auto I) __attribute__((always_inline)) {
        constexpr int i = decltype(I)::value;
        const int mrow = (2 * i + wm) * 32;
        const i32x4 lo = *(const i32x4*)(A + mrow * F8_SK + roff0);
        const i32x4 hi = *(const i32x4*)(A + mrow * F8_SK + roff1);
        const i32x8 afr = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        if constexpr (FIRST) {
          const float sa = SA[mrow + l32];
#pragma unroll
          for (int j = 0; j < 2; j++) {
            const float sc = sa * swj[j];
            const float se = sc != 0.0f ? sc : sprev[i][j];
            const float r = sprev[i][j] * __builtin_amdgcn_rcpf(se);
            sprev[i][j] = se;
#pragma unroll
            for (int e = 0; e < 16; e++) acc[i][j][e] *= r;
          }
        }
        // cbsz = blgp = 0: both operands E4M3; scale exponents 127 = 2^0
#pragma unroll
        for (int j = 0; j < 2; j++)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bfr[j], afr, acc[i][j], 0, 0, 0, 127, 0, 127);
        if constexpr (SPREAD && i + 1 < NPARTS) {
          __builtin_amdgcn_sched_barrier(0);
          issue_part(std::integral_constant<int, i + 1>{}, SAL{}, ksl, bufl);
          __builtin_amdgcn_sched_barrier(0);
        }
      });
    }
    static_for<NPARTS>([&](auto p_tag) __attribute__((always_inline)) {
      constexpr int P = decltype(p_tag)::value;
      if constexpr (SPREAD && P > NA) issue_part(p_tag, SAL{}, ksl, bufl);
    });
    __builtin_amdgcn_sched_barrier(0);
  };

  // Four-stage ring: wait for this wave's loads of stage ks, barrier (every
  // wave's data for ks is in LDS, every wave is done with ks-1), refill ks-1's
  // buffer with ks+3 while multiplying ks. Past
  // the last stage the refills repeat it into buffers no later stage reads,
  // so every wave issues the same loads per stage.
  auto k_loop = [&](auto na_tag) __attribute__((always_inline)) {
    const int last = KS - 1;
    issue(std::true_type{}, 0, 0);
    issue(std::false_type{}, min(1, last), 1);
    issue(std::true_type{}, min(2, last), 2);
    // K % 128 == 0: the stages come in pairs, the first of each pair rescales
    for (int ks = 0; ks < KS; ks += 2) {
      wait_stage();
      __syncthreads();
      compute_na(na_tag, std::true_type{}, ks & 3, ks, min(ks + 3, last), (ks + 3) & 3);
      wait_stage();
      __syncthreads();
      compute_na(na_tag, std::false_type{}, (ks + 1) & 3, ks + 1, min(ks + 4, last), (ks + 4) & 3);
    }
    wait_vmcnt<0>();   // no LDS write may land after the workgroup ends
  };
  switch (__builtin_amdgcn_readfirstlane(mb_active)) {
    case 0: k_loop(std::integral_constant<int, 0>{}); break;
    case 1: k_loop(std::integral_constant<int, 1>{}); break;
    case 2: k_loop(std::integral_constant<int, 2>{}); break;
    case 3: k_loop(std::integral_constant<int, (MB >= 3 ? 3 : MB)>{}); break;
    case 4: k_loop(std::integral_constant<int, (MB >= 4 ? 4 : MB)>{}); break;
    default: k_loop(std::integral_constant<int, MB>{}); break;
  }
  // back from units of the last 128-block's scale
#pragma unroll
  for (int i = 0; i < MB; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int e = 0; e < 16; e++) acc[i][j][e] *= sprev[i][j];

  // Each lane holds one activation row (its column in the MFMA layout) and, per block,
  // 16 weight rows 8q + 4*khalf + e: 4 consecutive output columns per q.
  if constexpr (SWIGLU) {
    if (a.out_q) {
      // H quantised here, in 1x128 tiles along I: a tile is this n-tile's 128 H columns of
      // one row, 32 per wave wn and 16 per lane. Its amax over the lane pair (khalf) and
      // the 4 waves goes through LDS; scale and codes as the activation quantiser makes them.
      __shared__ float samax[4][BM];
      // H values once, for every block (inactive ones hold zeros): the accumulators die here
      float hv[MB][16];
#pragma unroll
      for (int i = 0; i < MB; i++) {
        float m = 0.f;
#pragma unroll
        for (int r = 0; r < 16; r++) {
          hv[i][r] = silu_mul(acc[i][0][r], acc[i][1][r]);
          m = fmaxf(m, fabsf(hv[i][r]));
        }
        m = fmaxf(m, __shfl_xor(m, 32));
        if (i < mb_active && khalf == 0) samax[wn][(2 * i + wm) * 32 + l32] = m;
      }
      __syncthreads();
      const int tpr = a.N / 128;
#pragma unroll
      for (int i = 0; i < MB; i++) {
        const int row = (2 * i + wm) * 32 + l32;
        if (i < mb_active && row < mvalid && (unsigned)(row0 + row) < (unsigned)a.rows_bound) {
          const float m = fmaxf(fmaxf(samax[0][row], samax[1][row]), fmaxf(samax[2][row], samax[3][row]));
          const float sc = m == 0.0f ? 1.0f : m / 448.0f;
          // column c = ntile*128 + wn*32 + 8q + 4khalf of H: row-major, or K-blocked for the down
          // GEMM (m-tile mt, step c/64, tile row `row`, 16-byte chunk (c%64)/16 at its swizzled slot)
          const int c0 = ntile * HN + wn * 32 + 4 * khalf;
          uint8_t* qrow = a.out_blocked ? a.out_q + (size_t)mt * BM * a.N + (size_t)row * F8_SK
                                        : a.out_q + (size_t)(row0 + row) * a.N;
#pragma unroll
          for (int q = 0; q < 4; q++) {
            const int c = c0 + 8 * q;
            const int at = a.out_blocked
                ? (c / F8_SK) * BM * F8_SK + ((((c % F8_SK) >> 4) ^ ((row >> 2) & 3)) << 4) + (c & 15)
                : c;
            *(uint32_t*)(qrow + at) = e4m3_encode4(hv[i][4 * q] / sc, hv[i][4 * q + 1] / sc,
                                                   hv[i][4 * q + 2] / sc, hv[i][4 * q + 3] / sc);
          }
          if (wn == 0 && khalf == 0) a.out_qs[(size_t)(row0 + row) * tpr + ntile] = sc;
        }
      }
      return;
    }
  }
  // Without out_q, GEMM1 writes H in fp32; GEMM2 writes Y in bf16.
#pragma unroll
  for (int i = 0; i < MB; i++) {
    const int row = (2 * i + wm) * 32 + l32;
    if (i < mb_active && row < mvalid && (unsigned)(row0 + row) < (unsigned)a.rows_bound) {
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int m = 8 * q + 4 * khalf;
        if (SWIGLU) {
          float* orow = (float*)a.out + (size_t)(row0 + row) * a.N + ntile * HN + wn * 32 + m;
          f32x4 h;
#pragma unroll
          for (int e = 0; e < 4; e++) h[e] = silu_mul(acc[i][0][4 * q + e], acc[i][1][4 * q + e]);
          *(f32x4*)orow = h;
        } else {
          uint16_t* orow = (uint16_t*)a.out + (size_t)(row0 + row) * a.N + ntile * BN + wn * 64 + m;
#pragma unroll
          for (int j = 0; j < 2; j++) {
            const uint32_t lo = f32_to_bf16(acc[i][j][4 * q]) | ((uint32_t)f32_to_bf16(acc[i][j][4 * q + 1]) << 16);
            const uint32_t hi = f32_to_bf16(acc[i][j][4 * q + 2]) | ((uint32_t)f32_to_bf16(acc[i][j][4 * q + 3]) << 16);
            *(uint2*)(orow + 32 * j) = make_uint2(lo, hi);
          }
        }
      }
    }
  }
}

template <int MB, bool SWIGLU>
static hipError_t launch_fp8_dma(const GemmArgs& a, hipStream_t s) {
  using C = F8DmaCfg<MB>;
  if (a.K / F8_BK > F8_MAX_KB) return hipErrorInvalidValue;
  const int n_tiles = SWIGLU ? a.N / (C::BN / 2) : a.N / C::BN;
  const long grid = (((long)a.rows_bound / C::BM + a.n_seg) * n_tiles + 7) / 8 * 8;
  if (grid <= 0) return hipSuccess;
  auto k = gemm_fp8_dma_kernel<MB, SWIGLU>;
  hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, C::BYTES);
  if (e != hipSuccess) return e;
  k<<<dim3((unsigned)grid), C::THREADS, C::BYTES, s>>>(a);
  return hipGetLastError();
}

template <int MB, bool SWIGLU>
static hipError_t launch_fp8_t(const GemmArgs& a, hipStream_t s) {
  const int n_tiles = SWIGLU ? a.N / 64 : a.N / GF_BN;
  const long grid = (((long)a.rows_bound / (64 * MB) + a.n_seg) * n_tiles + 7) / 8 * 8;
  if (grid <= 0) return hipSuccess;
  auto k = gemm_fp8_kernel<MB, SWIGLU>;
  hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     Fp8Lds<MB>::BYTES);
  if (e != hipSuccess) return e;
  k<<<dim3((unsigned)grid), GF_THREADS, Fp8Lds<MB>::BYTES, s>>>(a);
  return hipGetLastError();
}

// dst[mat][tile][step][256 rows][64 bytes]: row r's 16-byte chunk c of a
// 64-element step sits at slot c ^ ((r >> 2) & 3), where the LDS-DMA kernel's
// lane for that slot fetches it from a row-major operand
__global__ void pack_blocked_f8_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, long n_chunks,
                                       int rows, int K, int swiglu_i) {
  const int steps = K / F8_SK, tiles = rows / 256;
  for (long q = (long)blockIdx.x * blockDim.x + threadIdx.x; q < n_chunks; q += (long)gridDim.x * blockDim.x) {
    const int slot = (int)(q & 3);
    const int r = (int)((q >> 2) & 255);
    long rest = q >> 10;
    const int ks = (int)(rest % steps);
    rest /= steps;
    const int t = (int)(rest % tiles);
    const long mat = rest / tiles;
    const int srow = swiglu_i > 0 ? (r < 128 ? t * 128 + r : swiglu_i + t * 128 + (r - 128)) : t * 256 + r;
    const int c = slot ^ ((r >> 2) & 3);
    *(i32x4*)(dst + (size_t)q * 16) = *(const i32x4*)(src + ((size_t)mat * rows + srow) * K + ks * F8_SK + c * 16);
  }
}

hipError_t launch_pack_blocked_f8(const uint8_t* src, uint8_t* dst, int n_mat, int rows, int K, int swiglu_i,
                                  hipStream_t s) {
  if (rows % 256 || K % F8_BK || (swiglu_i > 0 && rows != 2 * swiglu_i)) return hipErrorInvalidValue;
  const long n_chunks = (long)n_mat * rows * (K / 16);
  if (n_chunks <= 0) return hipSuccess;
  const int blocks = (int)std::min<long>(cdiv<long>(n_chunks, 256), 8192);
  pack_blocked_f8_kernel<<<blocks, 256, 0, s>>>(src, dst, n_chunks, rows, K, swiglu_i);
  return hipGetLastError();
}

hipError_t launch_gemm_fp8(const GemmArgs& a, bool swiglu, int bm, hipStream_t s) {
  // K-blocked weights only on the LDS-DMA kernel; blocked activations are a bf16 feature
  // blocked activation codes: the down GEMM reads them (x_blocked), the gate/up GEMM's fused
  // quantisation writes them (out_blocked), both on the LDS-DMA kernel (256- or 320-row tiles)
  const bool dma = bm == 256 || bm == 320;
  if ((a.x_blocked && (swiglu || !dma || a.row_index)) || (a.out_blocked && (!swiglu || !dma || !a.out_q)) ||
      (a.w_blocked && !dma))
    return hipErrorInvalidValue;
  if (a.out_q && (!swiglu || !a.out_qs || a.N % 128)) return hipErrorInvalidValue;
  if (a.out_q && bm == 192) {
    // the 192-row kernel writes fp32 H (a.out); it is quantised by the activation quantiser
    GemmArgs b = a;
    b.out_q = nullptr;
    b.out_qs = nullptr;
    hipError_t e = launch_fp8_t<3, true>(b, s);
    if (e != hipSuccess) return e;
    return launch_quant_act(a.out, MOE_F32, a.rows_bound, a.N, nullptr, a.out_q, a.out_qs, s);
  }
  // 256- and 320-row tiles: the LDS-DMA kernel (needs the down GEMM's width a multiple of 256)
  if (bm == 256) return swiglu ? launch_fp8_dma<4, true>(a, s) : launch_fp8_dma<4, false>(a, s);
  if (bm == 320) return swiglu ? launch_fp8_dma<5, true>(a, s) : launch_fp8_dma<5, false>(a, s);
  if (bm == 192) return swiglu ? launch_fp8_t<3, true>(a, s) : launch_fp8_t<3, false>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace moe
