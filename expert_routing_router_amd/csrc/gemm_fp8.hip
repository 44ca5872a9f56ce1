// Grouped expert GEMMs with E4M3 operands and fine-grained fp32 scales.
//
// The pages' FP8 recipe (DeepSeek-V3 guides on xyznot.com, FP8 key idea;
// pwwt.cn note section 3): E4M3 inputs, one scale per 1x128 activation tile
// and per 128x128 weight block, partial sums promoted to fp32 every 128
// K-elements. On gfx950 the MFMA already accumulates in fp32, so the promotion
// becomes: for every 128-wide K block, two v_mfma 32x32x64 f8f6f4 produce a
// fresh fp32 partial, which is folded into the accumulator as
//   acc += partial * (s_act[row, kb] * s_w[nblock, kb]).
// The per-row activation scales of the tile are staged in LDS beside A.
// Tiling, ragged segments and the SwiGLU epilogue follow the bf16 kernel.
#include "common.h"
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
// 8 waves (2 along M x 4 along N), tile 64*MB rows x 256 weight rows, one
// 128-wide K block (= one scale block) per stage, two stages. Buffer loads
// write the E4M3 rows and the rows' activation scales straight into LDS. The
// two weight-block scales a workgroup needs per K block (gate and up rows for
// SwiGLU, the two 128-row halves of the tile for the down GEMM) are staged in
// LDS once, for all K blocks.
//
// A stage row is 128 bytes = 8 chunks of 16; one load instruction of a wave
// fills 8 rows (1 KB): lane l writes row l>>3, slot l&7 and fetches chunk
// slot ^ ((row >> 1) & 7), so the MFMA operand reads (16 lanes = 16
// consecutive rows, one chunk) hit 16 distinct 4-bank groups.
constexpr int F8_BK = 128;
constexpr int F8_MAX_KB = 256;          // K <= 32768

template <int MB>
struct F8DmaCfg {
  static constexpr int THREADS = 512;
  static constexpr int BM = 64 * MB;
  static constexpr int BN = 256;
  static constexpr int A_BLOCKS = BM / 8;            // 1 KB blocks
  static constexpr int B_BLOCKS = BN / 8;
  static constexpr int A_BYTES = BM * F8_BK;
  static constexpr int B_BYTES = BN * F8_BK;
  static constexpr int SA_BYTES = BM * 4;
  static constexpr int STAGE = A_BYTES + B_BYTES + SA_BYTES;
  static constexpr int BYTES = 2 * STAGE;
  static constexpr int A_PER_WAVE = A_BLOCKS / 8;
  static constexpr int B_PER_WAVE = B_BLOCKS / 8;
  static constexpr int SA_WAVES = BM / 64;           // waves that load 64 row scales each
  static_assert(A_BLOCKS % 8 == 0 && B_BLOCKS % 8 == 0, "blocks split evenly over 8 waves");
  static_assert(SA_WAVES <= 8, "row scales");
  static_assert(BYTES + 2 * F8_MAX_KB * 4 + 2048 <= 160 * 1024, "LDS budget");
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
  const int K = a.K, KB = K / F8_BK;
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

  // ---- per-lane global offsets of this wave's blocks (fixed over K)
  const int brow = lane >> 3;
  const int bchunk = (lane & 7) ^ ((((wave & 1) << 2) + (lane >> 4)) & 7);   // block parity = wave parity
  const i32x4 xr = rsrc_words(a.x, a.x_rows * (long)K);
  const i32x4 sr = rsrc_words(a.x_scale, a.x_rows * (long)KB * 4);
  // K-blocked weights (moe_pack_expert_weights): the tile's 256 rows per 128-element block are one
  // contiguous 32 KB with this kernel's chunk swizzle applied, so block i of a stage is its kilobyte i
  const bool wblk = a.w_blocked;
  const i32x4 wr = wblk ? rsrc_words(wbase + (size_t)ntile * BN * K, (long)BN * K)
                        : rsrc_words(wbase, (long)(SWIGLU ? 2 * a.N : a.N) * K);
  const int bstep = wblk ? BN * F8_BK : F8_BK;
  int aoff[C::A_PER_WAVE];
#pragma unroll
  for (int i = 0; i < C::A_PER_WAVE; i++) {
    const int r = (wave + 8 * i) * 8 + brow;
    const int rr = min(max(row0 + min(r, mvalid - 1), 0), a.rows_bound - 1);   // in range for any offsets
    const int src = a.row_index ? a.row_index[rr] : rr;
    aoff[i] = r < mvalid ? src * K + bchunk * 16 : kOutOfRange;
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
    const int r = (wave + 8 * i) * 8 + brow;
    const int wrow = SWIGLU ? (r < HN ? ntile * HN + r : a.N + ntile * HN + (r - HN)) : ntile * BN + r;
    boff[i] = wblk ? (wave + 8 * i) * 1024 + lane * 16 : wrow * K + bchunk * 16;
  }
  const uint32_t lds0 = lds_addr(lds);
  const bool sa_wave = wave < C::SA_WAVES;
  auto issue = [&](int kb, int buf) __attribute__((always_inline)) {
    const int koff = kb * F8_BK;
    const uint32_t sbase = lds0 + buf * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::A_PER_WAVE; i++) dma_b128(xr, aoff[i], koff, sbase + (wave + 8 * i) * 1024);
#pragma unroll
    for (int i = 0; i < C::B_PER_WAVE; i++)
      dma_b128(wr, boff[i], kb * bstep, sbase + C::A_BYTES + (wave + 8 * i) * 1024);
    if (sa_wave) dma_b32(sr, soff_row, kb * 4, sbase + C::A_BYTES + C::B_BYTES + wave * 256);
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

  // operand reads: rows block*32 + l32 share (row >> 1) & 7 == (l32 >> 1) & 7
  const int l32 = lane & 31, khalf = lane >> 5;
  const int sw = (l32 >> 1) & 7;
  int roff[2][2];
#pragma unroll
  for (int h = 0; h < 2; h++)
#pragma unroll
    for (int c = 0; c < 2; c++) roff[h][c] = l32 * 128 + (((h * 4 + khalf * 2 + c) ^ sw) << 4);
  const int bro[2] = {(SWIGLU ? wn * 32 : wn * 64) * 128, (SWIGLU ? HN + wn * 32 : wn * 64 + 32) * 128};
  // which staged weight-scale row each of this wave's two n-blocks uses
  const int wsel0 = SWIGLU ? 0 : (wn >> 1), wsel1 = SWIGLU ? 1 : (wn >> 1);

  // One K block from stage `buf`: per 32x32 block two MFMAs into a fresh fp32
  // partial, then acc += partial * (s_act[row] * s_w).
  auto compute_na = [&](auto na_tag, int buf, int kb) __attribute__((always_inline)) {
    constexpr int NA = decltype(na_tag)::value;
    const uint8_t* A = lds + buf * C::STAGE;
    const uint8_t* B = A + C::A_BYTES;
    const float* SA = (const float*)(B + C::B_BYTES);
    const float swj[2] = {ssw[wsel0][kb], ssw[wsel1][kb]};
    i32x8 bfr[2][2];
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int h = 0; h < 2; h++) {
        const i32x4 lo = *(const i32x4*)(B + bro[j] + roff[h][0]);
        const i32x4 hi = *(const i32x4*)(B + bro[j] + roff[h][1]);
        bfr[j][h] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
    for (int i = 0; i < NA; i++) {
      const int mrow = (2 * i + wm) * 32;
      i32x8 afr[2];
#pragma unroll
      for (int h = 0; h < 2; h++) {
        const i32x4 lo = *(const i32x4*)(A + mrow * 128 + roff[h][0]);
        const i32x4 hi = *(const i32x4*)(A + mrow * 128 + roff[h][1]);
        afr[h] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
      // this lane's 16 accumulator rows: 8*q + 4*khalf + e, q, e in 0..3
      f32x4 sa[4];
#pragma unroll
      for (int q = 0; q < 4; q++) sa[q] = *(const f32x4*)(SA + mrow + 8 * q + 4 * khalf);
#pragma unroll
      for (int j = 0; j < 2; j++) {
        f32x16 p;
#pragma unroll
        for (int r = 0; r < 16; r++) p[r] = 0.f;
        // cbsz = blgp = 0: both operands E4M3; scale exponents 127 = 2^0
        p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(afr[0], bfr[j][0], p, 0, 0, 0, 127, 0, 127);
        p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(afr[1], bfr[j][1], p, 0, 0, 0, 127, 0, 127);
#pragma unroll
        for (int r = 0; r < 16; r++) acc[i][j][r] = fmaf(p[r], sa[r >> 2][r & 3] * swj[j], acc[i][j][r]);
      }
    }
  };

  // Two-stage ring: wait for this wave's loads of stage kb, barrier (every
  // wave's data for kb is in LDS, every wave is done with kb-1), refill the
  // other buffer with kb+1, multiply kb.
  auto k_loop = [&](auto na_tag) __attribute__((always_inline)) {
    issue(0, 0);
    for (int kb = 0; kb < KB; kb++) {
      wait_vmcnt<0>();
      __syncthreads();
      issue(min(kb + 1, KB - 1), (kb + 1) & 1);
      compute_na(na_tag, kb & 1, kb);
    }
    wait_vmcnt<0>();   // no LDS write may land after the workgroup ends
  };
  switch (__builtin_amdgcn_readfirstlane(mb_active)) {
    case 0: k_loop(std::integral_constant<int, 0>{}); break;
    case 1: k_loop(std::integral_constant<int, 1>{}); break;
    case 2: k_loop(std::integral_constant<int, 2>{}); break;
    case 3: k_loop(std::integral_constant<int, (MB >= 3 ? 3 : MB)>{}); break;
    default: k_loop(std::integral_constant<int, MB>{}); break;
  }

  // GEMM1 writes H in fp32 (re-quantised per 1x128 tile next); GEMM2 writes Y in bf16.
#pragma unroll
  for (int i = 0; i < MB; i++) {
    if (i < mb_active) {
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int row = (2 * i + wm) * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
        if (row < mvalid && (unsigned)(row0 + row) < (unsigned)a.rows_bound) {
          if (SWIGLU) {
            float* orow = (float*)a.out + (size_t)(row0 + row) * a.N;
            orow[ntile * HN + wn * 32 + l32] = silu_mul(acc[i][0][r], acc[i][1][r]);
          } else {
            uint16_t* orow = (uint16_t*)a.out + (size_t)(row0 + row) * a.N;
            const int col = ntile * BN + wn * 64 + l32;
            orow[col] = f32_to_bf16(acc[i][0][r]);
            orow[col + 32] = f32_to_bf16(acc[i][1][r]);
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

// dst[mat][tile][block][256 rows][128 bytes]: row r's 16-byte chunk c of a
// 128-element block sits at slot c ^ ((r >> 1) & 7), where the LDS-DMA kernel's
// lane for that slot fetches it from a row-major operand
__global__ void pack_blocked_f8_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, long n_chunks,
                                       int rows, int K, int swiglu_i) {
  const int blocks = K / F8_BK, tiles = rows / 256;
  for (long q = (long)blockIdx.x * blockDim.x + threadIdx.x; q < n_chunks; q += (long)gridDim.x * blockDim.x) {
    const int slot = (int)(q & 7);
    const int r = (int)((q >> 3) & 255);
    long rest = q >> 11;
    const int kb = (int)(rest % blocks);
    rest /= blocks;
    const int t = (int)(rest % tiles);
    const long mat = rest / tiles;
    const int srow = swiglu_i > 0 ? (r < 128 ? t * 128 + r : swiglu_i + t * 128 + (r - 128)) : t * 256 + r;
    const int c = slot ^ ((r >> 1) & 7);
    *(i32x4*)(dst + (size_t)q * 16) = *(const i32x4*)(src + ((size_t)mat * rows + srow) * K + kb * F8_BK + c * 16);
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
  if (a.x_blocked || a.out_blocked || (a.w_blocked && bm != 256)) return hipErrorInvalidValue;
  // 256-row tiles: the LDS-DMA kernel (needs the down GEMM's width a multiple of 256)
  if (bm == 256) return swiglu ? launch_fp8_dma<4, true>(a, s) : launch_fp8_dma<4, false>(a, s);
  if (bm == 192) return swiglu ? launch_fp8_t<3, true>(a, s) : launch_fp8_t<3, false>(a, s);
  return hipErrorInvalidValue;
}

}  // namespace moe
