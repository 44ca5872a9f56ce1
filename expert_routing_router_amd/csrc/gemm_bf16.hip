// Grouped expert GEMMs in bf16 on gfx950 MFMA (fp32 accumulation).
//
// The layer's expert FFNs (output equation of the DeepSeek-V3 guides,
// "Metodo" section 2) run as two grouped GEMMs over the permuted rows:
//   GEMM1 (swiglu): H[r, n] = SiLU(x_r . W1_e[n]) * (x_r . W3_e[n])
//   GEMM2 (down):   Y[r, n] = H_r . W2_e[n]
// for every row r of segment e. Segments are the routed experts followed by
// the shared experts (their rows are every token, identity order).
//
// Tiling. A workgroup is 4 waves (2 along M x 2 along N) and owns one
// (segment, n-tile, m-tile). The m-tile is 64*MB rows tall, sized on the host
// so that one m-tile covers a typical expert's rows: each weight tile then
// streams from HBM about once per forward. Waves take interleaved 32-row
// m-blocks (wave wm: blocks wm, wm+2, ...) so a partly filled m-tile keeps
// both M-waves equally busy; m-blocks past the segment's end skip their
// MFMAs. B tiles are 128 weight rows: for GEMM1, 64 rows of W1 and the same
// 64 rows of W3, so the gate and up accumulators of one output element sit in
// the same lane and SwiGLU is applied in registers.
//
// Data path: global -> registers (prefetch of step k+1) -> LDS (double
// buffer, 16-byte chunks XOR-swizzled by row so MFMA operand reads are
// conflict-free) -> v_mfma_f32_32x32x16_bf16.
#include "common.h"
#include "lds_dma.h"
#include "tile_order.h"
#include "moe_internal.h"
#include <cmath>
#include <type_traits>

namespace moe {

constexpr int GB_BK = 64;          // bf16 elements per K step (128 bytes per row)

// MB: 32-row m-blocks per wave (tile height 64*MB); WN: waves along N. The
// workgroup is 2*WN waves (2 along M); its B tile is 64*WN weight rows.
template <int MB, int WN>
struct GemmCfg {
  static constexpr int THREADS = 128 * WN;
  static constexpr int BM = 64 * MB;
  static constexpr int BN = 64 * WN;
  static constexpr int A_BYTES = BM * GB_BK * 2;
  static constexpr int B_BYTES = BN * GB_BK * 2;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int BYTES = 2 * STAGE;
  static constexpr int ROWS_PER_PASS = THREADS / 8;   // rows one load instruction covers per WG
  static constexpr int ACH = BM / ROWS_PER_PASS;       // A 16-byte chunks per thread
  static constexpr int BCH = BN / ROWS_PER_PASS;       // B chunks per thread
};

// 16-byte chunk c of row r sits in slot c ^ (r & 7) ^ ((r >> 3) & 1) of the
// row's 128 bytes: the MFMA operand reads (16 consecutive lanes = 16
// consecutive rows, one chunk) then touch 16 distinct 4-bank groups of a
// 64-bank LDS, and any 8 consecutive rows 8 distinct groups of a 32-bank one.
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * 128 + ((chunk ^ (row & 7) ^ ((row >> 3) & 1)) << 4);
}

template <int MB, int WN, bool SWIGLU>
__global__ __launch_bounds__(128 * WN, 1) void gemm_bf16_kernel(GemmArgs a) {
  using C = GemmCfg<MB, WN>;
  constexpr int BM = C::BM, BN = C::BN, ACH = C::ACH, BCH = C::BCH, RPP = C::ROWS_PER_PASS;
  constexpr int HN = BN / 2;              // SwiGLU: output columns per tile
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ int32_t sprefix[512];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;

  for (int i = tid; i <= a.n_seg; i += C::THREADS) sprefix[i] = a.mtile_prefix[i];
  __syncthreads();
  const int n_tiles = SWIGLU ? a.N / HN : a.N / BN;
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

  const int seg_begin = a.offsets[seg], seg_end = a.offsets[seg + 1];
  const int row0 = seg_begin + mtile * BM;
  const int mvalid = min(BM, seg_end - row0);
  const int K = a.K;
  const uint16_t* wbase = seg < a.n_first
      ? (const uint16_t*)a.w0 + (size_t)seg * a.wstride0
      : (const uint16_t*)a.w1 + (size_t)(seg - a.n_first) * a.wstride1;

  // ---- per-thread global source offsets, fixed over K
  const int cch = tid & 7;          // 16-byte chunk within a 128-byte row slice
  const int rbase = tid >> 3;       // 0 .. RPP-1
  // A rows: byte offsets into x; rows past the segment read zeros (out of range)
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(a.x, a.x_rows * (long)K * 2);
  int aoff[ACH];
#pragma unroll
  for (int i = 0; i < ACH; i++) {
    const int r = rbase + RPP * i;
    const int rr = min(max(row0 + min(r, mvalid - 1), 0), a.rows_bound - 1);   // in range for any offsets
    const int src = a.row_index ? a.row_index[rr] : rr;
    aoff[i] = r < mvalid ? (src * K + cch * 8) * 2 : kOutOfRange;
  }
  const __amdgpu_buffer_rsrc_t wr = make_rsrc(wbase, (long)(SWIGLU ? 2 * a.N : a.N) * K * 2);
  int boff[BCH];
#pragma unroll
  for (int i = 0; i < BCH; i++) {
    const int br = rbase + RPP * i;   // 0 .. BN-1
    int wrow;
    if (SWIGLU) wrow = br < HN ? ntile * HN + br : (a.N + ntile * HN + (br - HN));
    else wrow = ntile * BN + br;
    boff[i] = (wrow * K + cch * 8) * 2;
  }

  i32x4 ra[ACH], rb[BCH];
  auto gload = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < ACH; i++) ra[i] = __builtin_amdgcn_raw_buffer_load_b128(xr, aoff[i] + k0 * 2, 0, 0);
#pragma unroll
    for (int i = 0; i < BCH; i++)   // weights are streamed once: non-temporal (slc)
      rb[i] = __builtin_amdgcn_raw_buffer_load_b128(wr, boff[i] + k0 * 2, 0, 2);
  };
  auto sstore = [&](int buf) __attribute__((always_inline)) {
    uint8_t* A = lds + buf * C::STAGE;
    uint8_t* B = A + C::A_BYTES;
#pragma unroll
    for (int i = 0; i < ACH; i++) *(i32x4*)(A + swz(rbase + RPP * i, cch)) = ra[i];
#pragma unroll
    for (int i = 0; i < BCH; i++) *(i32x4*)(B + swz(rbase + RPP * i, cch)) = rb[i];
  };

  f32x16 acc[MB][2];
#pragma unroll
  for (int i = 0; i < MB; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;

  // active m-blocks of this wave (wave-uniform)
  int mb_active = 0;
#pragma unroll
  for (int i = 0; i < MB; i++)
    if ((2 * i + wm) * 32 < mvalid) mb_active = i + 1;

  const int l32 = lane & 31, khalf = lane >> 5;
  // One K step from LDS buffer `buf` with NA active m-blocks, NA a compile-time
  // count: straight-line code, all LDS reads of a k-substep ahead of its MFMAs.
  auto compute_na = [&](auto na_tag, int buf) __attribute__((always_inline)) {
    constexpr int NA = decltype(na_tag)::value;
    const uint8_t* A = lds + buf * C::STAGE;
    const uint8_t* B = A + C::A_BYTES;
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
      const int ch = ks * 2 + khalf;
      bf16x8 bfr[2], afr[NA > 0 ? NA : 1];
#pragma unroll
      for (int j = 0; j < 2; j++) {
        const int brow = (SWIGLU ? j * HN + wn * 32 : wn * 64 + j * 32) + l32;
        bfr[j] = *(const bf16x8*)(B + swz(brow, ch));
      }
#pragma unroll
      for (int i = 0; i < NA; i++) afr[i] = *(const bf16x8*)(A + swz((2 * i + wm) * 32 + l32, ch));
#pragma unroll
      for (int i = 0; i < NA; i++) {
        acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afr[i], bfr[0], acc[i][0], 0, 0, 0);
        acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afr[i], bfr[1], acc[i][1], 0, 0, 0);
      }
    }
  };
  // Every load and LDS store in the K loop is unconditional (the trailing
  // prefetch re-reads the last step): with no branch around a memory op the
  // compiler's wait counting stays in order.
  const int nk = K / GB_BK;
  auto k_loop = [&](auto na_tag) __attribute__((always_inline)) {
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; kt++) {
      gload(min(kt + 1, nk - 1) * GB_BK);
      compute_na(na_tag, kt & 1);
      sstore((kt + 1) & 1);
      __syncthreads();
    }
  };
  // mb_active is the same in every lane of the wave: branch once, outside the
  // loop. A wave with no active m-block still loads its share and takes part
  // in every barrier.
  switch (__builtin_amdgcn_readfirstlane(mb_active)) {
    case 0: k_loop(std::integral_constant<int, 0>{}); break;
    case 1: k_loop(std::integral_constant<int, 1>{}); break;
    case 2: k_loop(std::integral_constant<int, 2>{}); break;
    case 3: k_loop(std::integral_constant<int, (MB >= 3 ? 3 : MB)>{}); break;
    case 4: k_loop(std::integral_constant<int, (MB >= 4 ? 4 : MB)>{}); break;
    default: k_loop(std::integral_constant<int, MB>{}); break;
  }

  // ---- epilogue: D element (8*(r>>2) + 4*(lane>>5) + (r&3), lane&31) in register r
  uint16_t* out = (uint16_t*)a.out;
#pragma unroll
  for (int i = 0; i < MB; i++) {
    if (i < mb_active) {
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int row = (2 * i + wm) * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
        if (row < mvalid && (unsigned)(row0 + row) < (unsigned)a.rows_bound) {
          uint16_t* orow = out + (size_t)(row0 + row) * a.N;
          if (SWIGLU) {
            const int col = ntile * HN + wn * 32 + l32;
            orow[col] = f32_to_bf16(silu_mul(acc[i][0][r], acc[i][1][r]));
          } else {
            const int col = ntile * BN + wn * 64 + l32;
            orow[col] = f32_to_bf16(acc[i][0][r]);
            orow[col + 32] = f32_to_bf16(acc[i][1][r]);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------- LDS-DMA path
// Same tile and wave layout as gemm_bf16_kernel<MB, 4, ...> (8 waves, 64*MB x
// 256 weight rows), but operands go from global memory straight into LDS with
// buffer loads that write LDS (no register staging), through a ring of K=32
// stages, as many as the LDS holds (4 for 256- and 320-row tiles, 6 and 7 for
// 128- and 64-row tiles): all but one are in flight while one is multiplied,
// so each CU keeps ~108 KB of loads outstanding instead of one K step's worth.
//
// A stage holds RB = 64 bytes per row (K=32 stages: two 16-element k-substeps,
// which the operand read-ahead of the kernel needs), CPR = RB/16 chunks of 16 bytes. One load instruction of a
// wave fills one 1 KB block of RPB = 1024/RB rows; lane l writes block byte
// 16*l, i.e. row l/CPR, slot l%CPR, and fetches the chunk
// c = slot ^ ((row >> SH) & (CPR-1)), SH = log2(16/CPR). The MFMA operand
// reads (16 lanes = 16 consecutive rows, one chunk) then hit 16 distinct
// 4-bank groups.
template <int MB, int RB>
struct DmaCfg {
  static constexpr int THREADS = 512;
  static constexpr int BM = 64 * MB;
  static constexpr int BN = 256;
  static constexpr int BK = RB / 2;                     // bf16 elements per stage row
  static constexpr int CPR = RB / 16;
  static constexpr int RPB = 1024 / RB;
  static constexpr int SH = 2;
  static constexpr int SUB = RB / 32;                   // 16-element k-substeps per stage
  // as many K=32 stages as the LDS holds (up to 7: small-row tiles keep more weight bytes in flight)
  static constexpr int STAGES = (160 * 1024 - 2048) / ((BM + BN) * RB) < 7
                                    ? (160 * 1024 - 2048) / ((BM + BN) * RB) : 7;
  static constexpr int A_BLOCKS = BM / RPB;             // 1 KB blocks per stage
  static constexpr int B_BLOCKS = BN / RPB;
  static constexpr int A_BYTES = BM * RB;
  static constexpr int STAGE = (BM + BN) * RB;
  static constexpr int BYTES = STAGES * STAGE;
  static constexpr int A_PER_WAVE = (A_BLOCKS + 7) / 8;  // waves below A_BLOCKS % 8 take one more
  static constexpr int A_EXTRA = A_BLOCKS % 8;
  static constexpr int B_PER_WAVE = B_BLOCKS / 8;
  static_assert(RB == 64, "stage row bytes");
  static_assert(B_BLOCKS % 8 == 0, "B blocks split evenly over 8 waves");
  static_assert(BYTES <= 160 * 1024 - 2048, "LDS budget");
};

// WBLK: the weights are K-blocked (a.w_blocked); they are then read with the
// non-temporal hint, whole lines at a time, so they do not push the activation
// rows the tile's other n-tiles re-read out of L2
template <int MB, bool SWIGLU, int RB, bool WBLK>
__global__ __launch_bounds__(512, 1) void gemm_bf16_dma_kernel(GemmArgs a) {
  using C = DmaCfg<MB, RB>;
  constexpr int BM = C::BM, BN = C::BN, HN = BN / 2;
  extern __shared__ __align__(16) uint8_t lds[];
  __shared__ int32_t sprefix[512];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;

  for (int i = tid; i <= a.n_seg; i += C::THREADS) sprefix[i] = a.mtile_prefix[i];
  __syncthreads();
  const int n_tiles = SWIGLU ? a.N / HN : a.N / BN;
  int seg, ntile, mtile;
  // XCD-contiguous logical ranges, as in gemm_bf16_kernel
  const int total_tiles = sprefix[a.n_seg] * n_tiles;
  const int per_xcd = (total_tiles + 7) >> 3;
  const int lt = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if ((int)(blockIdx.x >> 3) >= per_xcd) return;
  if (!decode_tile(sprefix, a.n_seg, n_tiles, lt, seg, ntile, mtile)) return;

  const int seg_begin = a.offsets[seg], seg_end = a.offsets[seg + 1];
  const int row0 = seg_begin + mtile * BM;
  const int mvalid = min(BM, seg_end - row0);
  const int K = a.K;
  const int mt = sprefix[seg] + mtile;                // this m-tile's index over all segments
  const uint16_t* wbase = seg < a.n_first
      ? (const uint16_t*)a.w0 + (size_t)seg * a.wstride0
      : (const uint16_t*)a.w1 + (size_t)(seg - a.n_first) * a.wstride1;
  const bool xblk = a.x_blocked;
  constexpr bool wblk = WBLK;

  // ---- per-lane global offsets of this wave's blocks (fixed over K). Block
  // wave + 8i starts at row RPB*(wave + 8i); the +8i part leaves the swizzle unchanged.
  const int brow = lane / C::CPR;                              // row within a block
  const int bchunk = (lane % C::CPR) ^ (((C::RPB * wave + brow) >> C::SH) & (C::CPR - 1));
  // K-blocked operands: the tile's block is the buffer (rows past mvalid hold
  // padding, whose products only reach output rows that are not stored), and
  // block i of a stage is its kilobyte i; else rows are addressed in place
  const i32x4 xr = xblk ? rsrc_words((const uint16_t*)a.x + (size_t)mt * BM * K, (long)BM * K * 2)
                        : rsrc_words(a.x, a.x_rows * (long)K * 2);
  const i32x4 wr = wblk ? rsrc_words(wbase + (size_t)ntile * BN * K, (long)BN * K * 2)
                        : rsrc_words(wbase, (long)(SWIGLU ? 2 * a.N : a.N) * K * 2);
  const int astep = xblk ? BM * RB : RB, bstep = wblk ? BN * RB : RB;   // bytes per K step
  int aoff[C::A_PER_WAVE];
#pragma unroll
  for (int i = 0; i < C::A_PER_WAVE; i++) {
    const int r = (wave + 8 * i) * C::RPB + brow;   // blocks past A_BLOCKS are never issued
    const int rr = min(max(row0 + min(r, mvalid - 1), 0), a.rows_bound - 1);   // in range for any offsets
    const int src = a.row_index ? a.row_index[rr] : rr;
    aoff[i] = xblk ? (wave + 8 * i) * 1024 + lane * 16 : r < mvalid ? (src * K + bchunk * 8) * 2 : kOutOfRange;
  }
  int boff[C::B_PER_WAVE];
#pragma unroll
  for (int i = 0; i < C::B_PER_WAVE; i++) {
    const int r = (wave + 8 * i) * C::RPB + brow;   // 0 .. BN-1
    const int wrow = SWIGLU ? (r < HN ? ntile * HN + r : a.N + ntile * HN + (r - HN)) : ntile * BN + r;
    boff[i] = wblk ? (wave + 8 * i) * 1024 + lane * 16 : (wrow * K + bchunk * 8) * 2;
  }
  const uint32_t lds0 = lds_addr(lds);
  constexpr int A_EXTRA = C::A_EXTRA;           // waves below this issue A_PER_WAVE blocks
  const bool a_full = A_EXTRA == 0 || wave < A_EXTRA;
  // Part P of this wave's stage loads for step kt into buffer buf: its A
  // blocks first (the last one only on waves that have it), then its B blocks.
  auto issue_part = [&](auto p_tag, int kt, int buf) __attribute__((always_inline)) {
    constexpr int P = decltype(p_tag)::value;
    const uint32_t sbase = lds0 + buf * C::STAGE;
    if constexpr (P < C::A_PER_WAVE) {
      if (P < C::A_PER_WAVE - 1 || a_full) dma_b128(xr, aoff[P], kt * astep, sbase + (wave + 8 * P) * 1024);
    } else if constexpr (P < C::A_PER_WAVE + C::B_PER_WAVE) {
      constexpr int Q = P - C::A_PER_WAVE;
      if constexpr (WBLK) dma_b128_nt(wr, boff[Q], kt * bstep, sbase + C::A_BYTES + (wave + 8 * Q) * 1024);
      else dma_b128(wr, boff[Q], kt * bstep, sbase + C::A_BYTES + (wave + 8 * Q) * 1024);
    }
  };
  constexpr int NPARTS = C::A_PER_WAVE + C::B_PER_WAVE;
  auto issue = [&](int kt, int buf) __attribute__((always_inline)) {
    static_for<NPARTS>([&](auto p) __attribute__((always_inline)) { issue_part(p, kt, buf); });
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

  // operand read offsets: row = block*32 + l32 has the swizzle of row l32
  const int l32 = lane & 31, khalf = lane >> 5;
  const int sw = (l32 >> C::SH) & (C::CPR - 1);
  int roff[C::SUB];                                  // k-substep ks: chunk 2*ks + khalf
#pragma unroll
  for (int ks = 0; ks < C::SUB; ks++) roff[ks] = l32 * RB + (((2 * ks + khalf) ^ sw) << 4);
  // B rows of this wave: SwiGLU gate rows wn*32.. and up rows HN + wn*32..; else wn*64 + j*32
  const int bro0 = (SWIGLU ? wn * 32 : wn * 64) * RB;
  const int bro1 = (SWIGLU ? HN + wn * 32 : wn * 64 + 32) * RB;

  // Operand reads run half a stage ahead of the MFMAs, across the barrier.
  // Iteration kt enters with k-substep 0 of stage kt in registers. It
  // multiplies that substep while reading substep 1 of stage kt, waits for
  // stage kt+1 and meets the barrier, reads substep 0 of stage kt+1, then
  // multiplies substep 1 of stage kt. The matrix core thus holds queued work
  // while the waves meet at the barrier, and the first MFMAs after it need no
  // read. Stage kt's buffer is free at that barrier (every wave has read it,
  // and the barrier waits for the reads), so stage kt+S is loaded into it:
  // its first PA loads between the MFMAs of substep 1, the rest between those
  // of substep 0 of the next iteration, before its barrier.
  static_assert(C::SUB == 2, "two 16-element k-substeps per stage");
  constexpr int S = C::STAGES;
  // loads of stage kt+S issued right after the barrier (the rest go before the next one):
  // the gate/up GEMM at MB = 5 issues 3 of its 5 there (measured at V3: 4.28 -> 4.23 ms
  // against 2; 4 gained nothing), the down GEMM half (1 or 3 moved it within noise)
  constexpr int PA = SWIGLU && NPARTS == 5 ? 3 : NPARTS / 2;
  const int nk = K / C::BK;
  auto k_loop = [&](auto na_tag) __attribute__((always_inline)) {
    constexpr int NA = decltype(na_tag)::value;
    constexpr int NA1 = NA > 0 ? NA : 1;
    bf16x8 ra[2][NA1], rb[2][2];             // [k-substep]
    auto read_sub = [&](auto s_tag, int buf) __attribute__((always_inline)) {
      constexpr int SS = decltype(s_tag)::value;
      const uint8_t* A = lds + buf * C::STAGE;
      const uint8_t* B = A + C::A_BYTES;
      rb[SS][0] = *(const bf16x8*)(B + bro0 + roff[SS]);
      rb[SS][1] = *(const bf16x8*)(B + bro1 + roff[SS]);
#pragma unroll
      for (int i = 0; i < NA; i++) ra[SS][i] = *(const bf16x8*)(A + (2 * i + wm) * 32 * RB + roff[SS]);
    };
    // the NA MFMA pairs of k-substep SS, with loads P0..P1-1 of step kti into buffer
    // bufi spread between them (the rest after them when few m-blocks are active)
    auto mma_sub = [&](auto s_tag, auto p0_tag, auto p1_tag, int kti, int bufi) __attribute__((always_inline)) {
      constexpr int SS = decltype(s_tag)::value;
      constexpr int P0 = decltype(p0_tag)::value, P1 = decltype(p1_tag)::value;
      constexpr int NP = P1 - P0;
      constexpr int PER = NA > 0 && NP > 0 ? (NA + NP - 1) / NP : 1;
      if constexpr (NP > 0) issue_part(std::integral_constant<int, P0>{}, kti, bufi);
      __builtin_amdgcn_sched_barrier(0);
      static_for<MB>([&](auto q_tag) __attribute__((always_inline)) {
        constexpr int q = decltype(q_tag)::value;
        if constexpr (q < NA) {
          // weight rows first: each lane's results are 4-column runs of one activation row
          acc[q][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rb[SS][0], ra[SS][q], acc[q][0], 0, 0, 0);
          acc[q][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rb[SS][1], ra[SS][q], acc[q][1], 0, 0, 0);
          if constexpr ((q + 1) % PER == 0 && (q + 1) / PER < NP) {
            __builtin_amdgcn_sched_barrier(0);
            issue_part(std::integral_constant<int, P0 + (q + 1) / PER>{}, kti, bufi);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      });
      static_for<NPARTS>([&](auto p_tag) __attribute__((always_inline)) {
        constexpr int P = decltype(p_tag)::value;
        if constexpr (P > P0 && P < P1 && P - P0 > NA / PER) issue_part(p_tag, kti, bufi);
      });
      __builtin_amdgcn_sched_barrier(0);
    };
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    using PAc = std::integral_constant<int, PA>;
    // prologue: stages 0..S-2 whole and the first part of stage S-1 (clamped re-reads of
    // the last step past it, into buffers never read again), then substep 0 of stage 0
#pragma unroll
    for (int p = 0; p < S - 1; p++) issue(min(p, nk - 1), p);
    static_for<PA>([&](auto p) __attribute__((always_inline)) { issue_part(p, min(S - 1, nk - 1), S - 1); });
    if (a_full) wait_vmcnt<(S - 2) * NPARTS + PA>();
    else wait_vmcnt<(S - 2) * (NPARTS - 1) + (PA > C::A_PER_WAVE - 1 ? PA - 1 : PA)>();
    __syncthreads();
    read_sub(S0{}, 0);
    for (int kt = 0; kt < nk - 1; kt++) {
      // substep 0 of stage kt, with the second part of stage kt+S-1's loads
      mma_sub(S0{}, PAc{}, std::integral_constant<int, NPARTS>{}, min(kt + S - 1, nk - 1), (kt + S - 1) % S);
      read_sub(S1{}, kt % S);
      // stage kt+1 has landed once this wave's loads of it are done (the S-2 younger
      // stages may stay outstanding) and every wave has passed the barrier
      if (a_full) wait_vmcnt<(S - 2) * NPARTS>();
      else wait_vmcnt<(S - 2) * (NPARTS - 1)>();
      __syncthreads();
      read_sub(S0{}, (kt + 1) % S);
      __builtin_amdgcn_sched_barrier(0);
      // substep 1 of stage kt, with the first part of stage kt+S's loads into stage kt's buffer
      mma_sub(S1{}, S0{}, PAc{}, min(kt + S, nk - 1), kt % S);
    }
    // the last stage: no further stage to wait for, read or load
    mma_sub(S0{}, S0{}, S0{}, 0, 0);
    read_sub(S1{}, (nk - 1) % S);
    mma_sub(S1{}, S0{}, S0{}, 0, 0);
    wait_vmcnt<0>();   // no LDS write may land after the workgroup ends
  };
  switch (__builtin_amdgcn_readfirstlane(mb_active)) {
    case 0: k_loop(std::integral_constant<int, 0>{}); break;
    case 1: k_loop(std::integral_constant<int, 1>{}); break;
    case 2: k_loop(std::integral_constant<int, (MB >= 2 ? 2 : MB)>{}); break;
    case 3: k_loop(std::integral_constant<int, (MB >= 3 ? 3 : MB)>{}); break;
    case 4: k_loop(std::integral_constant<int, (MB >= 4 ? 4 : MB)>{}); break;
    default: k_loop(std::integral_constant<int, MB>{}); break;
  }

  // The MFMA takes the weight rows as its first operand, so lane l holds activation row
  // (block row + l32) and, in registers 4q..4q+3, the 4 output columns 8q + 4*khalf + e of
  // each 32-column n-block: every (q) is one 8-byte store of 4 bf16.
  uint16_t* out = (uint16_t*)a.out;
  // K-blocked H (SwiGLU only): this wave's 32 columns are one 32-element step of the down GEMM
  uint16_t* hblk = out + ((size_t)mt * (a.N / 32) + (ntile * HN + wn * 32) / 32) * BM * 32;
  auto pack4 = [](float v0, float v1, float v2, float v3) __attribute__((always_inline)) {
    return make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
  };
#pragma unroll
  for (int i = 0; i < MB; i++) {
    const int row = (2 * i + wm) * 32 + l32;
    if (i < mb_active && row < mvalid && (unsigned)(row0 + row) < (unsigned)a.rows_bound) {
      uint16_t* orow = out + (size_t)(row0 + row) * a.N;
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const int c = 8 * q + 4 * khalf;
        if (SWIGLU) {
          const uint2 h = pack4(silu_mul(acc[i][0][4 * q], acc[i][1][4 * q]),
                                silu_mul(acc[i][0][4 * q + 1], acc[i][1][4 * q + 1]),
                                silu_mul(acc[i][0][4 * q + 2], acc[i][1][4 * q + 2]),
                                silu_mul(acc[i][0][4 * q + 3], acc[i][1][4 * q + 3]));
          // blocked: chunk q of the row at its swizzled slot, elements 4*khalf.. within it
          uint16_t* dst = a.out_blocked ? hblk + row * 32 + ((q ^ ((row >> 2) & 3)) << 3) + 4 * khalf
                                        : orow + ntile * HN + wn * 32 + c;
          *(uint2*)dst = h;
        } else {
#pragma unroll
          for (int j = 0; j < 2; j++)
            *(uint2*)(orow + ntile * BN + wn * 64 + j * 32 + c) =
                pack4(acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------- fp32 path
// fp32 experts (the small fp32 layer): MI355X's fp32 vector rate equals its
// fp32 matrix rate, so a plain VALU kernel is the fp32 path. One thread per
// output element, fp32 FMA along K.
template <bool SWIGLU>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs a) {
  __shared__ int32_t soff[512];
  for (int i = threadIdx.x; i <= a.n_seg; i += 256) soff[i] = a.offsets[i];
  __syncthreads();
  const int col = blockIdx.x * 64 + (threadIdx.x & 63);
  const int r = blockIdx.y * 4 + (threadIdx.x >> 6);
  if (r >= soff[a.n_seg] || col >= a.N) return;
  int lo = 0, hi = a.n_seg - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (soff[mid] <= r) lo = mid; else hi = mid - 1;
  }
  const int seg = lo;
  const float* w = seg < a.n_first ? (const float*)a.w0 + (size_t)seg * a.wstride0
                                   : (const float*)a.w1 + (size_t)(seg - a.n_first) * a.wstride1;
  const int src = a.row_index ? a.row_index[r] : r;
  const float* xr = (const float*)a.x + (size_t)src * a.K;
  float* out = (float*)a.out + (size_t)r * a.N + col;
  if (SWIGLU) {
    const float* w1 = w + (size_t)col * a.K;
    const float* w3 = w + (size_t)(a.N + col) * a.K;
    float g = 0.f, u = 0.f;
    for (int k = 0; k < a.K; k++) {
      g = fmaf(xr[k], w1[k], g);
      u = fmaf(xr[k], w3[k], u);
    }
    *out = g / (1.0f + expf(-g)) * u;
  } else {
    const float* w2 = w + (size_t)col * a.K;
    float y = 0.f;
    for (int k = 0; k < a.K; k++) y = fmaf(xr[k], w2[k], y);
    *out = y;
  }
}

int gemm_bm(int dtype, int mean_rows, int dmodel, int inter) {
  // one m-tile per expert when the mean load (+4 sigma of a binomial load) fits;
  // 64- and 128-row tiles (deeper load ring) for small loads when every product's
  // width suits the LDS-DMA kernel
  const int need = mean_rows + 4 * (int)std::sqrt((double)(mean_rows > 0 ? mean_rows : 1));
  // FP8: 256- or 320-row tiles of the LDS-DMA kernel when the down GEMM's width is a
  // multiple of its 256-row weight tile, else the register-staged 192-row kernel.
  if (dtype == MOE_FP8_E4M3) return dmodel % 256 != 0 ? 192 : need <= 256 ? 256 : 320;
  const bool dma_all = dmodel % 256 == 0 && inter % 256 == 0;
  if (dma_all && need <= 64) return 64;
  if (dma_all && need <= 128) return 128;
  if (need <= 256) return 256;
  return 320;
}

template <int MB, int WN, bool SWIGLU>
static hipError_t launch_bf16(const GemmArgs& a, hipStream_t s) {
  using C = GemmCfg<MB, WN>;
  const int n_tiles = SWIGLU ? a.N / (C::BN / 2) : a.N / C::BN;
  const long mtiles_bound = (long)a.rows_bound / C::BM + a.n_seg;
  const long grid = (mtiles_bound * n_tiles + 7) / 8 * 8;   // a multiple of the 8 XCDs
  if (grid <= 0) return hipSuccess;
  auto k = gemm_bf16_kernel<MB, WN, SWIGLU>;
  hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, C::BYTES);
  if (e != hipSuccess) return e;
  k<<<dim3((unsigned)grid), C::THREADS, C::BYTES, s>>>(a);
  return hipGetLastError();
}

template <int MB, bool SWIGLU>
static hipError_t launch_bf16_dma(const GemmArgs& a, hipStream_t s) {
  constexpr int RB = 64;
  using C = DmaCfg<MB, RB>;
  const int n_tiles = SWIGLU ? a.N / (C::BN / 2) : a.N / C::BN;
  const long mtiles_bound = (long)a.rows_bound / C::BM + a.n_seg;
  const long grid = (mtiles_bound * n_tiles + 7) / 8 * 8;
  if (grid <= 0) return hipSuccess;
  auto k = a.w_blocked ? gemm_bf16_dma_kernel<MB, SWIGLU, RB, true> : gemm_bf16_dma_kernel<MB, SWIGLU, RB, false>;
  hipError_t e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, C::BYTES);
  if (e != hipSuccess) return e;
  k<<<dim3((unsigned)grid), C::THREADS, C::BYTES, s>>>(a);
  return hipGetLastError();
}

template <bool SWIGLU>
static hipError_t launch_any(const GemmArgs& a, int dtype, int bm, hipStream_t s) {
  if (dtype == MOE_F32) {
    const dim3 grid(cdiv(a.N, 64), cdiv(a.rows_bound, 4));
    if (grid.y == 0) return hipSuccess;
    gemm_f32_kernel<SWIGLU><<<grid, 256, 0, s>>>(a);
    return hipGetLastError();
  }
  if (dtype == MOE_BF16) {
    // 256 weight rows per tile (8 waves) when the output width allows it,
    // else 128 (4 waves)
    const bool wide = SWIGLU ? a.N % 128 == 0 : a.N % 256 == 0;
    if ((a.w_blocked || a.x_blocked || a.out_blocked) && (!wide || a.K % 32)) return hipErrorInvalidValue;
    if (bm == 64) return wide ? launch_bf16_dma<1, SWIGLU>(a, s) : hipErrorInvalidValue;
    if (bm == 128) return wide ? launch_bf16_dma<2, SWIGLU>(a, s) : hipErrorInvalidValue;
    if (bm == 256) return wide ? launch_bf16_dma<4, SWIGLU>(a, s) : launch_bf16<4, 2, SWIGLU>(a, s);
    if (bm == 320) return wide ? launch_bf16_dma<5, SWIGLU>(a, s) : launch_bf16<5, 2, SWIGLU>(a, s);
    return hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------- K-blocked weights
// dst[mat][tile][step][256 rows][32 elements]: row r of a tile stores its
// 16-byte chunk c of the step at slot c ^ ((r >> 2) & 3), which is where the
// LDS-DMA kernel's lane for that slot fetches it from a row-major operand.
__global__ void pack_blocked_kernel(const uint16_t* __restrict__ src, uint16_t* __restrict__ dst, long n_chunks,
                                    int rows, int K, int swiglu_i) {
  const int steps = K / 32, tiles = rows / 256;
  for (long q = (long)blockIdx.x * blockDim.x + threadIdx.x; q < n_chunks; q += (long)gridDim.x * blockDim.x) {
    const int slot = (int)(q & 3);
    const int r = (int)((q >> 2) & 255);
    long rest = q >> 10;
    const int kt = (int)(rest % steps);
    rest /= steps;
    const int t = (int)(rest % tiles);
    const long mat = rest / tiles;
    const int srow = swiglu_i > 0 ? (r < 128 ? t * 128 + r : swiglu_i + t * 128 + (r - 128)) : t * 256 + r;
    const int c = slot ^ ((r >> 2) & 3);
    const i32x4 v = *(const i32x4*)(src + ((size_t)mat * rows + srow) * K + kt * 32 + c * 8);
    *(i32x4*)(dst + (size_t)q * 8) = v;
  }
}

hipError_t launch_pack_blocked(const uint16_t* src, uint16_t* dst, int n_mat, int rows, int K, int swiglu_i,
                               hipStream_t s) {
  if (rows % 256 || K % 32 || (swiglu_i > 0 && rows != 2 * swiglu_i)) return hipErrorInvalidValue;
  const long n_chunks = (long)n_mat * rows * (K / 8);
  if (n_chunks <= 0) return hipSuccess;
  const int blocks = (int)std::min<long>(cdiv<long>(n_chunks, 256), 8192);
  pack_blocked_kernel<<<blocks, 256, 0, s>>>(src, dst, n_chunks, rows, K, swiglu_i);
  return hipGetLastError();
}

hipError_t launch_gemm_fp8(const GemmArgs& a, bool swiglu, int bm, hipStream_t s);

hipError_t launch_gemm_swiglu(const GemmArgs& a, int dtype, int bm, hipStream_t s) {
  if (dtype == MOE_FP8_E4M3) return launch_gemm_fp8(a, true, bm, s);
  return launch_any<true>(a, dtype, bm, s);
}
hipError_t launch_gemm_down(const GemmArgs& a, int dtype, int bm, hipStream_t s) {
  if (dtype == MOE_FP8_E4M3) return launch_gemm_fp8(a, false, bm, s);
  return launch_any<false>(a, dtype, bm, s);
}

}  // namespace moe
