// Backward pass of the DeepSeekMoE layer (bf16 experts), for the routing the
// forward chose.
//
// Forward (output equation of the xyznot.com DeepSeek-V3 guides, "Metodo"
// section 2): out_t = u_t + sum_s FFN_s(u_t) + sum_k g_{t,k} FFN_{idx_k}(u_t),
// g = s_sel / sum(s_sel), s = Sigmoid(u E^T), FFN(x) = W2 (SiLU(W1 x) * W3 x).
// The selection and the bias are piecewise constant (the bias only routes:
// pwwt.cn note 1.1.2-1.1.3), so with dout = d(loss)/d(out):
//   dY_{t,k}   = g_{t,k} dout_t              (routed rows), dout_t (shared rows)
//   dg_{t,k}   = <dout_t, Y_{t,k}>
//   dH = dY W2,  dA = dH * B * sig(A) * (1 + A (1 - sig(A))),  dB = dH * SiLU(A)
//   dX = [dA dB] W13,  dW2 = dY^T H,  dW13 = [dA dB]^T X       (per expert)
//   ds_{t,k}   = (dg_{t,k} - sum_j g_{t,j} dg_{t,j}) / sum_j s_{t,j}
//   dz_{t,k}   = ds_{t,k} s_{t,k} (1 - s_{t,k})
//   du_t = dout_t + sum_s dX_s,t + sum_k dX_{t,k} + sum_k dz_{t,k} e_{idx_k}
//   dE_i = sum over tokens that selected i of dz_{t,k} u_t
// This file holds the element-wise pieces, the per-expert weight-gradient
// GEMM and the weight transposes; the dense GEMMs (A|B, Y, dH, dX) reuse the
// forward's grouped GEMM kernels with transposed weight copies.
#include "common.h"
#include "lds_dma.h"
#include "moe_internal.h"

namespace moe {

__device__ __forceinline__ void load_bf16x8(const uint16_t* p, float* v) {
  const i32x4 q = *(const i32x4*)p;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    v[2 * i] = __uint_as_float(((uint32_t)q[i]) << 16);
    v[2 * i + 1] = __uint_as_float(((uint32_t)q[i]) & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void store_bf16x8(uint16_t* p, const float* v) {
  i32x4 q;
#pragma unroll
  for (int i = 0; i < 4; i++) q[i] = (int)pack_bf16x2(v[2 * i], v[2 * i + 1]);
  *(i32x4*)p = q;
}
// 8 consecutive elements of a bf16 (F32 = false) or fp32 array, as fp32
template <bool F32>
__device__ __forceinline__ void ld8(const void* p, size_t i, float* v) {
  if constexpr (F32) {
    const f32x4 a = *(const f32x4*)((const float*)p + i), b = *(const f32x4*)((const float*)p + i + 4);
#pragma unroll
    for (int k = 0; k < 4; k++) { v[k] = a[k]; v[4 + k] = b[k]; }
  } else {
    load_bf16x8((const uint16_t*)p + i, v);
  }
}
template <bool F32>
__device__ __forceinline__ void st8(void* p, size_t i, const float* v) {
  if constexpr (F32) {
    *(f32x4*)((float*)p + i) = f32x4{v[0], v[1], v[2], v[3]};
    *(f32x4*)((float*)p + i + 4) = f32x4{v[4], v[5], v[6], v[7]};
  } else {
    store_bf16x8((uint16_t*)p + i, v);
  }
}
__device__ __forceinline__ float sigmoidf_(float a) { return 1.0f / (1.0f + __expf(-a)); }

// H = SiLU(A) * B from AB = [A | B] (rows of 2I), bf16 (or fp32) in and out, fp32 math
template <bool F32>
__global__ void swiglu_fwd_kernel(const void* __restrict__ ab, void* __restrict__ h, long rows, int I) {
  const long n8 = rows * (I / 8);
  for (long p = (long)blockIdx.x * blockDim.x + threadIdx.x; p < n8; p += (long)gridDim.x * blockDim.x) {
    const long r = p / (I / 8);
    const int c = (int)(p - r * (I / 8)) * 8;
    float a[8], b[8], o[8];
    ld8<F32>(ab, r * 2 * I + c, a);
    ld8<F32>(ab, r * 2 * I + I + c, b);
#pragma unroll
    for (int i = 0; i < 8; i++) o[i] = a[i] * sigmoidf_(a[i]) * b[i];
    st8<F32>(h, r * I + c, o);
  }
}

// dA, dB from dH and AB: dA = dH * B * sig(A) * (1 + A (1 - sig(A))), dB = dH * SiLU(A)
template <bool F32>
__global__ void swiglu_bwd_kernel(const void* __restrict__ dh, const void* __restrict__ ab,
                                  void* __restrict__ dab, long rows, int I) {
  const long n8 = rows * (I / 8);
  for (long p = (long)blockIdx.x * blockDim.x + threadIdx.x; p < n8; p += (long)gridDim.x * blockDim.x) {
    const long r = p / (I / 8);
    const int c = (int)(p - r * (I / 8)) * 8;
    float a[8], b[8], g[8], da[8], db[8];
    ld8<F32>(ab, r * 2 * I + c, a);
    ld8<F32>(ab, r * 2 * I + I + c, b);
    ld8<F32>(dh, r * I + c, g);
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const float sg = sigmoidf_(a[i]);
      da[i] = g[i] * b[i] * sg * (1.0f + a[i] * (1.0f - sg));
      db[i] = g[i] * a[i] * sg;
    }
    st8<F32>(dab, r * 2 * I + c, da);
    st8<F32>(dab, r * 2 * I + I + c, db);
  }
}

// One workgroup per token: the K gate gradients dg = <dout_t, Y_{t,k}> (fp32),
// and the rows of dY: g * dout for its routed rows, dout for its shared rows.
template <bool F32>
__global__ __launch_bounds__(256) void dgate_dy_kernel(const void* __restrict__ dout, const void* __restrict__ y,
                                                       const int32_t* __restrict__ slot_row, const float* __restrict__ gate,
                                                       int d, int K, int n_shared, long shared_base, long shared_stride,
                                                       float* __restrict__ dg, void* __restrict__ dy) {
  __shared__ float red[64][4];
  const int t = blockIdx.x, lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const size_t drow = (size_t)t * d;
  for (int k = 0; k < K; k++) {
    const long row = slot_row[(size_t)t * K + k];
    const float g = gate[(size_t)t * K + k];
    float acc = 0.f;
    for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
      float a[8], b[8], o[8];
      ld8<F32>(dout, drow + c, a);
      ld8<F32>(y, row * d + c, b);
#pragma unroll
      for (int i = 0; i < 8; i++) { acc = fmaf(a[i], b[i], acc); o[i] = g * a[i]; }
      st8<F32>(dy, row * d + c, o);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (lane == 0) red[k & 63][w] = acc;
  }
  for (int s = 0; s < n_shared; s++) {
    const long row = shared_base + (long)s * shared_stride + t;
    for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
      float a[8];
      ld8<F32>(dout, drow + c, a);
      st8<F32>(dy, row * d + c, a);
    }
  }
  __syncthreads();
  if (threadIdx.x < K) {
    const int k = threadIdx.x;
    dg[(size_t)t * K + k] = ((red[k][0] + red[k][1]) + red[k][2]) + red[k][3];
  }
}

// Per token: dz_{t,k} = (dg_k - sum_j g_j dg_j) / sum_j s_j * s_k (1 - s_k), in fp64
__global__ void dz_kernel(const float* __restrict__ scores, const int32_t* __restrict__ idx,
                          const float* __restrict__ dg, int T, int N, int K, float* __restrict__ dz) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  double S = 0.0;
  for (int k = 0; k < K; k++) S += (double)scores[(size_t)t * N + idx[(size_t)t * K + k]];
  double gdg = 0.0;
  for (int k = 0; k < K; k++) {
    const double s = scores[(size_t)t * N + idx[(size_t)t * K + k]];
    gdg += (S > 0.0 ? s / S : 1.0 / K) * (double)dg[(size_t)t * K + k];
  }
  for (int k = 0; k < K; k++) {
    const double s = scores[(size_t)t * N + idx[(size_t)t * K + k]];
    const double ds = S > 0.0 ? ((double)dg[(size_t)t * K + k] - gdg) / S : 0.0;
    dz[(size_t)t * K + k] = (float)(ds * s * (1.0 - s));
  }
}

// One workgroup per token: du_t = dout_t + sum_s dX_s,t + sum_k dX_{t,k} + sum_k dz_{t,k} e_{idx_k}
template <bool E_BF16, bool F32>
__global__ __launch_bounds__(256) void du_kernel(const void* __restrict__ dout, const void* __restrict__ dx,
                                                 const int32_t* __restrict__ slot_row, const int32_t* __restrict__ idx,
                                                 const float* __restrict__ dz, const void* __restrict__ E, int d, int K,
                                                 int n_shared, long shared_base, long shared_stride,
                                                 float* __restrict__ du) {
  const int t = blockIdx.x;
  for (int c = threadIdx.x * 8; c < d; c += 256 * 8) {
    float acc[8], v[8];
    ld8<F32>(dout, (size_t)t * d + c, acc);
    for (int s = 0; s < n_shared; s++) {
      ld8<F32>(dx, (shared_base + (long)s * shared_stride + t) * d + c, v);
#pragma unroll
      for (int i = 0; i < 8; i++) acc[i] += v[i];
    }
    for (int k = 0; k < K; k++) {
      ld8<F32>(dx, (size_t)slot_row[(size_t)t * K + k] * d + c, v);
#pragma unroll
      for (int i = 0; i < 8; i++) acc[i] += v[i];
    }
    for (int k = 0; k < K; k++) {
      const float z = dz[(size_t)t * K + k];
      const size_t er = (size_t)idx[(size_t)t * K + k] * d + c;
      if (E_BF16) {
        load_bf16x8((const uint16_t*)E + er, v);
      } else {
#pragma unroll
        for (int i = 0; i < 8; i++) v[i] = ((const float*)E)[er + i];
      }
#pragma unroll
      for (int i = 0; i < 8; i++) acc[i] = fmaf(z, v[i], acc[i]);
    }
    float* o = du + (size_t)t * d + c;
    *(f32x4*)o = f32x4{acc[0], acc[1], acc[2], acc[3]};
    *(f32x4*)(o + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
  }
}

// grid (N_r, ceil(d/2048)): dE_i = sum over expert i's rows (ascending token)
// of dz_{t,k} u_t, fp32; k is where i sits in the token's selection.
template <bool F32>
__global__ __launch_bounds__(256) void de_kernel(const void* __restrict__ u, const int32_t* __restrict__ offsets,
                                                 const int32_t* __restrict__ row_token, const int32_t* __restrict__ idx,
                                                 const float* __restrict__ dz, int d, int K, float* __restrict__ dE) {
  const int i = blockIdx.x;
  const int c = (blockIdx.y * 256 + threadIdx.x) * 8;
  if (c >= d) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int r = offsets[i]; r < offsets[i + 1]; r++) {
    const int t = row_token[r];
    int k = 0;
    while (k < K - 1 && idx[(size_t)t * K + k] != i) k++;
    const float z = dz[(size_t)t * K + k];
    float v[8];
    ld8<F32>(u, (size_t)t * d + c, v);
#pragma unroll
    for (int j = 0; j < 8; j++) acc[j] = fmaf(z, v[j], acc[j]);
  }
  float* o = dE + (size_t)i * d + c;
  *(f32x4*)o = f32x4{acc[0], acc[1], acc[2], acc[3]};
  *(f32x4*)(o + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
}

// ---------------------------------------------------------------- weight gradients
// C_e[m][n] = sum over segment e's rows r of P[r][m] * Q[q(r)][n]  (fp32 out)
// P [R][M] bf16 (the permuted rows), Q rows bf16 (gathered through q_row when
// not null). One workgroup (4 waves, 2x2 of 64x64) per 128x128 block of C;
// the segment's rows go through LDS in chunks of 64. The MFMA operands need 8
// consecutive rows per lane, the rows in memory hold consecutive columns, so
// each thread loads an 8x8 (rows x columns) micro-tile of P or Q, transposes
// it in registers and writes 8 columns x 16 bytes to LDS. The next chunk is
// loaded while the current one is multiplied. Every block of C is one
// workgroup's full sum: no atomics, a fixed order.
constexpr int WG_T = 128;          // block edge
constexpr int WG_R = 64;           // rows per chunk (four MFMA k-steps)
constexpr int WG_PITCH = 72;       // bf16 per LDS row (64 used + 8 pad: conflict-free operand reads)

// columns j of 8 rows (one i32x4 of 8 bf16 per row) -> 8 bf16 of column j, rows in order
__device__ __forceinline__ i32x4 column_of(const i32x4* v, int j) {
  i32x4 o;
#pragma unroll
  for (int q = 0; q < 4; q++) {
    const uint32_t x = (uint32_t)v[2 * q][j >> 1], y = (uint32_t)v[2 * q + 1][j >> 1];
    o[q] = (int)((j & 1) ? ((x >> 16) | (y & 0xFFFF0000u)) : ((x & 0xFFFFu) | (y << 16)));
  }
  return o;
}

__global__ __launch_bounds__(256) void wgrad_kernel(WgradArgs a) {
  __shared__ __align__(16) uint16_t lds[2][2][WG_T][WG_PITCH];     // [operand][buffer][column][row]
  // Blocks go in super-tiles of 8x8 blocks of one segment; super-tile k runs on
  // XCD k % 8 (workgroup i runs on XCD i % 8) as 64 consecutive workgroups
  // there, which then share 8 column slices of P and 8 of Q in that XCD's L2.
  // Dealing super-tiles round-robin keeps segments of very different row
  // counts spread over all XCDs.
  const int nb = a.Nn / WG_T, mb = a.M / WG_T;
  const int snb = (nb + 7) / 8, smb = (mb + 7) / 8;
  const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
  const int st = xcd + 8 * (j >> 6), w = j & 63;
  const int seg = st / (smb * snb);
  if (seg >= a.n_seg) return;
  const int srem = st - seg * smb * snb;
  const int mblk = (srem / snb) * 8 + (w >> 3), nblk = (srem % snb) * 8 + (w & 7);
  if (mblk >= mb || nblk >= nb) return;
  const int m0 = mblk * WG_T, n0 = nblk * WG_T;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int rb = a.offsets[seg], re = a.offsets[seg + 1];
  float* out = seg < a.n_first ? a.out0 + (size_t)seg * a.ostride0 : a.out1 + (size_t)(seg - a.n_first) * a.ostride1;
  const int nchunk = (re - rb + WG_R - 1) / WG_R;

  // loader: threads 0..127 take P, 128..255 Q; micro-tile (8 rows at 8*rt, 8 columns at 8*ct)
  const int op = tid >> 7, ct = tid & 15, rt = (tid >> 4) & 7;
  const int ncols = op ? a.Nn : a.M;
  const int c0 = (op ? n0 : m0) + 8 * ct;
  const __amdgpu_buffer_rsrc_t src = op ? make_rsrc(a.Q, (long)a.q_rows * a.Nn * 2)
                                        : make_rsrc(a.P, (long)re * a.M * 2);
  i32x4 v[8];
  // source rows of a chunk, fetched one chunk ahead of their use (the Q rows
  // may be gathered through q_row)
  int srow[8];
  auto rows_of = [&](int r0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const int r = r0 + 8 * rt + i;
      srow[i] = r < re ? (op && a.q_row ? a.q_row[r] : r) : -1;
    }
  };
  auto gload = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const int off = srow[i] >= 0 ? (int)(((long)srow[i] * ncols + c0) * 2) : kOutOfRange;
      v[i] = __builtin_amdgcn_raw_buffer_load_b128(src, off, 0, 0);
    }
  };
  auto sstore = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < 8; j++) *(i32x4*)&lds[op][buf][8 * ct + j][8 * rt] = column_of(v, j);
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;
  const int l32 = lane & 31, kh = lane >> 5;
  if (nchunk > 0) {
    rows_of(rb);
    gload();
    rows_of(rb + WG_R);
    sstore(0);
    __syncthreads();
    for (int c = 0; c < nchunk; c++) {
      const int buf = c & 1;
      if (c + 1 < nchunk) {
        gload();
        rows_of(rb + (c + 2) * WG_R);
      }
#pragma unroll
      for (int ks = 0; ks < WG_R / 16; ks++) {
        bf16x8 af[2], bf[2];
#pragma unroll
        for (int i = 0; i < 2; i++) af[i] = *(const bf16x8*)&lds[0][buf][wm * 64 + i * 32 + l32][ks * 16 + kh * 8];
#pragma unroll
        for (int j = 0; j < 2; j++) bf[j] = *(const bf16x8*)&lds[1][buf][wn * 64 + j * 32 + l32][ks * 16 + kh * 8];
#pragma unroll
        for (int i = 0; i < 2; i++)
#pragma unroll
          for (int j = 0; j < 2; j++)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
      }
      if (c + 1 < nchunk) sstore(buf ^ 1);
      __syncthreads();
    }
  }
  // D element (8*(r>>2) + 4*(lane>>5) + (r&3), lane&31)
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * kh + (r & 3);
        const int n = n0 + wn * 64 + j * 32 + l32;
        out[(size_t)m * a.Nn + n] = acc[i][j][r];
      }
}

// ---------------------------------------------------------------- weight gradients, large shapes
// When M and Nn are multiples of 256 the products run as grouped GEMMs whose
// contraction runs along memory: P and Q are first transposed, segment by
// segment, into PT [M][pitch] and QT [Nn][pitch] with each segment's rows
// padded with zeros to a multiple of 64 (kofs[e] = where segment e starts),
// then C_e = PT_e QT_e^T with the forward GEMM's operand path: 256x256 tiles,
// 8 waves, LDS-DMA ring of four K=32 stages. The kernel is persistent (256
// workgroups, one per CU), so one tile's fp32 stores drain while the next
// tile's loads and MFMAs run.
constexpr int WT_PAD = 64;

// kofs[e] = sum over e' < e of roundup(n_e', pad); kofs[n_seg] = padded total
__global__ __launch_bounds__(64) void wg_kofs_kernel(const int32_t* __restrict__ offsets, int n_seg, int pad,
                                                     int32_t* __restrict__ kofs) {
  __shared__ int32_t so[512];
  for (int i = threadIdx.x; i <= n_seg; i += 64) so[i] = offsets[i];
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int e = 0; e < n_seg; e++) {
      kofs[e] = acc;
      acc += (so[e + 1] - so[e] + pad - 1) / pad * pad;
    }
    kofs[n_seg] = acc;
  }
}

// dst[c][kofs[e] + j] = src[row(offsets[e] + j)][c] for j < n_e, 0 for the padding;
// row(r) = q_row ? q_row[r] : r. grid (cols / 256, upper bound on padded positions / 64),
// 256 threads; thread (rt, ct) moves the 8x8 micro-tile of positions p0 + 8 rt .. and
// columns c0 + 8 ct .., transposed in registers.
__global__ __launch_bounds__(256) void seg_transpose_kernel(const uint16_t* __restrict__ src,
                                                            const int32_t* __restrict__ q_row,
                                                            const int32_t* __restrict__ offsets,
                                                            const int32_t* __restrict__ kofs, int n_seg, int cols,
                                                            long pitch, uint16_t* __restrict__ dst) {
  const int p0 = blockIdx.y * WT_PAD;
  if (p0 >= kofs[n_seg]) return;
  // the segment holding p0: the last e with kofs[e] <= p0 (empty segments before it share its kofs)
  int lo = 0, hi = n_seg - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (kofs[mid] <= p0) lo = mid; else hi = mid - 1;
  }
  const int j0 = p0 - kofs[lo], rb = offsets[lo], n = offsets[lo + 1] - rb;
  const int rt = threadIdx.x & 7, ct = threadIdx.x >> 3;
  const int c0 = blockIdx.x * 256 + ct * 8;
  i32x4 v[8];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const int j = j0 + 8 * rt + i;
    if (j < n) {
      const int r = rb + j;
      const long sr = q_row ? q_row[r] : r;
      v[i] = *(const i32x4*)(src + sr * cols + c0);
    } else {
      v[i] = i32x4{0, 0, 0, 0};
    }
  }
#pragma unroll
  for (int jj = 0; jj < 8; jj++) *(i32x4*)(dst + (size_t)(c0 + jj) * pitch + p0 + 8 * rt) = column_of(v, jj);
}

struct WgDma {
  static constexpr int THREADS = 512, BM = 256, BN = 256, RB = 64, BK = 32, CPR = 4, RPB = 16, STAGES = 4;
  static constexpr int A_BYTES = BM * RB, STAGE = (BM + BN) * RB, BYTES = STAGES * STAGE;
  static constexpr int PER_OP = BM / RPB / 8;         // 1 KB blocks of each operand per wave per stage
  static constexpr int NPARTS = 2 * PER_OP;
  static constexpr int GRID = 256;                    // 32 workgroups per XCD
  static constexpr int SUPER = GRID / 8;              // tiles per super-tile
  static_assert(BYTES <= 160 * 1024, "LDS budget");
};

struct WgradDmaArgs {
  const uint16_t* PT; const uint16_t* QT; long pitch; const int32_t* kofs;
  int n_seg, M, Nn, sm, sn;                           // super-tile of sm x sn tiles (sm * sn = 32)
  float* out0; float* out1; long ostride0, ostride1; int n_first;
};

__global__ __launch_bounds__(512, 1) void wgrad_dma_kernel(WgradDmaArgs a) {
  using C = WgDma;
  extern __shared__ __align__(16) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  // Workgroup i runs on XCD i % 8. Super-tile st (sm x sn tiles of one segment) goes to
  // XCD st % 8, whose 32 workgroups take one tile each, so the tiles running together on an
  // XCD share their operand rows in its L2; super-tiles are dealt round-robin so segments of
  // very different lengths spread over all XCDs.
  const int xcd = blockIdx.x & 7, q = blockIdx.x >> 3;
  const int MT = a.M / C::BM, NT = a.Nn / C::BN;
  const int smt = (MT + a.sm - 1) / a.sm, snt = (NT + a.sn - 1) / a.sn;
  const int per_seg = smt * snt, n_super = a.n_seg * per_seg;
  const uint32_t lds0 = lds_addr(lds);
  const int brow = lane / C::CPR;
  const int bchunk = (lane % C::CPR) ^ ((brow >> 2) & 3);
  const int l32 = lane & 31, khalf = lane >> 5;
  const int sw = (l32 >> 2) & 3;
  int roff[2];
#pragma unroll
  for (int ks = 0; ks < 2; ks++) roff[ks] = l32 * C::RB + (((2 * ks + khalf) ^ sw) << 4);
  const i32x4 pr = rsrc_words(a.PT, (long)a.M * a.pitch * 2);
  const i32x4 qr = rsrc_words(a.QT, (long)a.Nn * a.pitch * 2);

  for (int sidx = 0;; sidx++) {
    const int st = xcd + 8 * sidx;
    if (st >= n_super) break;
    const int seg = st / per_seg, srem = st - seg * per_seg;
    const int mt = (srem / snt) * a.sm + q / a.sn, nt = (srem % snt) * a.sn + q % a.sn;
    if (mt >= MT || nt >= NT) continue;
    const int k0 = a.kofs[seg];
    const int nk = (a.kofs[seg + 1] - k0) / C::BK;
    int aoff[C::PER_OP], boff[C::PER_OP];
#pragma unroll
    for (int i = 0; i < C::PER_OP; i++) {
      const int r = (wave + 8 * i) * C::RPB + brow;
      aoff[i] = (int)(((long)(mt * C::BM + r) * a.pitch + k0 + bchunk * 8) * 2);
      boff[i] = (int)(((long)(nt * C::BN + r) * a.pitch + k0 + bchunk * 8) * 2);
    }
    auto issue_part = [&](auto p_tag, int kt, int buf) __attribute__((always_inline)) {
      constexpr int P = decltype(p_tag)::value;
      const uint32_t sbase = lds0 + buf * C::STAGE;
      if constexpr (P < C::PER_OP)
        dma_b128(pr, aoff[P], kt * C::RB, sbase + (wave + 8 * P) * 1024);
      else
        dma_b128(qr, boff[P - C::PER_OP], kt * C::RB, sbase + C::A_BYTES + (wave + 8 * (P - C::PER_OP)) * 1024);
    };
    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 2; j++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;
    __syncthreads();   // every wave is done reading the previous tile's stages
    if (nk > 0) {
      constexpr int S = C::STAGES;
#pragma unroll
      for (int p = 0; p < S - 1; p++)
        static_for<C::NPARTS>([&](auto pp) __attribute__((always_inline)) { issue_part(pp, min(p, nk - 1), p); });
      for (int kt = 0; kt < nk; kt++) {
        wait_vmcnt<(S - 2) * C::NPARTS>();
        __syncthreads();
        const int buf = kt % S, kti = min(kt + S - 1, nk - 1), bufi = (kt + S - 1) % S;
        const uint8_t* A = lds + buf * C::STAGE;
        const uint8_t* B = A + C::A_BYTES;
        bf16x8 af[2][4], bf[2][2];
#pragma unroll
        for (int ks = 0; ks < 2; ks++) {
#pragma unroll
          for (int i = 0; i < 4; i++) af[ks][i] = *(const bf16x8*)(A + (2 * i + wm) * 32 * C::RB + roff[ks]);
#pragma unroll
          for (int j = 0; j < 2; j++) bf[ks][j] = *(const bf16x8*)(B + (wn * 64 + j * 32) * C::RB + roff[ks]);
        }
        // 16 MFMAs in four groups, one refill load in front of each group
        static_for<4>([&](auto g_tag) __attribute__((always_inline)) {
          constexpr int g = decltype(g_tag)::value, ks = g >> 1, i0 = (g & 1) * 2;
          issue_part(std::integral_constant<int, g>{}, kti, bufi);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int i = i0; i < i0 + 2; i++)
#pragma unroll
            for (int j = 0; j < 2; j++)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks][i], bf[ks][j], acc[i][j], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        });
      }
      wait_vmcnt<0>();   // no LDS write may land after the tile's reads
    }
    float* out = seg < a.n_first ? a.out0 + (size_t)seg * a.ostride0
                                 : a.out1 + (size_t)(seg - a.n_first) * a.ostride1;
    // D element (8*(r>>2) + 4*(lane>>5) + (r&3), lane&31) of each 32x32 block
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 2; j++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int m = mt * C::BM + (2 * i + wm) * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
          const int n = nt * C::BN + wn * 64 + j * 32 + l32;
          __builtin_nontemporal_store(acc[i][j][r], out + (size_t)m * a.Nn + n);
        }
  }
}

// ---------------------------------------------------------------- FP8 weight gradients
// C_e = PT_e QT_e^T over segment e's rows with E4M3 operands (the pages' Wgrad in
// FP8): PT [M][pitch] and QT [Nn][pitch] hold each segment's transposed rows
// padded with zeros to a multiple of 128 (kofs, from wg_kofs_kernel with pad
// 128), quantised in 1x128 tiles along pitch, i.e. 128-row tiles of the
// original rows aligned at the segment's first row; their fp32 scales are stored
// transposed, SPT [pitch/128][M] and SQT [pitch/128][Nn], so a stage's 256
// scales are one contiguous kilobyte. 256x256 tiles, 8 waves (each 128x64 as
// 4x2 blocks of 32x32), K = 128 per stage (one scale tile) in a two-stage ring
// of LDS-DMA loads; per block and stage two v_mfma_scale_f32_32x32x64_f8f6f4
// make a fresh fp32 partial p, folded as acc += p * s_P[row] * s_Q[col].
// Persistent over super-tiles as wgrad_dma_kernel; no atomics, deterministic.
struct WgF8 {
  static constexpr int THREADS = 512, BM = 256, BN = 256, BK = 128;
  static constexpr int A_BYTES = BM * BK, B_BYTES = BN * BK, S_BYTES = 1024;
  static constexpr int STAGE = A_BYTES + B_BYTES + 2 * S_BYTES, BYTES = 2 * STAGE;
  static constexpr int PER_OP = BM / 8 / 8;           // 1 KB blocks of 8 rows per operand per wave
  static constexpr int GRID = 256;
  static constexpr int SUPER = GRID / 8;
  static_assert(BYTES <= 160 * 1024, "LDS budget");
};

struct WgradF8Args {
  const uint8_t* PT; const uint8_t* QT; const float* SPT; const float* SQT; long pitch; const int32_t* kofs;
  int n_seg, M, Nn, sm, sn;
  float* out0; float* out1; long ostride0, ostride1; int n_first;
};

__global__ __launch_bounds__(512, 1) void wgrad_f8_kernel(WgradF8Args a) {
  using C = WgF8;
  extern __shared__ __align__(16) uint8_t lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  const int xcd = blockIdx.x & 7, q = blockIdx.x >> 3;
  const int MT = a.M / C::BM, NT = a.Nn / C::BN;
  const int smt = (MT + a.sm - 1) / a.sm, snt = (NT + a.sn - 1) / a.sn;
  const int per_seg = smt * snt, n_super = a.n_seg * per_seg;
  const uint32_t lds0 = lds_addr(lds);
  // block b of a stage holds rows 8b..8b+7; lane l writes row l >> 3, slot l & 7 and fetches
  // chunk slot ^ ((row >> 1) & 7): blocks b = wave + 8i share b's parity with the wave
  const int brow = lane >> 3;
  const int bchunk = (lane & 7) ^ ((((wave & 1) << 2) + (lane >> 4)) & 7);
  const int l32 = lane & 31, khalf = lane >> 5;
  const int sw = (l32 >> 1) & 7;
  int roff[2][2];
#pragma unroll
  for (int h = 0; h < 2; h++)
#pragma unroll
    for (int c = 0; c < 2; c++) roff[h][c] = l32 * 128 + (((h * 4 + khalf * 2 + c) ^ sw) << 4);
  const long kb_total = a.pitch / C::BK;
  const i32x4 pr = rsrc_words(a.PT, (long)a.M * a.pitch);
  const i32x4 qr = rsrc_words(a.QT, (long)a.Nn * a.pitch);
  const i32x4 spr = rsrc_words(a.SPT, kb_total * a.M * 4);
  const i32x4 sqr = rsrc_words(a.SQT, kb_total * a.Nn * 4);

  for (int sidx = 0;; sidx++) {
    const int st = xcd + 8 * sidx;
    if (st >= n_super) break;
    const int seg = st / per_seg, srem = st - seg * per_seg;
    const int mt = (srem / snt) * a.sm + q / a.sn, nt = (srem % snt) * a.sn + q % a.sn;
    if (mt >= MT || nt >= NT) continue;
    const int k0 = a.kofs[seg];
    const int nkb = (a.kofs[seg + 1] - k0) / C::BK;
    int aoff[C::PER_OP], boff[C::PER_OP];
#pragma unroll
    for (int i = 0; i < C::PER_OP; i++) {
      const int r = (wave + 8 * i) * 8 + brow;
      aoff[i] = (int)((long)(mt * C::BM + r) * a.pitch + k0 + bchunk * 16);
      boff[i] = (int)((long)(nt * C::BN + r) * a.pitch + k0 + bchunk * 16);
    }
    const int soff = (int)(((long)(k0 / C::BK) * (wave == 0 ? a.M : a.Nn) + (wave == 0 ? mt * C::BM : nt * C::BN)) * 4
                           + lane * 16);
    auto issue = [&](int kb, int buf) __attribute__((always_inline)) {
      const uint32_t sbase = lds0 + buf * C::STAGE;
#pragma unroll
      for (int i = 0; i < C::PER_OP; i++) dma_b128(pr, aoff[i], kb * C::BK, sbase + (wave + 8 * i) * 1024);
#pragma unroll
      for (int i = 0; i < C::PER_OP; i++)
        dma_b128(qr, boff[i], kb * C::BK, sbase + C::A_BYTES + (wave + 8 * i) * 1024);
      // the stage's 256 row scales of each operand: one kilobyte each
      if (wave == 0) dma_b128(spr, soff, kb * a.M * 4, sbase + C::A_BYTES + C::B_BYTES);
      if (wave == 1) dma_b128(sqr, soff, kb * a.Nn * 4, sbase + C::A_BYTES + C::B_BYTES + C::S_BYTES);
    };
    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 2; j++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;
    __syncthreads();   // every wave is done reading the previous tile's stages
    if (nkb > 0) {
      issue(0, 0);
      for (int kb = 0; kb < nkb; kb++) {
        wait_vmcnt<0>();
        __syncthreads();
        issue(min(kb + 1, nkb - 1), (kb + 1) & 1);
        const uint8_t* A = lds + (kb & 1) * C::STAGE;
        const uint8_t* B = A + C::A_BYTES;
        const float* SA = (const float*)(B + C::B_BYTES);
        const float* SB = SA + C::S_BYTES / 4;
        i32x8 bfr[2][2];
        float sb[2];
#pragma unroll
        for (int j = 0; j < 2; j++) {
          const int brow0 = wn * 64 + j * 32;
#pragma unroll
          for (int h = 0; h < 2; h++) {
            const i32x4 lo = *(const i32x4*)(B + brow0 * 128 + roff[h][0]);
            const i32x4 hi = *(const i32x4*)(B + brow0 * 128 + roff[h][1]);
            bfr[j][h] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          }
          sb[j] = SB[brow0 + l32];
        }
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int mrow = (2 * i + wm) * 32;
          i32x8 afr[2];
#pragma unroll
          for (int h = 0; h < 2; h++) {
            const i32x4 lo = *(const i32x4*)(A + mrow * 128 + roff[h][0]);
            const i32x4 hi = *(const i32x4*)(A + mrow * 128 + roff[h][1]);
            afr[h] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          }
          // this lane's 16 accumulator rows: 8*qq + 4*khalf + e
          f32x4 sa[4];
#pragma unroll
          for (int qq = 0; qq < 4; qq++) sa[qq] = *(const f32x4*)(SA + mrow + 8 * qq + 4 * khalf);
#pragma unroll
          for (int j = 0; j < 2; j++) {
            f32x16 p;
#pragma unroll
            for (int r = 0; r < 16; r++) p[r] = 0.f;
            // cbsz = blgp = 0: both operands E4M3; scale exponents 127 = 2^0
            p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(afr[0], bfr[j][0], p, 0, 0, 0, 127, 0, 127);
            p = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(afr[1], bfr[j][1], p, 0, 0, 0, 127, 0, 127);
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = fmaf(p[r], sa[r >> 2][r & 3] * sb[j], acc[i][j][r]);
          }
        }
      }
      wait_vmcnt<0>();   // no LDS write may land after the tile's reads
    }
    float* out = seg < a.n_first ? a.out0 + (size_t)seg * a.ostride0
                                 : a.out1 + (size_t)(seg - a.n_first) * a.ostride1;
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 2; j++)
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int m = mt * C::BM + (2 * i + wm) * 32 + 8 * (r >> 2) + 4 * khalf + (r & 3);
          const int n = nt * C::BN + wn * 64 + j * 32 + l32;
          __builtin_nontemporal_store(acc[i][j][r], out + (size_t)m * a.Nn + n);
        }
  }
}

long wgrad_pitch(long rows, int n_seg, int pad) { return (rows + (long)pad * n_seg + pad - 1) / pad * pad; }

static hipError_t launch_wgrad_dma(const WgradArgs& a, hipStream_t s) {
  hipError_t e;
  wg_kofs_kernel<<<1, 64, 0, s>>>(a.offsets, a.n_seg, WT_PAD, a.kofs);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const dim3 gp(a.M / 256, (unsigned)(a.pitch / WT_PAD)), gq(a.Nn / 256, (unsigned)(a.pitch / WT_PAD));
  seg_transpose_kernel<<<gp, 256, 0, s>>>(a.P, nullptr, a.offsets, a.kofs, a.n_seg, a.M, a.pitch, a.pt);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  seg_transpose_kernel<<<gq, 256, 0, s>>>(a.Q, a.q_row, a.offsets, a.kofs, a.n_seg, a.Nn, a.pitch, a.qt);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  WgradDmaArgs g;
  g.PT = a.pt; g.QT = a.qt; g.pitch = a.pitch; g.kofs = a.kofs;
  g.n_seg = a.n_seg; g.M = a.M; g.Nn = a.Nn;
  const int NT = a.Nn / 256;
  g.sn = NT % 8 == 0 ? 8 : NT % 4 == 0 ? 4 : NT >= 8 ? 8 : (NT >= 4 ? 4 : (NT >= 2 ? 2 : 1));
  g.sm = WgDma::SUPER / g.sn;
  g.out0 = a.out0; g.out1 = a.out1; g.ostride0 = a.ostride0; g.ostride1 = a.ostride1; g.n_first = a.n_first;
  auto k = wgrad_dma_kernel;
  if ((e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, WgDma::BYTES)) !=
      hipSuccess)
    return e;
  k<<<WgDma::GRID, WgDma::THREADS, WgDma::BYTES, s>>>(g);
  return hipGetLastError();
}

// fp32 layers (the small fp32 configuration): C_e[m][n] = sum over segment e's rows r of
// P[r][m] * Q[q(r)][n] with plain fp32 FMAs in row order, one thread per element of C.
// grid (ceil(Nn/64), ceil(M/4), n_seg), 256 threads: 4 rows of C x 64 columns.
__global__ __launch_bounds__(256) void wgrad_f32_kernel(const float* __restrict__ P, const float* __restrict__ Q,
                                                        const int32_t* __restrict__ q_row,
                                                        const int32_t* __restrict__ offsets, int M, int Nn,
                                                        float* __restrict__ out0, float* __restrict__ out1,
                                                        long ostride0, long ostride1, int n_first) {
  const int seg = blockIdx.z;
  const int m = blockIdx.y * 4 + (threadIdx.x >> 6), n = blockIdx.x * 64 + (threadIdx.x & 63);
  if (m >= M || n >= Nn) return;
  float acc = 0.f;
  for (int r = offsets[seg]; r < offsets[seg + 1]; r++) {
    const long qr = q_row ? q_row[r] : r;
    acc = fmaf(P[(size_t)r * M + m], Q[(size_t)qr * Nn + n], acc);
  }
  float* out = seg < n_first ? out0 + (size_t)seg * ostride0 : out1 + (size_t)(seg - n_first) * ostride1;
  out[(size_t)m * Nn + n] = acc;
}

// ---------------------------------------------------------------- transposes
// dst[b][c][r] = src[b][r][c] for [batch][rows][cols] of 1-, 2- or 4-byte elements, 64x64 tiles via LDS
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ src, T* __restrict__ dst,
                                                        int rows, int cols) {
  __shared__ T tile[64][65];
  const size_t base = (size_t)blockIdx.z * rows * cols;
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int r = i >> 6, c = i & 63;
    if (r0 + r < rows && c0 + c < cols) tile[r][c] = src[base + (size_t)(r0 + r) * cols + c0 + c];
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 64 * 64; i += 256) {
    const int c = i >> 6, r = i & 63;
    if (r0 + r < rows && c0 + c < cols) dst[base + (size_t)(c0 + c) * rows + r0 + r] = tile[r][c];
  }
}

// ---------------------------------------------------------------- launchers
static dim3 grid_1d(long n, int per_block) {
  return dim3((unsigned)std::min<long>(cdiv<long>(n, per_block), 8192));
}

hipError_t launch_swiglu_fwd(const void* ab, void* h, long rows, int I, int dtype, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (dtype == MOE_F32) swiglu_fwd_kernel<true><<<grid_1d(rows * (I / 8), 256), 256, 0, s>>>(ab, h, rows, I);
  else swiglu_fwd_kernel<false><<<grid_1d(rows * (I / 8), 256), 256, 0, s>>>(ab, h, rows, I);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const void* dh, const void* ab, void* dab, long rows, int I, int dtype, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (dtype == MOE_F32) swiglu_bwd_kernel<true><<<grid_1d(rows * (I / 8), 256), 256, 0, s>>>(dh, ab, dab, rows, I);
  else swiglu_bwd_kernel<false><<<grid_1d(rows * (I / 8), 256), 256, 0, s>>>(dh, ab, dab, rows, I);
  return hipGetLastError();
}

hipError_t launch_dgate_dy(const void* dout, const void* y, const int32_t* slot_row, const float* gate, int T, int d,
                           int K, int n_shared, long shared_base, long shared_stride, float* dg, void* dy, int dtype,
                           hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (dtype == MOE_F32)
    dgate_dy_kernel<true><<<T, 256, 0, s>>>(dout, y, slot_row, gate, d, K, n_shared, shared_base, shared_stride, dg, dy);
  else
    dgate_dy_kernel<false><<<T, 256, 0, s>>>(dout, y, slot_row, gate, d, K, n_shared, shared_base, shared_stride, dg,
                                             dy);
  return hipGetLastError();
}

hipError_t launch_router_bwd(const float* scores, const int32_t* idx, const float* dg, const void* dout,
                             const void* dx, const int32_t* slot_row, const void* E, int e_dtype, const void* u,
                             const int32_t* offsets, const int32_t* row_token, int T, int N, int d, int K,
                             int n_shared, long shared_base, long shared_stride, float* dz, float* du, float* dE,
                             int dtype, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  dz_kernel<<<cdiv(T, 256), 256, 0, s>>>(scores, idx, dg, T, N, K, dz);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool f32 = dtype == MOE_F32;
  if (e_dtype == MOE_BF16 && !f32)
    du_kernel<true, false><<<T, 256, 0, s>>>(dout, dx, slot_row, idx, dz, E, d, K, n_shared, shared_base,
                                             shared_stride, du);
  else if (e_dtype == MOE_BF16)
    du_kernel<true, true><<<T, 256, 0, s>>>(dout, dx, slot_row, idx, dz, E, d, K, n_shared, shared_base,
                                            shared_stride, du);
  else if (!f32)
    du_kernel<false, false><<<T, 256, 0, s>>>(dout, dx, slot_row, idx, dz, E, d, K, n_shared, shared_base,
                                              shared_stride, du);
  else
    du_kernel<false, true><<<T, 256, 0, s>>>(dout, dx, slot_row, idx, dz, E, d, K, n_shared, shared_base,
                                             shared_stride, du);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (f32) de_kernel<true><<<dim3(N, cdiv(d, 2048)), 256, 0, s>>>(u, offsets, row_token, idx, dz, d, K, dE);
  else de_kernel<false><<<dim3(N, cdiv(d, 2048)), 256, 0, s>>>(u, offsets, row_token, idx, dz, d, K, dE);
  return hipGetLastError();
}

hipError_t launch_wgrad_f32(const WgradArgs& a, const float* P, const float* Q, hipStream_t s) {
  if (a.n_seg <= 0) return hipSuccess;
  wgrad_f32_kernel<<<dim3(cdiv(a.Nn, 64), cdiv(a.M, 4), a.n_seg), 256, 0, s>>>(
      P, Q, a.q_row, a.offsets, a.M, a.Nn, a.out0, a.out1, a.ostride0, a.ostride1, a.n_first);
  return hipGetLastError();
}

hipError_t launch_wgrad(const WgradArgs& a, hipStream_t s) {
  if (a.n_seg <= 0) return hipSuccess;
  if (a.pt && a.qt && a.kofs && a.M % 256 == 0 && a.Nn % 256 == 0) return launch_wgrad_dma(a, s);
  const long supers = (long)a.n_seg * ((a.M / WG_T + 7) / 8) * ((a.Nn / WG_T + 7) / 8);
  const long blocks = (supers + 7) / 8 * 8 * 64;
  wgrad_kernel<<<dim3((unsigned)blocks), 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_wgrad_f8(const WgradArgs& a, const WgradF8Scratch& f, hipStream_t s) {
  if (a.M % 256 || a.Nn % 256 || !f.pt8 || !f.qt8 || !f.spt || !f.sqt) return hipErrorInvalidValue;
  hipError_t e;
  wg_kofs_kernel<<<1, 64, 0, s>>>(a.offsets, a.n_seg, 128, a.kofs);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // transposed bf16 copies (segments padded to 128 rows), then their 1x128 tiles in E4M3
  const dim3 gp(a.M / 256, (unsigned)(a.pitch / WT_PAD)), gq(a.Nn / 256, (unsigned)(a.pitch / WT_PAD));
  seg_transpose_kernel<<<gp, 256, 0, s>>>(a.P, nullptr, a.offsets, a.kofs, a.n_seg, a.M, a.pitch, a.pt);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  seg_transpose_kernel<<<gq, 256, 0, s>>>(a.Q, a.q_row, a.offsets, a.kofs, a.n_seg, a.Nn, a.pitch, a.qt);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if ((e = launch_quant_act_tscale(a.pt, a.M, (int)a.pitch, f.pt8, f.spt, s)) != hipSuccess) return e;
  if ((e = launch_quant_act_tscale(a.qt, a.Nn, (int)a.pitch, f.qt8, f.sqt, s)) != hipSuccess) return e;
  WgradF8Args g;
  g.PT = f.pt8; g.QT = f.qt8; g.SPT = f.spt; g.SQT = f.sqt; g.pitch = a.pitch; g.kofs = a.kofs;
  g.n_seg = a.n_seg; g.M = a.M; g.Nn = a.Nn;
  const int NT = a.Nn / 256;
  g.sn = NT % 8 == 0 ? 8 : NT % 4 == 0 ? 4 : NT >= 8 ? 8 : (NT >= 4 ? 4 : (NT >= 2 ? 2 : 1));
  g.sm = WgF8::SUPER / g.sn;
  g.out0 = a.out0; g.out1 = a.out1; g.ostride0 = a.ostride0; g.ostride1 = a.ostride1; g.n_first = a.n_first;
  auto k = wgrad_f8_kernel;
  if ((e = hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, WgF8::BYTES)) !=
      hipSuccess)
    return e;
  k<<<WgF8::GRID, WgF8::THREADS, WgF8::BYTES, s>>>(g);
  return hipGetLastError();
}

hipError_t launch_transpose(const void* src, void* dst, int batch, int rows, int cols, int dtype, hipStream_t s) {
  if (batch <= 0 || rows <= 0 || cols <= 0) return hipSuccess;
  const dim3 grid(cdiv(cols, 64), cdiv(rows, 64), batch);
  if (dtype == MOE_F32)
    transpose_kernel<float><<<grid, 256, 0, s>>>((const float*)src, (float*)dst, rows, cols);
  else if (dtype == MOE_FP8_E4M3)
    transpose_kernel<uint8_t><<<grid, 256, 0, s>>>((const uint8_t*)src, (uint8_t*)dst, rows, cols);
  else
    transpose_kernel<uint16_t><<<grid, 256, 0, s>>>((const uint16_t*)src, (uint16_t*)dst, rows, cols);
  return hipGetLastError();
}

}  // namespace moe
