// Dispatch layout on one GPU: per-expert loads, exclusive scan, and a stable
// token permutation with no capacity limit.
//
// The pwwt.cn note (section 4) describes dispatch as sending each token to the
// devices that hold its experts and combine as the gated sum on the home
// device; on one GPU the same step is a permutation that groups the T*K
// (token, expert) rows by expert. No row is ever dropped (note section 1.4).
//
// Construction (deterministic, no float atomics, no sort):
//   1. bitmap[w][e]: bit j set when token 64*w + j picked expert e
//      (one wave per 64 tokens, OR-ed in LDS, written coalesced over e);
//   2. per expert, the running popcount over words gives wprefix[w][e] and
//      the load c_e; an exclusive scan over experts gives offsets;
//   3. row of (t, k) = offsets[e] + wprefix[t/64][e] + popcount of the bits of
//      tokens below t in t's word -- rows of an expert are in token order.
#include "common.h"
#include "moe_internal.h"

namespace moe {

constexpr int PM_NMAX = 256;

__global__ __launch_bounds__(256) void bitmap_kernel(const int32_t* __restrict__ idx, int T, int K,
                                                     int N, const int32_t* __restrict__ keep,
                                                     uint64_t* __restrict__ bitmap) {
  __shared__ uint64_t words[4][PM_NMAX];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int e = lane; e < N; e += 64) words[wave][e] = 0ull;
  __syncthreads();
  const int w = blockIdx.x * 4 + wave;
  const int t = w * 64 + lane;
  if (t < T)
    for (int k = 0; k < K; k++) {
      const int e = idx[(size_t)t * K + k];
      // an expert id outside [0, N) gets no row (as a dropped selection)
      if ((unsigned)e < (unsigned)N && (!keep || keep[(size_t)t * K + k]))
        atomicOr((unsigned long long*)&words[wave][e], 1ull << lane);
    }
  __syncthreads();
  const int W = cdiv(T, 64);
  if (w < W)
    for (int e = lane; e < N; e += 64) bitmap[(size_t)w * N + e] = words[wave][e];
}

// Inclusive prefix sum over one workgroup of 256 threads (4 waves).
__device__ __forceinline__ int block_inclusive_scan(int v, int* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; w++) base += wsum[w];
  __syncthreads();
  return v + base;
}

// One workgroup: per-expert word prefix and load, then offsets over the
// segments (routed experts, then identity segments of T rows for the shared
// experts) and the prefix of m-tiles of `bm` rows per segment.
__global__ __launch_bounds__(256) void scan_kernel(const uint64_t* __restrict__ bitmap, int T, int K,
                                                   int N, int n_extra, int32_t* __restrict__ wprefix,
                                                   int32_t* __restrict__ offsets,
                                                   int32_t* __restrict__ counts_out,
                                                   int32_t* __restrict__ mtile_prefix, int bm) {
  __shared__ int wsum[4];
  const int tid = threadIdx.x;
  const int W = cdiv(T, 64);
  const int n_seg = N + n_extra;
  int c = 0;
  if (tid < N) {
    int w = 0;
    for (; w + 8 <= W; w += 8) {          // eight independent loads in flight
      uint64_t v[8];
#pragma unroll
      for (int i = 0; i < 8; i++) v[i] = bitmap[(size_t)(w + i) * N + tid];
#pragma unroll
      for (int i = 0; i < 8; i++) {
        wprefix[(size_t)(w + i) * N + tid] = c;
        c += __popcll(v[i]);
      }
    }
    for (; w < W; w++) {
      wprefix[(size_t)w * N + tid] = c;
      c += __popcll(bitmap[(size_t)w * N + tid]);
    }
    if (counts_out) counts_out[tid] = c;
  }
  // each thread owns segments 2*tid and 2*tid+1 (n_seg <= 320 < 512)
  int n[2], m[2];
#pragma unroll
  for (int i = 0; i < 2; i++) {
    const int e = 2 * tid + i;
    n[i] = e < N ? 0 : (e < n_seg ? T : 0);
  }
  __shared__ int sc[512];
  if (tid < N) sc[tid] = c;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; i++) {
    const int e = 2 * tid + i;
    if (e < N) n[i] = sc[e];
    m[i] = bm > 0 ? cdiv(n[i], bm) : 0;
  }
  const int n_inc = block_inclusive_scan(n[0] + n[1], wsum);
  const int m_inc = block_inclusive_scan(m[0] + m[1], wsum);
  const int n_exc = n_inc - n[0] - n[1], m_exc = m_inc - m[0] - m[1];
#pragma unroll
  for (int i = 0; i < 2; i++) {
    const int e = 2 * tid + i;
    const int no = n_exc + (i ? n[0] : 0), mo = m_exc + (i ? m[0] : 0);
    if (e <= n_seg) {
      offsets[e] = no;
      if (mtile_prefix) mtile_prefix[e] = mo;
    }
  }
}

__global__ __launch_bounds__(256) void scatter_kernel(const int32_t* __restrict__ idx, int T, int K,
                                                      int N, int n_extra,
                                                      const uint64_t* __restrict__ bitmap,
                                                      const int32_t* __restrict__ wprefix,
                                                      const int32_t* __restrict__ offsets,
                                                      const int32_t* __restrict__ keep,
                                                      int32_t* __restrict__ row_token,
                                                      int32_t* __restrict__ slot_row) {
  const long TK = (long)T * K;
  const long total = TK + (long)n_extra * T;
  for (long p = (long)blockIdx.x * blockDim.x + threadIdx.x; p < total; p += (long)gridDim.x * blockDim.x) {
    if (p < TK && ((keep && !keep[p]) || (unsigned)idx[p] >= (unsigned)N)) {
      slot_row[p] = -1;                     // dropped selection (or an id outside [0, N)): no row
    } else if (p < TK) {
      const int t = (int)(p / K);
      const int e = idx[p];
      const int w = t >> 6, bit = t & 63;
      const uint64_t word = bitmap[(size_t)w * N + e];
      const int below = __popcll(word & ((1ull << bit) - 1ull));
      const int r = offsets[e] + wprefix[(size_t)w * N + e] + below;
      row_token[r] = t;
      slot_row[p] = r;
    } else {
      row_token[p] = (int)((p - TK) % T);   // shared experts: every token, in order
    }
  }
}

__global__ void mtile_prefix_kernel(const int32_t* __restrict__ offsets, int n_seg, int bm,
                                    int32_t* __restrict__ out) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    int acc = 0;
    for (int e = 0; e < n_seg; e++) {
      out[e] = acc;
      acc += cdiv(offsets[e + 1] - offsets[e], bm);
    }
    out[n_seg] = acc;
  }
}

// rows r < *n_valid only (the rows the dispatch wrote), and only source rows inside src
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint8_t* __restrict__ src, long src_rows,
                                                          const int32_t* __restrict__ row_token,
                                                          const int32_t* __restrict__ n_valid,
                                                          uint8_t* __restrict__ dst, int row_bytes) {
  const long r = blockIdx.x;
  if (r >= *n_valid) return;
  const int t = row_token[r];
  if ((unsigned long)t >= (unsigned long)src_rows) return;
  const uint8_t* s = src + (size_t)t * row_bytes;
  uint8_t* d = dst + (size_t)r * row_bytes;
  for (int c = threadIdx.x * 16; c < row_bytes; c += blockDim.x * 16)
    *(i32x4*)(d + c) = *(const i32x4*)(s + c);
}

hipError_t launch_permute(const PermuteArgs& a, hipStream_t s) {
  const int W = cdiv(a.T, 64);
  bitmap_kernel<<<cdiv(W, 4), 256, 0, s>>>(a.idx, a.T, a.K, a.n_routed, a.keep, a.bitmap);
  scan_kernel<<<1, 256, 0, s>>>(a.bitmap, a.T, a.K, a.n_routed, a.n_extra_seg, a.wprefix, a.offsets,
                                a.counts_out, a.mtile_prefix, a.bm);
  const long total = (long)a.T * a.K + (long)a.n_extra_seg * a.T;
  const int blocks = (int)std::min<long>(cdiv<long>(total, 256), 2048);
  scatter_kernel<<<blocks, 256, 0, s>>>(a.idx, a.T, a.K, a.n_routed, a.n_extra_seg, a.bitmap,
                                        a.wprefix, a.offsets, a.keep, a.row_token, a.slot_row);
  return hipGetLastError();
}

hipError_t launch_mtile_prefix(const int32_t* offsets, int n_seg, int bm, int32_t* out, hipStream_t s) {
  mtile_prefix_kernel<<<1, 64, 0, s>>>(offsets, n_seg, bm, out);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* src, long src_rows, const int32_t* row_token, const int32_t* n_valid,
                              void* dst, long rows, int row_bytes, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  gather_rows_kernel<<<(unsigned)rows, 256, 0, s>>>((const uint8_t*)src, src_rows, row_token, n_valid,
                                                    (uint8_t*)dst, row_bytes);
  return hipGetLastError();
}

}  // namespace moe
