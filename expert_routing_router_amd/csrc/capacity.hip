// Capacity limit with token dropping: the DeepSeek-V2-style baseline that the
// DeepSeek-V3 method does without (pwwt.cn note on the report, section 1.4).
// An expert chosen more than `cap` times keeps the `cap` selections with the
// largest affinity s_{i,t} (ties: lower token) and drops the rest; a dropped
// selection skips that expert's FFN and adds nothing to the token's output.
#include "common.h"
#include "moe_internal.h"

namespace moe {

__device__ __forceinline__ int block_sum_int(int v, int* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

// one workgroup (256 threads) per expert; rows [offsets[e], offsets[e+1]) of the
// no-drop layout are the expert's selections in token order
__global__ __launch_bounds__(256) void capacity_kernel(const int32_t* __restrict__ offsets,
                                                       const int32_t* __restrict__ row_token,
                                                       const int32_t* __restrict__ idx,
                                                       const float* __restrict__ scores, int N, int K, int cap,
                                                       int32_t* __restrict__ keep, int32_t* __restrict__ dropped) {
  __shared__ int red[4];
  const int e = blockIdx.x, tid = threadIdx.x;
  const int rb = offsets[e], re = offsets[e + 1];
  if (re - rb <= cap) return;
  auto key_of = [&](int r) __attribute__((always_inline)) {
    return ordered_f32(scores[(size_t)row_token[r] * N + e]);
  };
  auto count_ge = [&](uint32_t x, bool strict) __attribute__((always_inline)) {
    int c = 0;
    for (int r = rb + tid; r < re; r += 256) {
      const uint32_t k = key_of(r);
      c += strict ? (k > x) : (k >= x);
    }
    return block_sum_int(c, red);
  };
  // largest key value thr with at least cap selections at or above it
  uint32_t lo = 0u, hi = 0xFFFFFFFFu;
  while (lo < hi) {
    const uint32_t mid = lo + (uint32_t)((hi - lo + 1ull) / 2);
    if (count_ge(mid, false) >= cap) lo = mid; else hi = mid - 1;
  }
  const uint32_t thr = lo;
  const int need = cap - count_ge(thr, true);   // selections at exactly thr to keep, in token order
  int carry = 0, drops = 0;
  __shared__ int wtot[4];
  for (int base = rb; base < re; base += 256) {
    const int r = base + tid;
    const uint32_t k = r < re ? key_of(r) : 0u;
    const int eq = (r < re && k == thr) ? 1 : 0;
    // exclusive prefix of eq over the workgroup, in row order
    const int lane = tid & 63, w = tid >> 6;
    int incl = eq;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    __syncthreads();
    if (lane == 63) wtot[w] = incl;
    __syncthreads();
    int before = 0;
    for (int i = 0; i < w; i++) before += wtot[i];
    const int rank = carry + before + incl - eq;
    const bool drop = r < re && (k < thr || (eq && rank >= need));
    if (drop) {
      const int t = row_token[r];
      int kk = 0;
      while (kk < K - 1 && idx[(size_t)t * K + kk] != e) kk++;
      keep[(size_t)t * K + kk] = 0;
      drops++;
    }
    carry += wtot[0] + wtot[1] + wtot[2] + wtot[3];
  }
  const int total = block_sum_int(drops, red);
  if (tid == 0 && dropped) atomicAdd(dropped, total);
}

hipError_t launch_capacity(const int32_t* offsets, const int32_t* row_token, const int32_t* idx,
                           const float* scores, int T, int N, int K, int cap, int32_t* keep, int32_t* dropped,
                           hipStream_t s) {
  hipError_t e = launch_fill_i32(keep, 1, (long)T * K, s);
  if (e != hipSuccess) return e;
  if (dropped && (e = launch_fill_i32(dropped, 0, 1, s)) != hipSuccess) return e;
  capacity_kernel<<<N, 256, 0, s>>>(offsets, row_token, idx, scores, N, K, cap, keep, dropped);
  return hipGetLastError();
}

}  // namespace moe
