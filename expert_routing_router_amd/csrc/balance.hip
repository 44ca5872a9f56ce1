// Complementary sequence-wise balance loss: its forward value, from the
// router's affinities and selections.
//
// pwwt.cn note on the DeepSeek-V3 Technical Report, section 1.2: per
// sequence, alpha * sum_i f_i * P_i with f_i the expert's actual selection
// frequency in the sequence and P_i the probability that the router prefers
// it; alpha = 0.0001 (also the xyznot.com guides, section 2). The page's
// formula is missing; the normalisations taken are
//   f_i = (# of the sequence's K*T_s selections that are expert i) / (K*T_s)
//   P_i = mean over the sequence's tokens of s_{i,t} / sum_j s_{j,t}
//         (1/N_r for a token whose affinities sum to 0).
// All sums are fp64 in a fixed order, so the result does not depend on
// scheduling.
#include "common.h"
#include "moe_internal.h"

namespace moe {

constexpr int BL_EXPERTS = 64;     // experts per workgroup of the statistics kernel

// one wave per token: fp64 sum of its N affinities (lane sums, then a butterfly)
__global__ __launch_bounds__(256) void row_sum_kernel(const float* __restrict__ s, double* __restrict__ rowsum,
                                                      int T, int N) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = s + (size_t)t * N;
  double acc = 0.0;
  for (int e = lane; e < N; e += 64) acc += (double)row[e];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, 64);
  if (lane == 0) rowsum[t] = acc;
}

// grid (n_seq, ceil(N/64)), 256 threads: P and f of 64 experts of one sequence,
// and their part of sum_i f_i P_i
__global__ __launch_bounds__(256) void seq_stats_kernel(const float* __restrict__ s, const int32_t* __restrict__ idx,
                                                        const double* __restrict__ rowsum, int N, int K, int seq_len,
                                                        float* __restrict__ f_out, float* __restrict__ p_out,
                                                        double* __restrict__ partial) {
  __shared__ double psum[4][BL_EXPERTS];
  __shared__ int cnt[BL_EXPERTS];
  const int q = blockIdx.x, chunk = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int e = chunk * BL_EXPERTS + lane;
  const int t0 = q * seq_len;
  if (threadIdx.x < BL_EXPERTS) cnt[threadIdx.x] = 0;
  __syncthreads();
  // selections of this sequence that fall in this chunk
  const long nsel = (long)seq_len * K;
  const int32_t* sidx = idx + (size_t)t0 * K;
  for (long p = threadIdx.x; p < nsel; p += 256) {
    const int x = sidx[p] - chunk * BL_EXPERTS;
    if (x >= 0 && x < BL_EXPERTS) atomicAdd(&cnt[x], 1);
  }
  // normalised affinities, tokens w, w+4, ... in order
  double acc = 0.0;
  if (e < N) {
    const double uniform = 1.0 / (double)N;
    for (int t = w; t < seq_len; t += 4) {
      const double tot = rowsum[t0 + t];
      acc += tot > 0.0 ? (double)s[(size_t)(t0 + t) * N + e] / tot : uniform;
    }
  }
  psum[w][lane] = acc;
  __syncthreads();
  if (w == 0) {
    double fp = 0.0;
    if (e < N) {
      const double P = (((psum[0][lane] + psum[1][lane]) + psum[2][lane]) + psum[3][lane]) / (double)seq_len;
      const double f = (double)cnt[lane] / (double)nsel;
      if (f_out) f_out[(size_t)q * N + e] = (float)f;
      if (p_out) p_out[(size_t)q * N + e] = (float)P;
      fp = f * P;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) fp += __shfl_xor(fp, off, 64);
    if (lane == 0) partial[(size_t)q * gridDim.y + chunk] = fp;
  }
}

__global__ void seq_loss_kernel(const double* __restrict__ partial, int n_seq, int n_chunks, float alpha,
                                float* __restrict__ loss) {
  const int q = blockIdx.x * blockDim.x + threadIdx.x;
  if (q >= n_seq) return;
  double acc = 0.0;
  for (int c = 0; c < n_chunks; c++) acc += partial[(size_t)q * n_chunks + c];
  loss[q] = (float)((double)alpha * acc);
}

size_t seq_balance_ws_bytes(int T, int N, int seq_len) {
  const int n_seq = T / seq_len, n_chunks = cdiv(N, BL_EXPERTS);
  return (((size_t)T * 8 + 255) / 256) * 256 + (size_t)n_seq * n_chunks * 8;
}

hipError_t launch_seq_balance(const float* s, const int32_t* idx, int T, int N, int K, int seq_len, float alpha,
                              float* f, float* P, float* loss, void* ws, hipStream_t st) {
  const int n_seq = T / seq_len, n_chunks = cdiv(N, BL_EXPERTS);
  double* rowsum = (double*)ws;
  double* partial = (double*)((uint8_t*)ws + (((size_t)T * 8 + 255) / 256) * 256);
  row_sum_kernel<<<cdiv(T, 4), 256, 0, st>>>(s, rowsum, T, N);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  seq_stats_kernel<<<dim3(n_seq, n_chunks), 256, 0, st>>>(s, idx, rowsum, N, K, seq_len, f, P, partial);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  seq_loss_kernel<<<cdiv(n_seq, 64), 64, 0, st>>>(partial, n_seq, n_chunks, alpha, loss);
  return hipGetLastError();
}

}  // namespace moe
