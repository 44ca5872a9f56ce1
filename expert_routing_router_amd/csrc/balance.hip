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

constexpr int BL_TOKENS = 64;      // tokens per workgroup of the statistics kernel

// grid (n_seq * n_split, ceil(N/64)), 256 threads: for 64 tokens of one
// sequence and 64 experts, the fp64 sum of the normalised affinities and the
// number of selections (written per split, summed in order by seq_final_kernel)
__global__ __launch_bounds__(256) void seq_stats_kernel(const float* __restrict__ s, const int32_t* __restrict__ idx,
                                                        const double* __restrict__ rowsum, int N, int K, int seq_len,
                                                        int n_split, double* __restrict__ psum_out,
                                                        int32_t* __restrict__ cnt_out) {
  __shared__ double psum[4][BL_EXPERTS];
  __shared__ int cnt[BL_EXPERTS];
  const int q = blockIdx.x / n_split, split = blockIdx.x - q * n_split, chunk = blockIdx.y;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int e = chunk * BL_EXPERTS + lane;
  const int tb = split * BL_TOKENS, te = min(seq_len, tb + BL_TOKENS);
  const int t0 = q * seq_len;
  if (threadIdx.x < BL_EXPERTS) cnt[threadIdx.x] = 0;
  __syncthreads();
  const int32_t* sidx = idx + (size_t)(t0 + tb) * K;
  for (int p = threadIdx.x; p < (te - tb) * K; p += 256) {
    const int x = sidx[p] - chunk * BL_EXPERTS;
    if (x >= 0 && x < BL_EXPERTS) atomicAdd(&cnt[x], 1);
  }
  double acc = 0.0;
  if (e < N) {
    const double uniform = 1.0 / (double)N;
    for (int t = tb + w; t < te; t += 4) {
      const double tot = rowsum[t0 + t];
      acc += tot > 0.0 ? (double)s[(size_t)(t0 + t) * N + e] / tot : uniform;
    }
  }
  psum[w][lane] = acc;
  __syncthreads();
  if (w == 0 && e < N) {
    const size_t o = ((size_t)q * n_split + split) * N + e;
    psum_out[o] = ((psum[0][lane] + psum[1][lane]) + psum[2][lane]) + psum[3][lane];
    cnt_out[o] = cnt[lane];
  }
}

// one workgroup (256 threads, thread = expert) per sequence: f, P, and
// loss = alpha * sum_i f_i P_i with a fixed-order tree sum
__global__ __launch_bounds__(256) void seq_final_kernel(const double* __restrict__ psum, const int32_t* __restrict__ cnt,
                                                        int N, int K, int seq_len, int n_split, float alpha,
                                                        float* __restrict__ f_out, float* __restrict__ p_out,
                                                        float* __restrict__ loss) {
  __shared__ double red[256];
  const int q = blockIdx.x, e = threadIdx.x;
  double fp = 0.0;
  if (e < N) {
    double ps = 0.0;
    long c = 0;
    for (int sp = 0; sp < n_split; sp++) {
      const size_t o = ((size_t)q * n_split + sp) * N + e;
      ps += psum[o];
      c += cnt[o];
    }
    const double P = ps / (double)seq_len;
    const double f = (double)c / ((double)seq_len * K);
    if (f_out) f_out[(size_t)q * N + e] = (float)f;
    if (p_out) p_out[(size_t)q * N + e] = (float)P;
    fp = f * P;
  }
  red[e] = fp;
  __syncthreads();
  for (int h = 128; h >= 1; h >>= 1) {
    if (e < h) red[e] += red[e + h];
    __syncthreads();
  }
  if (e == 0) loss[q] = (float)((double)alpha * red[0]);
}

static int n_splits(int seq_len) { return (seq_len + BL_TOKENS - 1) / BL_TOKENS; }

size_t seq_balance_ws_bytes(int T, int N, int seq_len) {
  const size_t parts = (size_t)(T / seq_len) * n_splits(seq_len) * N;
  return (((size_t)T * 8 + 255) / 256) * 256 + ((parts * 8 + 255) / 256) * 256 + parts * 4;
}

hipError_t launch_seq_balance(const float* s, const int32_t* idx, int T, int N, int K, int seq_len, float alpha,
                              float* f, float* P, float* loss, void* ws, hipStream_t st) {
  const int n_seq = T / seq_len, n_split = n_splits(seq_len), n_chunks = cdiv(N, BL_EXPERTS);
  const size_t parts = (size_t)n_seq * n_split * N;
  uint8_t* base = (uint8_t*)ws;
  double* rowsum = (double*)base;
  double* psum = (double*)(base + (((size_t)T * 8 + 255) / 256) * 256);
  int32_t* cnt = (int32_t*)((uint8_t*)psum + ((parts * 8 + 255) / 256) * 256);
  row_sum_kernel<<<cdiv(T, 4), 256, 0, st>>>(s, rowsum, T, N);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  seq_stats_kernel<<<dim3(n_seq * n_split, n_chunks), 256, 0, st>>>(s, idx, rowsum, N, K, seq_len, n_split, psum, cnt);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  seq_final_kernel<<<n_seq, 256, 0, st>>>(psum, cnt, N, K, seq_len, n_split, alpha, f, P, loss);
  return hipGetLastError();
}

}  // namespace moe
