// Memory-bound kernels of the layer: the gated combine, the bias update and
// the FP8 quantisers.
#include "common.h"
#include "fp8_codec.h"
#include "moe_internal.h"

namespace moe {

// ---------------------------------------------------------------- combine
// out_t = u_t + sum_s Ys[s][t] + sum_k gate[t,k] * Y[slot_row[t*K+k]]
// (output equation of the DeepSeek-V3 guides, "Metodo" section 2; the pwwt.cn
// note's section 4 combine), fp32 accumulation in that fixed order. One wave
// per token: the token's row indices and gates are wave-uniform, so they come
// through the scalar cache (no LDS, no barrier), and every lane handles 8
// consecutive elements of CW chunks of 512 elements at once, so a lane has
// CW * (2 + K) loads in flight. Everything here is read or written once:
// loads and stores carry the non-temporal hint.
constexpr int CW = 8;                // 512-element chunks per lane and pass
constexpr int CWR = 2;               // routed rows loaded together

template <bool BF>
__device__ __forceinline__ void combine_load8_nt(const void* base, size_t row, int d, int c, float* v) {
  if (BF) {
    const i32x4 q = __builtin_nontemporal_load((const i32x4*)((const uint16_t*)base + row * d + c));
#pragma unroll
    for (int i = 0; i < 4; i++) {
      v[2 * i] = __uint_as_float(((uint32_t)q[i]) << 16);
      v[2 * i + 1] = __uint_as_float(((uint32_t)q[i]) & 0xFFFF0000u);
    }
  } else {
    const f32x4 p0 = __builtin_nontemporal_load((const f32x4*)((const float*)base + row * d + c));
    const f32x4 p1 = __builtin_nontemporal_load((const f32x4*)((const float*)base + row * d + c + 4));
#pragma unroll
    for (int i = 0; i < 4; i++) { v[i] = p0[i]; v[4 + i] = p1[i]; }
  }
}

template <bool IO_BF16, bool Y_BF16>
__global__ __launch_bounds__(64) void combine_wave_kernel(CombineArgs a) {
  const int t = blockIdx.x;
  const int lane = threadIdx.x;
  const unsigned n_rows = (unsigned)(a.T * a.K);
  const int32_t* srow = a.slot_row + (size_t)t * a.K;
  const float* sg = a.gate + (size_t)t * a.K;
  for (int c0 = lane * 8; c0 < a.d; c0 += 64 * 8 * CW) {
    float acc[CW][8];
    bool in[CW];
#pragma unroll
    for (int w = 0; w < CW; w++) {
      const int c = c0 + w * 512;
      in[w] = c < a.d;
      combine_load8_nt<IO_BF16>(a.u, t, a.d, in[w] ? c : 0, acc[w]);
    }
    for (int k0 = 0; k0 < a.K; k0 += CWR) {
      float v[CW][CWR][8];
      bool use[CWR];
#pragma unroll
      for (int j = 0; j < CWR; j++) {
        const int k = k0 + j;
        const int r = k < a.K ? srow[k] : 0;
        use[j] = k < a.K && (unsigned)r < n_rows;    // a dropped selection adds nothing
#pragma unroll
        for (int w = 0; w < CW; w++)
          combine_load8_nt<Y_BF16>(a.y, use[j] ? (size_t)r : 0, a.d, in[w] ? c0 + w * 512 : 0, v[w][j]);
      }
      if (k0 == 0) {
        for (int s = 0; s < a.n_shared; s++) {
#pragma unroll
          for (int w = 0; w < CW; w++) {
            float x[8];
            combine_load8_nt<Y_BF16>(a.y_shared, (size_t)s * a.shared_stride + t, a.d, in[w] ? c0 + w * 512 : 0, x);
#pragma unroll
            for (int i = 0; i < 8; i++) acc[w][i] += x[i];
          }
        }
      }
#pragma unroll
      for (int j = 0; j < CWR; j++) {
        if (use[j]) {
          const float g = sg[k0 + j];
#pragma unroll
          for (int w = 0; w < CW; w++)
#pragma unroll
            for (int i = 0; i < 8; i++) acc[w][i] = fmaf(g, v[w][j][i], acc[w][i]);
        }
      }
    }
#pragma unroll
    for (int w = 0; w < CW; w++) {
      if (!in[w]) continue;
      const int c = c0 + w * 512;
      if (IO_BF16) {
        i32x4 q;
#pragma unroll
        for (int i = 0; i < 4; i++) q[i] = (int)pack_bf16x2(acc[w][2 * i], acc[w][2 * i + 1]);
        __builtin_nontemporal_store(q, (i32x4*)((uint16_t*)a.out + (size_t)t * a.d + c));
      } else {
        float* o = (float*)a.out + (size_t)t * a.d + c;
        __builtin_nontemporal_store(f32x4{acc[w][0], acc[w][1], acc[w][2], acc[w][3]}, (f32x4*)o);
        __builtin_nontemporal_store(f32x4{acc[w][4], acc[w][5], acc[w][6], acc[w][7]}, (f32x4*)(o + 4));
      }
    }
  }
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
  if (a.T <= 0) return hipSuccess;
  const bool io = a.io_dtype == MOE_BF16, yb = a.y_dtype == MOE_BF16;
  if (io && yb) combine_wave_kernel<true, true><<<a.T, 64, 0, s>>>(a);
  else if (io) combine_wave_kernel<true, false><<<a.T, 64, 0, s>>>(a);
  else if (yb) combine_wave_kernel<false, true><<<a.T, 64, 0, s>>>(a);
  else combine_wave_kernel<false, false><<<a.T, 64, 0, s>>>(a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- bias update
// pwwt.cn note 1.1.3 / guides section 2: overloaded -> b - gamma, underloaded
// -> b + gamma. Overloaded means a load above the batch mean T*K/N_r, compared
// exactly in integers; a load equal to the mean leaves b unchanged.
__global__ void update_bias_kernel(const int32_t* __restrict__ counts, float* __restrict__ b,
                                   int n, long total, float gamma) {
  for (int e = blockIdx.x * blockDim.x + threadIdx.x; e < n; e += gridDim.x * blockDim.x) {
    const long lhs = (long)n * counts[e];
    if (lhs > total) b[e] = b[e] - gamma;
    else if (lhs < total) b[e] = b[e] + gamma;
  }
}

hipError_t launch_update_bias(const int32_t* counts, float* b, int n_routed, long total,
                              float gamma, hipStream_t s) {
  update_bias_kernel<<<cdiv(n_routed, 256), 256, 0, s>>>(counts, b, n_routed, total, gamma);
  return hipGetLastError();
}

// ---------------------------------------------------------------- FP8 quantisers
__device__ __forceinline__ float load_src(const void* p, size_t i, bool bf) {
  return bf ? bf16_to_f32(((const uint16_t*)p)[i]) : ((const float*)p)[i];
}

// 16 lanes per (row, 128-column tile), 8 consecutive columns per lane (one
// 16-byte bf16 or two 16-byte fp32 loads, one 8-byte store of codes), 16
// tiles per workgroup: amax over the tile by xor swizzles inside the 16-lane
// group, scale = fl32(amax/448), codes = e4m3(v / scale). A tile's 16 lanes
// are live or not together, so the swizzles never read a lane that left.
template <int OFF>
__device__ __forceinline__ float swz_xor(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1F | (OFF << 10)));
}
// TS: scales stored transposed, scale[c / 128][r]
template <bool BF, bool TS = false>
__global__ __launch_bounds__(256) void quant_act_kernel(const void* __restrict__ src, long rows, int cols,
                                                        const int32_t* __restrict__ row_index,
                                                        uint8_t* __restrict__ q, float* __restrict__ scale) {
  const int sub = threadIdx.x & 15;
  const long tile = ((long)blockIdx.x * 256 + threadIdx.x) >> 4;
  const int tpr = cols / 128;
  if (tile >= rows * tpr) return;
  const long r = tile / tpr;
  const int c0 = (int)(tile - r * tpr) * 128 + sub * 8;
  const long sr = row_index ? row_index[r] : r;
  float v[8];
  if (BF) {
    const i32x4 raw = *(const i32x4*)((const uint16_t*)src + (size_t)sr * cols + c0);
#pragma unroll
    for (int i = 0; i < 4; i++) {
      v[2 * i] = __uint_as_float((uint32_t)raw[i] << 16);
      v[2 * i + 1] = __uint_as_float((uint32_t)raw[i] & 0xFFFF0000u);
    }
  } else {
    const f32x4* p = (const f32x4*)((const float*)src + (size_t)sr * cols + c0);
    const f32x4 a = p[0], b = p[1];
#pragma unroll
    for (int i = 0; i < 4; i++) { v[i] = a[i]; v[4 + i] = b[i]; }
  }
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; i++) m = fmaxf(m, fabsf(v[i]));
  m = fmaxf(m, swz_xor<1>(m));
  m = fmaxf(m, swz_xor<2>(m));
  m = fmaxf(m, swz_xor<4>(m));
  m = fmaxf(m, swz_xor<8>(m));
  const float sc = m == 0.0f ? 1.0f : m / 448.0f;
  const uint32_t lo = e4m3_encode4(v[0] / sc, v[1] / sc, v[2] / sc, v[3] / sc);
  const uint32_t hi = e4m3_encode4(v[4] / sc, v[5] / sc, v[6] / sc, v[7] / sc);
  *(uint2*)(q + (size_t)r * cols + c0) = make_uint2(lo, hi);
  if (sub == 0) scale[TS ? (size_t)(c0 / 128) * rows + r : (size_t)r * tpr + c0 / 128] = sc;
}

// One workgroup per 128x128 block.
template <bool BF>
__global__ __launch_bounds__(256) void quant_w_kernel(const void* __restrict__ src, long rows, int cols,
                                                      uint8_t* __restrict__ q, float* __restrict__ scale) {
  __shared__ float red[4];
  const int bpr = cols / 128;
  const long br = blockIdx.x / bpr;
  const int bc = blockIdx.x - (int)(br * bpr);
  float m = 0.f;
  for (int i = threadIdx.x; i < 128 * 128; i += 256) {
    const long r = br * 128 + (i >> 7);
    const int c = bc * 128 + (i & 127);
    m = fmaxf(m, fabsf(load_src(src, (size_t)r * cols + c, BF)));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, kWave));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float sc = m == 0.0f ? 1.0f : m / 448.0f;
  for (int i = threadIdx.x; i < 128 * 128; i += 256) {
    const long r = br * 128 + (i >> 7);
    const int c = bc * 128 + (i & 127);
    q[(size_t)r * cols + c] = (uint8_t)e4m3_encode(load_src(src, (size_t)r * cols + c, BF) / sc);
  }
  if (threadIdx.x == 0) scale[(size_t)br * bpr + bc] = sc;
}

hipError_t launch_quant_act(const void* src, int src_dtype, long rows, int cols, const int32_t* row_index,
                            uint8_t* q, float* scale, hipStream_t s) {
  const long tiles = rows * (cols / 128);
  if (tiles <= 0) return hipSuccess;
  const unsigned grid = (unsigned)cdiv<long>(tiles, 16);
  if (src_dtype == MOE_BF16) quant_act_kernel<true><<<grid, 256, 0, s>>>(src, rows, cols, row_index, q, scale);
  else quant_act_kernel<false><<<grid, 256, 0, s>>>(src, rows, cols, row_index, q, scale);
  return hipGetLastError();
}

hipError_t launch_quant_act_tscale(const uint16_t* src, long rows, int cols, uint8_t* q, float* scale_t,
                                   hipStream_t s) {
  const long tiles = rows * (cols / 128);
  if (tiles <= 0) return hipSuccess;
  quant_act_kernel<true, true><<<(unsigned)cdiv<long>(tiles, 16), 256, 0, s>>>(src, rows, cols, nullptr, q, scale_t);
  return hipGetLastError();
}

hipError_t launch_quant_w(const void* src, int src_dtype, long rows, int cols, uint8_t* q, float* scale,
                          hipStream_t s) {
  const long blocks = (rows / 128) * (cols / 128);
  if (blocks <= 0) return hipSuccess;
  if (src_dtype == MOE_BF16) quant_w_kernel<true><<<(unsigned)blocks, 256, 0, s>>>(src, rows, cols, q, scale);
  else quant_w_kernel<false><<<(unsigned)blocks, 256, 0, s>>>(src, rows, cols, q, scale);
  return hipGetLastError();
}

}  // namespace moe
