// Diagnostics: the machine's attainable HBM read rate and bf16 MFMA rate, measured
// on the GPU that runs the layer, so roofline fractions can be given against the
// measured ceilings as well as against the published peaks.
#include "common.h"
#include "moe_internal.h"

namespace moe {

typedef __bf16 cal_bf16x8 __attribute__((ext_vector_type(8)));
typedef float cal_f32x16 __attribute__((ext_vector_type(16)));

constexpr int kCalUnroll = 8;

// Grid-stride streaming read, 16 B per lane per load, kCalUnroll loads in flight per lane,
// non-temporal (the data is touched once). The XOR of everything read feeds a store that
// never happens in practice, so no load can be dropped.
__global__ __launch_bounds__(256) void cal_read_kernel(const i32x4* __restrict__ p, long n16,
                                                       int32_t* __restrict__ sink) {
  i32x4 acc = {0, 0, 0, 0};
  const long stride = (long)gridDim.x * 256;
  long i = (long)blockIdx.x * 256 + threadIdx.x;
  for (; i + (kCalUnroll - 1) * stride < n16; i += kCalUnroll * stride) {
    i32x4 v[kCalUnroll];
#pragma unroll
    for (int u = 0; u < kCalUnroll; u++) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < kCalUnroll; u++) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= p[i];
  const int x = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (x == 0x5EED1234) sink[0] = x;
}

// Every wave issues `iters` rounds of 8 independent 32x32x16 bf16 MFMAs (32768 flops each).
__global__ __launch_bounds__(256) void cal_mfma_kernel(int iters, float* __restrict__ sink) {
  cal_bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    a[i] = (__bf16)(threadIdx.x * 1e-3f + i);
    b[i] = (__bf16)(1e-3f * i);
  }
  cal_f32x16 c[8] = {};
  for (int it = 0; it < iters; it++) {
#pragma unroll
    for (int j = 0; j < 8; j++) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; j++)
#pragma unroll
    for (int r = 0; r < 16; r++) s += c[j][r];
  if (s == 1234.5f) sink[0] = s;
}

hipError_t launch_cal_read(const void* buf, size_t bytes, int32_t* sink, hipStream_t s) {
  cal_read_kernel<<<4096, 256, 0, s>>>((const i32x4*)buf, (long)(bytes / 16), sink);
  return hipGetLastError();
}

hipError_t launch_cal_mfma(int iters, float* sink, hipStream_t s) {
  cal_mfma_kernel<<<kCalMfmaWaves / 4, 256, 0, s>>>(iters, sink);
  return hipGetLastError();
}

}  // namespace moe
