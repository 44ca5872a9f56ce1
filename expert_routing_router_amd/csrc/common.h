// Device helpers shared by the gfx950 kernels of the MoE layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <algorithm>

namespace moe {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;

constexpr int kWave = 64;

// ---------------------------------------------------------------- bf16
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}
// round to nearest even (finite inputs; NaN stays NaN)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (uint16_t)((u >> 16) | ((u & 0xFFFF) ? 0x40 : 0));
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// ---------------------------------------------------------------- ordering keys
// Monotone map fp32 -> uint32 with -0 and +0 mapped to the same value.
__device__ __forceinline__ uint32_t ordered_f32(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) == 0) u = 0;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
// (value desc, index asc) as one unsigned 64-bit key: larger = ranks first.
// 0 is reserved for "no candidate".
__device__ __forceinline__ uint64_t rank_key(float v, uint32_t idx) {
  return ((uint64_t)ordered_f32(v) << 32) | (uint64_t)(0xFFFFFFFFu - idx);
}
__device__ __forceinline__ uint32_t rank_key_index(uint64_t k) {
  return 0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFu);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint64_t o = __shfl_xor(v, off, kWave);
    v = o > v ? o : v;
  }
  return v;
}

// ---------------------------------------------------------------- buffer loads
// Raw buffer loads return zeros for offsets at or beyond num_records instead of
// faulting, so a row that does not exist is loaded from kOutOfRange without a
// branch (a branch around a load forces a full vmcnt wait at the join).
constexpr int kOutOfRange = (int)0x80000000u;
constexpr int kRawBufferFlags = 0x00020000;   // gfx9 raw buffer: DATA_FORMAT = 32-bit
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, long bytes) {
  const int n = bytes >= 0x7FFFFFFFL ? 0x7FFFFFFF : (int)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, kRawBufferFlags);
}

// ---------------------------------------------------------------- misc
__device__ __forceinline__ float silu_mul(float g, float u) {
  return g / (1.0f + __expf(-g)) * u;
}

template <typename T>
__host__ __device__ constexpr T cdiv(T a, T b) { return (a + b - 1) / b; }

}  // namespace moe
