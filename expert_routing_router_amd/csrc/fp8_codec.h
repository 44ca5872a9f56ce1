// E4M3 encoding shared by the activation quantisers and the FP8 gate/up GEMM's
// fused quantisation of H, so both produce the same codes from the same values.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// OCP E4M3FN encoding of an fp32 value: round to nearest even on 3 mantissa
// bits, subnormal step 2^-9, saturation to +-448 (no infinities).
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float ax = fabsf(x);
  if (ax != ax) return sign | 0x7Fu;
  if (ax >= 448.0f) return sign | 0x7Eu;
  if (ax < 0.015625f) {                                  // below 2^-6: multiples of 2^-9
    const uint32_t m = (uint32_t)rintf(ax * 512.0f);     // exact scaling, ties to even
    return sign | m;                                     // m == 8 is the code of 2^-6
  }
  int e = (int)((u >> 23) & 0xFFu) - 127;                // -6 .. 8
  uint32_t m3 = (u >> 20) & 7u;
  const uint32_t rem = u & 0xFFFFFu;
  if (rem > 0x80000u || (rem == 0x80000u && (m3 & 1u))) m3++;
  if (m3 == 8u) { m3 = 0; e++; }
  return sign | ((uint32_t)(e + 7) << 3) | m3;
}

// Four codes in one word (byte e from the e-th value) through gfx950's packed fp8 conversion
// (OCP E4M3, round to nearest even). An exhaustive comparison over every fp32 value of
// magnitude below 464, denormals and signed zeros included, finds it equal to e4m3_encode.
// Values are clamped to +-448 first (both saturate there; the conversion would give NaN from
// 464 on), and a word with a NaN in it is encoded by e4m3_encode (the conversion sets the
// sign bit of a positive NaN's code).
__device__ __forceinline__ uint32_t e4m3_encode4(float a, float b, float c, float d) {
  if (__builtin_expect(a != a || b != b || c != c || d != d, 0))
    return e4m3_encode(a) | (e4m3_encode(b) << 8) | (e4m3_encode(c) << 16) | (e4m3_encode(d) << 24);
  const float lim = 448.0f;
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(fminf(fmaxf(a, -lim), lim), fminf(fmaxf(b, -lim), lim), 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(fminf(fmaxf(c, -lim), lim), fminf(fmaxf(d, -lim), lim), w, true);
  return (uint32_t)w;
}

}  // namespace moe
