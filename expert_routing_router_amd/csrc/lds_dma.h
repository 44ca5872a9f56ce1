// Buffer loads that write LDS directly (gfx950 "lds" form), and the explicit
// vector-memory waits that go with them.
//
// The compiler does not see these loads (they are issued from inline
// assembly), so it inserts no waits for them: code that reads the LDS they
// fill waits with wait_vmcnt<N>() itself, N being the number of loads this
// wave issued after the ones it needs (vector-memory loads complete in order).
// Issued through the builtin instead, every LDS read after such a load would
// be made to wait for all loads in flight.
#pragma once
#include "common.h"
#include <type_traits>
#include <utility>

namespace moe {

// One 16-byte-per-lane buffer load that writes LDS at m0 + 16 * lane. The
// instruction has no register result; its completion is tracked by vmcnt,
// which the K loop waits on explicitly. s_nop covers the m0-write hazard.
__device__ __forceinline__ void dma_b128(i32x4 rsrc, int voff, int soff, uint32_t m0) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(m0) : "memory");
}

// The same with the non-temporal hint: for data read once (K-blocked weights,
// whose loads cover whole lines), so it is not kept in L2 at the expense of
// operands other workgroups re-read.
__device__ __forceinline__ void dma_b128_nt(i32x4 rsrc, int voff, int soff, uint32_t m0) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen nt lds"
               :: "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(m0) : "memory");
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// the same, and also every LDS read of this wave done (lgkmcnt 0)
template <int N>
__device__ __forceinline__ void wait_vmcnt_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}

// Buffer resource words of a raw buffer (the operands above need them in
// SGPRs: base and size must be the same in every lane).
__device__ __forceinline__ i32x4 rsrc_words(const void* base, long bytes) {
  const uint64_t a = (uint64_t)base;
  const int n = bytes >= 0x7FFFFFFFL ? 0x7FFFFFFF : (int)bytes;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));   // stride 0
  r[2] = __builtin_amdgcn_readfirstlane(n);
  r[3] = kRawBufferFlags;
  return r;
}

// 4 bytes per lane into LDS at m0 + 4 * lane.
__device__ __forceinline__ void dma_b32(i32x4 rsrc, int voff, int soff, uint32_t m0) {
  asm volatile("s_nop 0\n\tbuffer_load_dword %0, %1, %2 offen lds"
               :: "v"(voff), "s"(rsrc), "s"(soff), "{m0}"(m0) : "memory");
}

// f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>), unrolled at compile time
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// LDS byte address of a shared-memory pointer (the value m0 takes)
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint8_t*)p;
}

}  // namespace moe
