// lds_dma.h — direct global -> LDS loads on gfx950, and scalar pointers.
#pragma once

#include "xq_device.h"

namespace xq {

// One direct global -> LDS load (gfx950 global_load_lds_dwordx4 /
// global_load_lds_dword): lane l's bytes land at LDS address m0 + size*l; an
// inactive lane writes nothing. Issued as inline assembly so the compiler's
// wait-count pass does not treat the in-flight loads as hazards for other LDS
// reads; a kernel that uses them waits for them itself (vmcnt) before the
// barrier that publishes their bytes.
__device__ __forceinline__ void lds_dma16(const uint8_t* base, uint32_t off, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1\n\t"
      :
      : "v"(off), "s"(base), "s"(lds_addr)
      : "memory", "m0");
}

__device__ __forceinline__ void lds_dma4(const uint8_t* base, uint32_t off, uint32_t lds_addr) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %0, %1\n\t"
      :
      : "v"(off), "s"(base), "s"(lds_addr)
      : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// A pointer every lane holds the same value of, as a scalar (the direct
// loads take their base in scalar registers).
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<const uint8_t*>((static_cast<uint64_t>(hi) << 32) | lo);
}

}  // namespace xq
