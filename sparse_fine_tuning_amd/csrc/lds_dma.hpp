// Direct global -> LDS copies (gfx950 global_load_lds_dwordx4) and the
// explicit vmcnt waits that track them.
#pragma once

#include "common.hpp"

namespace usaf {

typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt with vmcnt <= n (expcnt and lgkmcnt left unconstrained).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// One wave-wide 16-byte-per-lane copy: lane l's 16 bytes land at
// lds_base + 16 l.  lds_base must be the same for the whole wave.  Issued as
// inline assembly: completion is tracked only by the explicit vmcnt waits of
// the pipeline (the compiler's own tracking would wait for every copy in
// flight before each LDS read).  M0 holds the LDS address; one wait state
// separates its write from the copy.
__device__ __forceinline__ void dma16(const void* g, unsigned char* lds_base) {
  const uint32_t l = __builtin_amdgcn_readfirstlane(uint32_t(size_t((lds_void_t*)lds_base)));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "s"(l)
               : "memory", "m0");
}

// The same with 4 bytes per lane: lane l's 4 bytes land at lds_base + 4 l.
// The global address must be 4-byte aligned.
__device__ __forceinline__ void dma4(const void* g, unsigned char* lds_base) {
  const uint32_t l = __builtin_amdgcn_readfirstlane(uint32_t(size_t((lds_void_t*)lds_base)));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :
               : "v"(g), "s"(l)
               : "memory", "m0");
}

}  // namespace usaf
