// Direct global -> LDS copies issued from inline assembly, with explicit
// vmcnt waits.
//
// global_load_lds_dwordx4 writes each lane's 16 bytes to LDS at M0 + 16 *
// lane, bypassing registers.  The compiler tracks such copies only as "some
// LDS write" and waits for every outstanding one before any LDS read, which
// serialises a multi-stage ring; issued from assembly they are invisible to
// it, and the kernel waits for exactly the stage it needs with
// s_waitcnt vmcnt(N) (vector-memory loads retire in issue order).  Rules for
// callers: no compiler-issued vector-memory load may be in flight across a
// ring wait that it does not cover (compiler loads issued after the copies
// make it wait conservatively, which is safe), every copy must have been
// waited for before the kernel ends, and no other code may use M0 (these
// kernels do no dynamic register indexing, LDS-DMA builtins or messages).
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

namespace dstill {

__device__ __forceinline__ uint32_t lds_u32(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// One direct global->LDS copy of 16 bytes per lane: global address base +
// voff (base wave-uniform, voff per lane, bytes), LDS address lds + 16 * lane
// (lds wave-uniform).  M0 carries the LDS address; s_nop covers the M0 write
// -> LDS-DMA read hazard.
// M0 is a reserved register: the clobber warns that the compiler does not
// preserve it around the statement, which is what these kernels rely on.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void *base, uint32_t voff, uint32_t lds) {
  const uint64_t b = (uint64_t)base;
  const uint64_t sb = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t sl = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sb), "s"(sl)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt vmcnt(N) (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and
// lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

}  // namespace dstill
