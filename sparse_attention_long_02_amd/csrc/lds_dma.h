// Direct global->LDS loads issued from inline asm, and the waits and barriers that order
// them (gfx950).  The compiler's wait-counter model does not see these loads, so LDS reads
// of the buffers they fill keep exact LDS-counter waits; the kernels order the buffers
// themselves with explicit vector-memory waits and block barriers.
#pragma once

#include "dsa_device.h"

namespace dsa {

#define VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))
#define LGKM0() __builtin_amdgcn_s_waitcnt(0xC07F)

// Workgroup barrier that is also a compiler memory barrier (LDS accesses stay on their side),
// with no wait-counter drain: the chunk loads stay in flight across it.
__device__ __forceinline__ void block_barrier() {
  __builtin_amdgcn_s_barrier();
  asm volatile("" : : : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t*)p;
}

// One direct global->LDS load of 16 bytes per lane: lane i's bytes go to LDS address
// lds + 16 i (a direct load the compiler can see would force every LDS wait behind it to
// zero).  No register is written; one wait state separates the M0 write from the load that
// reads it.  M0 holds nothing else in the kernels that use these loads, so clobbering it is
// safe.  Every active lane loads: a kernel that has nothing left to gather re-loads rows it
// already has into a buffer no later read uses, which costs less than narrowing the exec
// mask around each load.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16_saddr(const void* gbase, uint32_t voff, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2"
      :
      : "s"(lds), "v"(voff), "s"(gbase)
      : "memory", "m0");
}
__device__ __forceinline__ void dma16_vaddr(const void* gaddr, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off"
      :
      : "s"(lds), "v"(gaddr)
      : "memory", "m0");
}
// 4 bytes per lane (lane i's bytes go to lds + 4 i).
__device__ __forceinline__ void dma4_vaddr(const void* gaddr, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %1, off"
      :
      : "s"(lds), "v"(gaddr)
      : "memory", "m0");
}
#pragma clang diagnostic pop

}  // namespace dsa
