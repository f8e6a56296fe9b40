// Asynchronous global -> LDS copies (global_load_lds_dwordx4 / _dword).
// Lane i's 16 (or 4) bytes from base + voff land at LDS byte address
// lds + 16*i (4*i), so one instruction fills 1 KB (256 B) of contiguous LDS;
// a swizzled LDS layout is obtained by choosing which global chunk each lane
// fetches. Written as inline assembly so the compiler's wait insertion never
// serializes them with later LDS traffic: the issuing wave waits for them
// explicitly (dma_wait) before the barrier that publishes the data. They
// have no output registers, and their address operands are consumed at
// issue. m0 (the LDS base register of the copy) is restored afterwards.
#pragma once

#include "mla_device.h"

namespace mla {

__device__ __forceinline__ void dma_copy16(const void* base, uint32_t voff, const lds_char* lds) {
  const uint32_t lds_addr = (uint32_t)(uintptr_t)lds;
  uint32_t saved_m0;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved_m0)
      : "s"(lds_addr), "v"(voff), "s"(base)
      : "memory");
}

// The same with 4 bytes per lane (lane i's word lands at lds + 4*i).
__device__ __forceinline__ void dma_copy4(const void* base, uint32_t voff, const lds_char* lds) {
  const uint32_t lds_addr = (uint32_t)(uintptr_t)lds;
  uint32_t saved_m0;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved_m0)
      : "s"(lds_addr), "v"(voff), "s"(base)
      : "memory");
}

// Wait until at most N of this wave's copies (and other vector memory loads)
// are in flight; they complete in issue order.
template <int N>
__device__ __forceinline__ void dma_wait() {
  static_assert(N >= 0 && N <= 15, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// Workgroup barrier that orders LDS traffic: this wave's LDS operations
// complete (lgkmcnt 0), then all waves meet. Copies in flight (vmcnt) keep
// running across it; the memory clobber keeps the compiler from moving
// memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace mla
