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

// Four 1-KB copies sharing one LDS base: copy j moves lane i's 16 bytes from
// base + vj + 1024 j to LDS byte lds + 1024 j + 16 i (the instruction offset
// applies to the global and the LDS address alike). m0 is declared clobbered,
// so the compiler keeps nothing of its own there across the copies.
__device__ __forceinline__ void dma_copy16x4(const void* base, uint32_t v0, uint32_t v1, uint32_t v2,
                                             uint32_t v3, const lds_char* lds) {
  const uint32_t lds_addr = (uint32_t)(uintptr_t)lds;
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %5\n\t"
      "global_load_lds_dwordx4 %2, %5 offset:1024\n\t"
      "global_load_lds_dwordx4 %3, %5 offset:2048\n\t"
      "global_load_lds_dwordx4 %4, %5 offset:3072"
      :
      : "s"(lds_addr), "v"(v0), "v"(v1), "v"(v2), "v"(v3), "s"(base)
      : "memory", "m0");
}

// One 1-KB copy at instruction offset OFF (added to the global and the LDS
// address alike) with m0 declared clobbered: several copies can share one
// global base and one LDS base, with the per-copy offset in the instruction.
template <int OFF>
__device__ __forceinline__ void dma_copy16_off(const void* base, uint32_t voff, const lds_char* lds) {
  const uint32_t lds_addr = (uint32_t)(uintptr_t)lds;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 offset:%3"
               :
               : "s"(lds_addr), "v"(voff), "s"(base), "i"(OFF)
               : "memory", "m0");
}

// Single 16-byte and 4-byte copies with m0 declared clobbered (no restore).
__device__ __forceinline__ void dma_copy16_m0(const void* base, uint32_t voff, const lds_char* lds) {
  const uint32_t lds_addr = (uint32_t)(uintptr_t)lds;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds_addr), "v"(voff), "s"(base)
               : "memory", "m0");
}
__device__ __forceinline__ void dma_copy4_m0(const void* base, uint32_t voff, const lds_char* lds) {
  const uint32_t lds_addr = (uint32_t)(uintptr_t)lds;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
               :
               : "s"(lds_addr), "v"(voff), "s"(base)
               : "memory", "m0");
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

// The same barrier letting the N most recent LDS reads of this wave stay in
// flight (reads of data that no other wave overwrites before the next
// barrier).
template <int N>
__device__ __forceinline__ void lds_barrier_keep() {
  static_assert(N >= 0 && N <= 15, "lgkmcnt field");
  asm volatile("s_waitcnt lgkmcnt(%0)\n\ts_barrier" ::"i"(N) : "memory");
}

}  // namespace mla
