// Direct global->LDS DMA helpers shared by the GEMM kernels and the router.
#pragma once
#include <stdint.h>

#include "common.hpp"

namespace moe {

// LDS DMA into one LDS buffer indexed at run time: each lane's 16 (or 4) bytes land at
// M0 + lane * size.  Written as inline asm, invisible to the compiler's wait counting:
// as an LDS store of unknown place the builtin would make it wait for every
// outstanding DMA (vmcnt(0)) before each LDS read, which drains the pipeline.  The
// caller orders the DMA itself with s_waitcnt vmcnt and s_barrier.  The instruction has
// no VGPR result, so no register is left in flight.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// (An LDS DMA needs one wait state after the write of M0 that addresses it.)
__device__ __forceinline__ void dma16(const void* g, uint32_t m) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(m), "v"(g) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t m) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
               :: "s"(m), "v"(g) : "memory", "m0");
}

// Global->LDS DMA of 16 bytes per lane (lane L lands at lds_dst + 16 L) through a buffer
// resource with a 32-bit lane offset.  Written with the compiler builtin, so the
// compiler counts it among the vector memory operations (its waits for register loads
// stay exact) and, when every stage is an LDS object of its own, tells a DMA into one
// stage apart from reads of another.  (The flat-segment form of the same builtin makes
// the compiler assume a pending LDS access and wait for zero.)
__device__ __forceinline__ void dma16b(const void* base, uint32_t voff, void* lds_dst) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, -1, 0x00020000);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds_dst,
                                           16, voff, 0, 0, 0);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <int N>
__device__ __forceinline__ void wait_vmcnt_upto(int n) {
  // s_waitcnt needs an immediate: dispatch a runtime count in [0, N]
  if constexpr (N > 0) {
    if (n >= N) { wait_vmcnt<N>(); return; }
    wait_vmcnt_upto<N - 1>(n);
  } else {
    wait_vmcnt<0>();
  }
}

}  // namespace moe
