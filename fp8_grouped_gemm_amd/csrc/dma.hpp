// Direct global->LDS DMA helpers shared by the grouped GEMMs.
#pragma once
#include "common.hpp"

namespace moe {

// LDS DMA: each lane's 16 (or 4) bytes land at M0 + lane * size.  Written as inline
// asm so the compiler does not treat the DMA as an LDS store of unknown address: with
// the builtin it waits for every outstanding DMA (vmcnt(0)) before each LDS read, which
// drains the pipeline.  The K loop orders the DMA itself with s_waitcnt vmcnt and
// s_barrier.  The instruction has no VGPR result, so no register is left in flight.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ void dma16(const void* g, uint32_t m) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(m), "v"(g) : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void* g, uint32_t m) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, off"
               :: "s"(m), "v"(g) : "memory", "m0");
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
