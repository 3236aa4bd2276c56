// Device-side helpers shared by the gfx950 kernels: vector types, bf16 / e4m3
// conversions and wave64 reductions.
#pragma once
#include <type_traits>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr float kE4M3Max = 448.0f;

// fp32 -> bf16 bits, round to nearest even (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// Two fp32 values (already clamped to [-448, 448]) -> two e4m3 codes, round to
// nearest even, packed into the low 16 bits (a in byte 0, b in byte 1).
__device__ __forceinline__ uint32_t e4m3x2(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// Four clamped fp32 values -> four e4m3 codes in one dword (a in the low byte).
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

__device__ __forceinline__ float clamp448(float v) {
  return fminf(fmaxf(v, -kE4M3Max), kE4M3Max);
}

// The scale of a 1x128 / 128x128 block: fl32(amax / 448), 1 for an all-zero block.
__device__ __forceinline__ float block_scale(float amax) {
  return amax > 0.0f ? amax / kE4M3Max : 1.0f;
}

// wave64 reductions over lane groups of width W (a power of two <= 64).
template <int W>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = W / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

// silu with a hardware reciprocal (about 1 ulp) in place of the IEEE division; used in
// GEMM epilogues whose result is rounded to 8 bits right after.
__device__ __forceinline__ float silu_fast(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

constexpr int gcd_c(int a, int b) { return b == 0 ? a : gcd_c(b, a % b); }

// f(integral_constant<0>), ..., f(integral_constant<N-1>) in order
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(std::integral_constant<int, N - 1>{});
  }
}

}  // namespace moe
