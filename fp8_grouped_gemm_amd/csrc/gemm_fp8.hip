// Grouped FP8 GEMM for gfx950 with e4m3 weights in 128x128 scale blocks: the offline
// fragment-major weight packing and the launcher of the kernel template in
// gemm_fp8_kernel.hpp (where the design is described).
#include <algorithm>
#include <cstdlib>

#include "gemm_fp8_kernel.hpp"

namespace moe {

// Rows of the large-group tiles.  192-row tiles move 22% fewer operand bytes per FLOP
// than 128-row ones and measured faster wherever groups are tiled (Zipf grouped GEMM
// +3-5%, prefill layer 1-2%, the 4-bit-weight hash layer 6%: its ~128-row experts fit one
// tile; bit-identical results); a dense M is tiled by whichever
// size gives the shorter schedule: rounds of the grid times the tile's cost (a 192-row
// tile measured at ~1.37 times a 128-row one), so M = 8192 (four full rounds of 128-row
// tiles) keeps 128.  K above 128 * kGemmMaxKBlocks192 and the opt-in 256-row mode keep
// 128.  FP8GG_TILE_ROWS=128 or 192 in the environment (read at each call) overrides the
// choice where both are possible.
int large_tile_rows(int rows_mode, int M, int N, int K, bool swiglu, int num_cus, bool big) {
  if (big || K / 128 > kGemmMaxKBlocks192) return 128;
  if (const char* e = std::getenv("FP8GG_TILE_ROWS")) {
    const int v = std::atoi(e);
    if (v == 128 || v == 192) return v;
  }
  if (rows_mode != kRowsDense) return 192;
  const long tiles_n = swiglu ? N / 128 : (N + 255) / 256;
  auto cost = [&](int b, double unit) {
    const long tiles = (long)((M + b - 1) / b) * tiles_n;
    const long grid = std::max(1L, std::min<long>(tiles, num_cus));
    return (double)((tiles + grid - 1) / grid) * unit;
  };
  return cost(192, 1.37) < cost(128, 1.0) ? 192 : 128;
}

// Fragment-major weight layout: B [G][R][K] e4m3 -> Bf [G][R/16][K/128][2][64][16 B],
// where half h and lane l of fragment (nb, kb) hold
// B[16 nb + (l & 15)][128 kb + 32 (l >> 4) + 16 h .. +16] -- the 16x128 operand of one
// 16x16x128 MFMA, as lane l reads it (rows by lane & 15, 32-byte K chunks by lane >> 4).
__global__ void pack_weight_fp8_kernel(const uint8_t* __restrict__ B, uint8_t* __restrict__ Bf,
                                       int G, int R, int K) {
  const size_t total = (size_t)G * R * (size_t)(K / 16);
  const int KB = K / 128, R16 = R / 16;
  for (size_t p = (size_t)blockIdx.x * blockDim.x + threadIdx.x; p < total;
       p += (size_t)gridDim.x * blockDim.x) {
    const int l = (int)(p % 64);
    size_t q = p / 64;
    const int h = (int)(q % 2);
    q /= 2;
    const int kb = (int)(q % KB);
    q /= KB;
    const int nb = (int)(q % R16);
    const size_t g = q / R16;
    const int row = nb * 16 + (l & 15);
    const int k = kb * 128 + 32 * (l >> 4) + 16 * h;
    *reinterpret_cast<v4i*>(Bf + p * 16) =
        *reinterpret_cast<const v4i*>(B + (g * R + row) * (size_t)K + k);
  }
}

hipError_t launch_pack_weight_fp8(const uint8_t* B, int G, int R, int K, uint8_t* Bf,
                                  hipStream_t s) {
  const size_t pieces = (size_t)G * R * (size_t)(K / 16);
  const size_t blocks = std::min<size_t>((pieces + 255) / 256, 16384);
  hipLaunchKernelGGL(pack_weight_fp8_kernel, dim3((unsigned)blocks), dim3(256), 0, s, B, Bf, G,
                     R, K);
  return hipGetLastError();
}

hipError_t launch_gemm_fp8(const uint8_t* A, const float* sA, const int32_t* a_rows, int a_row_div,
                           const uint8_t* Bf, const float* sB, const int32_t* offsets, int G,
                           int R_cap, int N, int K, bool swiglu, void* C, float* sC, int bm,
                           int num_cus, hipStream_t s, int rows_mode, int cap, bool big) {
  // 256-column tiles (SwiGLU: 128 output columns from 256 weight rows), an even number of
  // K blocks, and a group's weights within 32-bit offsets
  big = big && (swiglu || N % 256 == 0) && (K / 128) % 2 == 0 &&
        (long long)(swiglu ? 2 * N : N) * K < (1LL << 31);
  if (big) {
    const hipError_t e = launch_gemm_fp8_big(A, sA, a_rows, a_row_div, Bf, sB, offsets, G, N, K,
                                             swiglu, C, sC, num_cus, s, rows_mode, cap);
    if (e != hipSuccess) return e;
  }
  return launch_gemm_impl<false>(A, sA, a_rows, a_row_div, Bf, sB, offsets, G, R_cap, N, K,
                                 swiglu, C, sC, bm, num_cus, s, rows_mode, cap,
                                 big ? big_rows_per_round(N, swiglu, num_cus) : -1,
                                 large_tile_rows(rows_mode, cap, N, K, swiglu, num_cus, big));
}

}  // namespace moe

