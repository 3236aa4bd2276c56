// Grouped GEMM with 4-bit expert weights on the FP8 matrix core (W4A8).
//
// The weights are the block-wise 4-bit codes of the DeepSeek-V4 lecture (tqpw.cn sec.
// 3.1, q = round(w / max|w| * 7) per output channel and 128-wide K block, one fp32
// scale s7 = max|w| / 7 per block) kept in memory as 4-bit codes: half the bytes of
// e4m3 weights.  The integers -7..7 are exact e4m3 values, so the kernel expands the
// codes in registers to e4m3 bytes and feeds the same 16x16x128 FP8 instruction as the
// e4m3 path, with the activations quantised 1x128 e4m3 as there.  Each 128-deep block's
// fp32 partial is promoted with the activation row's scale and the output channel's
// own weight scale: acc += sA[r, kb] * s7[n, kb] * partial.  The kernel is the template
// of gemm_fp8_kernel.hpp with W4 set; this file holds the offline packing into the
// fragment-major order it loads and the launcher.
#include <algorithm>

#include <cstdlib>

#include "gemm_fp8_kernel.hpp"

namespace moe {

// Codes q [G][R][K/2] (two per byte: byte 4p+b of a row holds k = 8p+b in its low nibble
// and k = 8p+4+b in its high nibble) -> qf [G][R/16][K/128][64][16 B], lane l of fragment
// (nb, kb) holding the 32 codes of row 16 nb + (l & 15), k = 128 kb + 32 (l >> 4) .. +32,
// i.e. bytes 64 kb + 16 (l >> 4) .. +16 of that row: the operand of one 16x16x128 MFMA as
// lane l supplies it, at half the bytes of the e4m3 fragment.
// Scales s7 [G][R][K/128] -> s7f [G][R/16][K/128][16]: the 16 rows of a fragment together.
__global__ void pack_weight_int4_kernel(const uint8_t* __restrict__ q, const float* __restrict__ s7,
                                        uint8_t* __restrict__ qf, float* __restrict__ s7f, int G,
                                        int R, int K) {
  const int KB = K / 128, R16 = R / 16;
  const size_t pieces = (size_t)G * R * KB * 4;    // 16-byte pieces of codes
  const size_t scales = (size_t)G * R * KB;
  for (size_t p = (size_t)blockIdx.x * blockDim.x + threadIdx.x; p < pieces + scales;
       p += (size_t)gridDim.x * blockDim.x) {
    if (p < pieces) {
      const int l = (int)(p % 64);
      size_t t = p / 64;
      const int kb = (int)(t % KB);
      t /= KB;
      const int nb = (int)(t % R16);
      const size_t g = t / R16;
      const int row = nb * 16 + (l & 15);
      const size_t src = (g * R + row) * (size_t)(K / 2) + (size_t)kb * 64 + 16 * (l >> 4);
      *reinterpret_cast<v4i*>(qf + p * 16) = *reinterpret_cast<const v4i*>(q + src);
    } else {
      const size_t e = p - pieces;
      const int i = (int)(e % 16);
      size_t t = e / 16;
      const int kb = (int)(t % KB);
      t /= KB;
      const int nb = (int)(t % R16);
      const size_t g = t / R16;
      s7f[e] = s7[(g * R + nb * 16 + i) * (size_t)KB + kb];
    }
  }
}

hipError_t launch_pack_weight_int4(const uint8_t* q, const float* s7, int G, int R, int K,
                                   uint8_t* qf, float* s7f, hipStream_t s) {
  const size_t items = (size_t)G * R * (K / 128) * 5;
  const size_t blocks = std::min<size_t>((items + 255) / 256, 16384);
  hipLaunchKernelGGL(pack_weight_int4_kernel, dim3((unsigned)blocks), dim3(256), 0, s, q, s7, qf,
                     s7f, G, R, K);
  return hipGetLastError();
}

hipError_t launch_gemm_w4a8(const uint8_t* A, const float* sA, const int32_t* a_rows,
                            int a_row_div, const uint8_t* Bf, const float* s7f,
                            const int32_t* offsets, int G, int R_cap, int N, int K, bool swiglu,
                            void* C, float* sC, int bm, int num_cus, hipStream_t s, int rows_mode,
                            int cap) {
  // groups of up to ~170 rows (the rows bound per group, R_cap / G, or the capacity):
  // 160-row tiles, one per group with less padding than 192 rows (hash W4A8 layer, ~128
  // rows per expert: 0.470 -> 0.428 ms, bit-identical); the FP8 GEMMs measured no gain
  // from them, so only this instance has them.  FP8GG_TILE_ROWS=160 forces them.
  int bmb = large_tile_rows(rows_mode, cap, N, K, swiglu, num_cus, false);
  const double rows_per_group =
      rows_mode == kRowsOffsets ? (double)R_cap / G : (double)cap;
  const char* e = std::getenv("FP8GG_TILE_ROWS");
  if (bmb == 192 && ((e && std::atoi(e) == 160) || (!e && rows_per_group <= 176)))
    bmb = 160;
  return launch_gemm_impl<true>(A, sA, a_rows, a_row_div, Bf, s7f, offsets, G, R_cap, N, K,
                                swiglu, C, sC, bm, num_cus, s, rows_mode, cap, -1, bmb);
}

}  // namespace moe
