// Grouped GEMM with int4 block weights and bf16 activations (W4A16).
//
// Weights are the block-wise 4-bit codes of the DeepSeek-V4 lecture (tqpw.cn sec.
// 3.1): one fp32 scale per output channel and 128-wide K block.  They are expanded
// in-kernel, on their way from HBM into LDS, to bf16(fl32(q * s7)) and fed with the
// bf16 activations to the 16x16x32 bf16 MFMA with fp32 accumulation; no promotion
// step is needed because the scale is applied before the product.
//
// Tile: 64 rows x 128 B rows (plain: 128 output columns; SwiGLU: 64 gate + 64 up rows
// for 64 output columns); 4 waves side by side over the B rows.  The same persistent,
// XCD-aware tile order as the FP8 kernel.
#include "common.hpp"
#include "launch.hpp"
#include "tiles.hpp"

namespace moe {

namespace {
struct W4Args {
  const uint16_t* A;
  const int32_t* a_rows;
  int a_row_div;
  const uint8_t* B;
  const float* s7;
  const int32_t* offsets;
  int G, N, K;
  uint16_t* C;
};
}  // namespace

template <bool SWIGLU>
__global__ __launch_bounds__(256, 1) void gemm_w4a16_kernel(W4Args args) {
  constexpr int BM = 64, BNB = 128;                 // tile rows, B rows per tile
  constexpr int BNO = SWIGLU ? 64 : 128;            // output columns per tile
  constexpr int ROWB = 256;                          // LDS bytes per row (128 bf16)
  constexpr int TM = 4, TN = 2;                      // per wave: 64 rows x 32 B rows
  __shared__ TileMap tm;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][(BM + BNB) * ROWB];
  __shared__ int row_src[BM];

  const int tid = threadIdx.x, lane = tid & 63, wn = tid >> 6;
  const int G = args.G, K = args.K, N = args.N, KB = K / 128;
  const int NBtot = SWIGLU ? 2 * N : N;
  const int tiles_n = N / BNO;
  build_tile_map<BM>(tm, args.offsets, G);
  const int total = tm.start[G] * tiles_n;
  const int P = gridDim.x, b = blockIdx.x;
  const int v = (P % 8 == 0) ? (b % 8) * (P / 8) + b / 8 : b;

  for (int t = v; t < total; t += P) {
    const int g = find_group(tm, G, t, tiles_n);
    const int mt = tm.start[g + 1] - tm.start[g];
    const int local = t - tm.start[g] * tiles_n;
    const int ni = local / mt, mi = local % mt;
    const int row0 = tm.off[g] + mi * BM, row_end = tm.off[g + 1];
    const int n0 = ni * BNO;
    for (int r = tid; r < BM; r += 256) {
      int lr = min(row0 + r, row_end - 1), src = lr;
      if (args.a_rows) {
        int sr = args.a_rows[lr];
        src = sr < 0 ? 0 : sr / args.a_row_div;
      }
      row_src[r] = src;
    }
    __syncthreads();
    // A: 64 rows x 16 pieces of 16 B -> 4 per thread.  B: 128 rows x 4 pieces of 16 B
    // (32 int4 codes each) -> 2 per thread.
    const uint16_t* a_ptr[4];
    int a_lds[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int c = tid + i * 256, row = c >> 4, piece = c & 15;
      a_ptr[i] = args.A + (size_t)row_src[row] * K + piece * 8;
      a_lds[i] = row * ROWB + ((piece ^ (row & 15)) << 4);
    }
    const uint8_t* b_ptr[2];
    const float* s_ptr[2];
    int b_row[2], b_sub[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      int c = tid + i * 256, row = c >> 2, sub = c & 3;
      int grow = SWIGLU ? (row < 64 ? n0 + row : N + n0 + row - 64) : n0 + row;
      b_ptr[i] = args.B + ((size_t)g * NBtot + grow) * (K / 2) + sub * 16;
      s_ptr[i] = args.s7 + ((size_t)g * NBtot + grow) * KB;
      b_row[i] = row;
      b_sub[i] = sub;
    }
    v4i ra[4], rb[2];
    float rs[2];
    auto fetch = [&](int kb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) ra[i] = *reinterpret_cast<const v4i*>(a_ptr[i] + (size_t)kb * 128);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        rb[i] = *reinterpret_cast<const v4i*>(b_ptr[i] + (size_t)kb * 64);
        rs[i] = s_ptr[i][kb];
      }
    };
    v4f acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    fetch(0);
    for (int kb = 0; kb < KB; ++kb) {
      uint8_t* L = lds[kb & 1];
#pragma unroll
      for (int i = 0; i < 4; ++i) *reinterpret_cast<v4i*>(L + a_lds[i]) = ra[i];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int row = b_row[i];
        uint8_t* brow = L + BM * ROWB + row * ROWB;
#pragma unroll
        for (int u = 0; u < 4; ++u) {           // 8 codes per dword -> one 16-byte piece
          const uint32_t word = (uint32_t)rb[i][u];
          uint32_t packed[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            int q0 = (int)((word >> (8 * e)) & 0xF);
            int q1 = (int)((word >> (8 * e + 4)) & 0xF);
            q0 = q0 > 7 ? q0 - 16 : q0;
            q1 = q1 > 7 ? q1 - 16 : q1;
            const uint32_t h0 = f32_to_bf16((float)q0 * rs[i]);
            const uint32_t h1 = f32_to_bf16((float)q1 * rs[i]);
            packed[e] = h0 | (h1 << 16);
          }
          const int piece = b_sub[i] * 4 + u;
          *reinterpret_cast<v4i*>(brow + ((piece ^ (row & 15)) << 4)) =
              v4i{(int)packed[0], (int)packed[1], (int)packed[2], (int)packed[3]};
        }
      }
      __syncthreads();
      if (kb + 1 < KB) fetch(kb + 1);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const int piece = ks * 4 + (lane >> 4);
        v8bf af[TM], bf[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          int row = i * 16 + (lane & 15);
          af[i] = *reinterpret_cast<const v8bf*>(L + row * ROWB + ((piece ^ (row & 15)) << 4));
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          int brow = SWIGLU ? j * 64 + wn * 16 + (lane & 15) : wn * 32 + j * 16 + (lane & 15);
          bf[j] = *reinterpret_cast<const v8bf*>(L + BM * ROWB + brow * ROWB +
                                                 ((piece ^ (brow & 15)) << 4));
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
      }
    }
    // epilogue (C layout: column lane%16, rows 4*(lane/16)+r)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = row0 + i * 16 + (lane >> 4) * 4 + r;
        if (row >= row_end) continue;
        if (SWIGLU) {
          const int col = n0 + wn * 16 + (lane & 15);
          args.C[(size_t)row * N + col] = f32_to_bf16(silu(acc[i][0][r]) * acc[i][1][r]);
        } else {
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const int col = n0 + wn * 32 + j * 16 + (lane & 15);
            args.C[(size_t)row * N + col] = f32_to_bf16(acc[i][j][r]);
          }
        }
      }
    __syncthreads();
  }
}

hipError_t launch_gemm_w4a16(const uint16_t* A, const int32_t* a_rows, int a_row_div,
                             const uint8_t* B, const float* s7, const int32_t* offsets, int G,
                             int R_cap, int N, int K, bool swiglu, uint16_t* C, int num_cus,
                             hipStream_t s) {
  W4Args a{A, a_rows, a_row_div, B, s7, offsets, G, N, K, C};
  const long tiles_n = N / (swiglu ? 64 : 128);
  const long mtiles = R_cap / 64 + G;
  long grid = std::min<long>(mtiles * tiles_n, (long)num_cus);
  if (grid >= 8) grid = grid / 8 * 8;
  if (grid < 1) grid = 1;
  if (swiglu)
    hipLaunchKernelGGL(gemm_w4a16_kernel<true>, dim3((unsigned)grid), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(gemm_w4a16_kernel<false>, dim3((unsigned)grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
