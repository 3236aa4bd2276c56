// Grouped GEMM with int4 block weights and bf16 activations (W4A16).
//
// Weights are the block-wise 4-bit codes of the DeepSeek-V4 lecture (tqpw.cn sec.
// 3.1): one fp32 scale per output channel and 128-wide K block.  The stored codes
// travel from HBM to LDS untouched (a quarter of the bytes of bf16).  Each wave then
// expands the codes of its own weight rows in registers, right before the MFMA that
// consumes them, to bf16(fl32(q * s7)): byte-unpack, float conversion and one FMA
// u' * s7 - 8 * s7 with u' = q + 8 (exactly fl32(q * s7): 8 * s7 is exact and the FMA
// rounds once), then the hardware round-to-nearest-even bf16 conversion.  The 16x16x32
// bf16 MFMA accumulates in fp32; the expansion runs on the vector ALU beside it.
//
// Tile: 128 rows x 256 weight rows (plain: 256 output columns, the last column tile
// possibly half used; SwiGLU: 128 gate + 128 up rows for 128 output columns).  Four
// waves side by side over the weight rows, each with all 128 rows (64 weight rows per
// wave).  Gathered activation rows, packed codes
// and scales arrive by direct global->LDS DMA in three stages, in the same persistent,
// XCD-aware tile order as the FP8 kernel.
#include "common.hpp"
#include "dma.hpp"
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

// 8 int4 codes (two's complement nibbles, element 2b low / 2b+1 high nibble of byte b)
// -> 8 bf16 values bf16(fl32(q * s)), in k order; off = -8 s.
__device__ __forceinline__ v8bf expand8(uint32_t w, float s, float off) {
  const uint32_t lo = (w & 0x0F0F0F0Fu) ^ 0x08080808u;          // q + 8 of even k
  const uint32_t hi = ((w >> 4) & 0x0F0F0F0Fu) ^ 0x08080808u;   // q + 8 of odd k
  v8bf r;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    r[2 * b] = (__bf16)fmaf((float)((lo >> (8 * b)) & 0xFFu), s, off);
    r[2 * b + 1] = (__bf16)fmaf((float)((hi >> (8 * b)) & 0xFFu), s, off);
  }
  return r;
}
}  // namespace

template <bool SWIGLU>
__global__ __launch_bounds__(256, 1) void gemm_w4a16_kernel(W4Args args) {
  constexpr int BM = 128, BNB = 256;                // tile rows, weight rows per tile
  constexpr int BNO = SWIGLU ? 128 : 256;           // output columns per tile
  constexpr int NS = 3;                             // DMA stages
  constexpr int ROWB = 256;                         // A bytes per row per K block
  constexpr int TM = 8, TN = 4;                     // per wave: 128 rows x 64 weight rows
  constexpr int A_IN = BM * ROWB / 1024 / 4;        // A DMA instructions per wave: 8
  constexpr int B_IN = BNB * 64 / 1024 / 4;         // code DMA instructions per wave: 4
  constexpr int PER_MAX = A_IN + B_IN + 1;          // + the scales
  constexpr int A_BYTES = BM * ROWB;                // 32 KB
  constexpr int BR_OFF = A_BYTES;                   // codes: 256 rows x 64 B
  constexpr int SC_OFF = BR_OFF + BNB * 64;         // scales: 256 floats
  constexpr int STAGE = SC_OFF + BNB * 4;
  static_assert(PER_MAX < 64, "vmcnt range");

  __shared__ TileMap tm;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NS][STAGE];
  __shared__ int row_src[BM];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int q4 = lane >> 4, l16 = lane & 15;
  const int G = args.G, K = args.K, N = args.N, KB = K / 128;
  const int NBtot = SWIGLU ? 2 * N : N;
  const int tiles_n = (N + BNO - 1) / BNO;
  build_tile_map<BM>(tm, args.offsets, G);
  const int total = tm.start[G] * tiles_n;
  const int P = gridDim.x, b = blockIdx.x;
  const int v = (P % 8 == 0) ? (b % 8) * (P / 8) + b / 8 : b;
  const uint32_t lds0 = lds_addr(&lds[0][0]);

  // weight row of tile row r = 64 * wave + s: plain n0 + r (past N: repeats row N-1,
  // unused); SwiGLU gate rows n0 + 32 * wave + s (s < 32) and up rows
  // N + n0 + 32 * wave + s - 32 (s >= 32)
  auto wrow = [&](int r, int n0) {
    if (!SWIGLU) return min(n0 + r, N - 1);
    const int w = r >> 6, s = r & 63;
    return s < 32 ? n0 + 32 * w + s : N + n0 + 32 * w + s - 32;
  };

  for (int t = v; t < total; t += P) {
    const int g = find_group(tm, G, t, tiles_n);
    const int mt = tm.start[g + 1] - tm.start[g];
    const int local = t - tm.start[g] * tiles_n;
    const int ni = local / mt, mi = local % mt;
    const int row0 = tm.off[g] + mi * BM, row_end = tm.off[g + 1];
    const int n_valid = min(row_end - row0, BM);   // >= 1
    const int tmv = (n_valid + 15) >> 4;           // 16-row blocks with a real row
    const int n0 = ni * BNO;
    const int ncols = min(BNO, N - n0);            // plain N % 256 == 128: last tile half
    const bool wactive = SWIGLU || wid * 64 < ncols;
    if (tid < BM) {
      int lr = min(row0 + tid, row_end - 1), src = lr;
      if (args.a_rows) {
        int sr = args.a_rows[lr];
        src = sr < 0 ? 0 : sr / args.a_row_div;
      }
      row_src[tid] = src;
    }
    __syncthreads();

    // A: an instruction fills 4 rows of 256 B; lane L lands at row L/16, slot L%16 and
    // fetches 16-byte piece (L%16) ^ (row%16), the XOR swizzle read back below.
    const uint8_t* a_src[A_IN];
#pragma unroll
    for (int i = 0; i < A_IN; ++i) {
      const int row = (wid * A_IN + i) * 4 + q4;
      a_src[i] = reinterpret_cast<const uint8_t*>(args.A + (size_t)row_src[row] * K) +
                 ((l16 ^ (row & 15)) << 4);
    }
    const int a_cnt = min(max((n_valid - wid * A_IN * 4 + 3) / 4, 0), A_IN);
    const int per = a_cnt + B_IN + 1;
    // codes: an instruction fills 16 weight rows of 64 B (row L/4, piece L%4); every
    // wave fetches its own 64 rows and their 64 scales
    const uint8_t* b_src[B_IN];
#pragma unroll
    for (int i = 0; i < B_IN; ++i)
      b_src[i] = args.B + ((size_t)g * NBtot + wrow(wid * 64 + i * 16 + (lane >> 2), n0)) *
                              (K / 2) + (lane & 3) * 16;
    const float* s_src = args.s7 + ((size_t)g * NBtot + wrow(wid * 64 + lane, n0)) * KB;
    const uint32_t m_a = lds0 + (uint32_t)wid * (A_IN * 1024);
    const uint32_t m_b = lds0 + BR_OFF + (uint32_t)wid * (B_IN * 1024);
    const uint32_t m_s = lds0 + SC_OFF + (uint32_t)wid * 256;
    auto issue = [&](int st, int kb) {
      const uint32_t so = (uint32_t)st * STAGE;
#pragma unroll
      for (int i = 0; i < A_IN; ++i)
        if (i < a_cnt) dma16(a_src[i] + (size_t)kb * ROWB, m_a + so + i * 1024);
#pragma unroll
      for (int i = 0; i < B_IN; ++i) dma16(b_src[i] + (size_t)kb * 64, m_b + so + i * 1024);
      dma4(s_src + kb, m_s + so);
    };

    v4f acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    // K loop: buffers hold blocks kb, kb+1, kb+2; one barrier per block publishes block
    // kb and certifies that every wave is done with block kb-1, whose buffer is refilled.
    issue(0, 0);
    if (KB > 1) issue(1, 1);
    int st = 0;
    for (int kb = 0; kb < KB; ++kb) {
      wait_vmcnt_upto<PER_MAX>(kb + 1 < KB ? per : 0);
      __builtin_amdgcn_s_barrier();
      if (kb + 2 < KB) issue(st == 0 ? 2 : st - 1, kb + 2);
      const uint8_t* L = lds[st];
      // this lane's codes: weight row 64 * wave + 16 j + l16, k = 32 q4 .. 32 q4 + 31
      v4i raw[TN];
      float sc[TN], so[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int r = wid * 64 + j * 16 + l16;
        raw[j] = *reinterpret_cast<const v4i*>(L + BR_OFF + r * 64 + q4 * 16);
        sc[j] = reinterpret_cast<const float*>(L + SC_OFF)[r];
        so[j] = -8.0f * sc[j];
      }
      // fragment ks holds k = 8 * (4 q4 + ks) + e, for A and B alike
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        v8bf bf[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) bf[j] = expand8((uint32_t)raw[j][ks], sc[j], so[j]);
        const int piece = 4 * q4 + ks;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          if (wactive && i < tmv) {
            const int row = i * 16 + l16;
            const v8bf af =
                *reinterpret_cast<const v8bf*>(L + row * ROWB + ((piece ^ (row & 15)) << 4));
#pragma unroll
            for (int j = 0; j < TN; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, bf[j], acc[i][j], 0, 0, 0);
          }
        }
      }
      st = st == NS - 1 ? 0 : st + 1;
    }

    // epilogue through LDS (stage buffers are idle): 16-byte row-contiguous stores
    __syncthreads();
    uint8_t* ot = &lds[0][0];
    constexpr int OB = BNO * 2;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if (wactive && i < tmv) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int trow = i * 16 + q4 * 4 + r;
          if (SWIGLU) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const int tcol = wid * 32 + j * 16 + l16;
              const float hv = silu(acc[i][j][r]) * acc[i][j + 2][r];
              *reinterpret_cast<uint16_t*>(ot + trow * OB + tcol * 2) = f32_to_bf16(hv);
            }
          } else {
#pragma unroll
            for (int j = 0; j < TN; ++j) {
              const int tcol = wid * 64 + j * 16 + l16;
              *reinterpret_cast<uint16_t*>(ot + trow * OB + tcol * 2) = f32_to_bf16(acc[i][j][r]);
            }
          }
        }
      }
    }
    __syncthreads();
    const int CPR = ncols / 8;                     // 16-byte chunks per output row
    uint8_t* C = reinterpret_cast<uint8_t*>(args.C);
    for (int c = tid; c < n_valid * CPR; c += 256) {
      const int trow = c / CPR, ch = c % CPR;
      *reinterpret_cast<v4i*>(C + ((size_t)(row0 + trow) * N + n0) * 2 + ch * 16) =
          *reinterpret_cast<const v4i*>(ot + trow * OB + ch * 16);
    }
    __syncthreads();
  }
}

hipError_t launch_gemm_w4a16(const uint16_t* A, const int32_t* a_rows, int a_row_div,
                             const uint8_t* B, const float* s7, const int32_t* offsets, int G,
                             int R_cap, int N, int K, bool swiglu, uint16_t* C, int num_cus,
                             hipStream_t s) {
  W4Args a{A, a_rows, a_row_div, B, s7, offsets, G, N, K, C};
  const long tiles_n = swiglu ? N / 128 : (N + 255) / 256;
  const long mtiles = R_cap / 128 + G;
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
