// Grouped FP8 GEMM for gfx950: C[rows of g] = A[rows of g] . B[g]^T with e4m3 operands,
// 1x128 activation scales and 128x128 weight scales.
//
// What it computes (MegaMoE walkthrough, discosf.com sec. 3.2): groups differ in M
// and share N and K; a global tile scheduler flattens every group's row tiles into
// one list so small and large groups keep the machine busy.  Each 128-deep K block
// is reduced by the FP8 matrix core into a fresh fp32 partial and then promoted into
// the fp32 accumulator with its two scales (the two-level accumulation of DeepGEMM's
// release notes, qidao123.com day 3).  The output is rounded to bf16 (RNE, walkthrough
// sec. 3.3) or, with the SwiGLU epilogue, silu(gate)*up is requantised to e4m3 1x128
// in registers (epilogue fusion, walkthrough sec. 3.2).
//
// gfx950 mapping
//   * v_mfma_f32_16x16x128_f8f6f4: one instruction covers one 16x16 output tile over
//     exactly one 128-deep scale block, so promotion is one fp32 FMA per output per
//     block: acc += (sA*sB) * mfma(a, b, 0).
//   * 256 threads = 4 wave64s; workgroup tile BM x 128 output columns; a SwiGLU tile
//     loads 128 gate rows and 128 up rows of B so the 1x128 requant block is complete
//     inside one workgroup.
//   * Operands are staged through LDS with a 16-byte XOR swizzle (row stride 128 B);
//     the next K block is fetched into registers while the current one is multiplied.
//   * Persistent grid: workgroup b works on tiles v, v+P, v+2P, ... where
//     v = (b mod 8) * P/8 + b/8, so consecutive tiles -- the row tiles that share one
//     B column tile -- run on the same XCD and share its L2.
#include "common.hpp"
#include "launch.hpp"
#include "tiles.hpp"

namespace moe {

namespace {
struct GemmArgs {
  const uint8_t* A;
  const float* sA;
  const int32_t* a_rows;
  int a_row_div;
  const uint8_t* B;
  const float* sB;
  const int32_t* offsets;
  int G;
  int N;  // output columns
  int K;
  void* C;
  float* sC;
};
}  // namespace

// BM rows x 128 output columns per tile.  SWIGLU: B tile = 128 gate + 128 up rows.
template <int BM, bool SWIGLU>
__global__ __launch_bounds__(256, 1) void gemm_fp8_kernel(GemmArgs args) {
  constexpr int BN = 128;                         // output columns per tile
  constexpr int BNB = SWIGLU ? 2 * BN : BN;       // B rows per tile
  constexpr int WM = (BM >= 128) ? 2 : 1;         // wave grid
  constexpr int WN = 4 / WM;
  constexpr int WTM = BM / WM;                    // rows per wave
  constexpr int TM = WTM / 16;                    // 16-row MFMA tiles per wave
  constexpr int WCOL = BN / WN;                   // output columns per wave
  constexpr int TN = (SWIGLU ? 2 : 1) * WCOL / 16;  // 16-col MFMA tiles per wave
  constexpr int A_PIECES = BM * 8, B_PIECES = BNB * 8;
  constexpr int NA = (A_PIECES + 255) / 256, NB = B_PIECES / 256;
  constexpr int STAGE = (BM + BNB) * 128;         // bytes of operands per stage
  static_assert(TM >= 1 && WCOL % 16 == 0, "tile shape");

  __shared__ TileMap tm;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][STAGE];
  __shared__ __attribute__((aligned(16))) float lds_sa[2][BM];
  __shared__ float lds_sb[2][2];
  __shared__ float red[SWIGLU ? WN : 1][SWIGLU ? BM : 1];
  __shared__ int row_src[BM];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WN, wn = wid % WN;
  const int G = args.G, K = args.K, N = args.N, KB = K / 128;
  const int tiles_n = N / BN;

  build_tile_map<BM>(tm, args.offsets, G);
  const int total = tm.start[G] * tiles_n;
  const int P = gridDim.x;
  const int b = blockIdx.x;
  const int v = (P % 8 == 0) ? (b % 8) * (P / 8) + b / 8 : b;

  for (int t = v; t < total; t += P) {
    // ---- locate the tile
    const int g = find_group(tm, G, t, tiles_n);
    const int mt = tm.start[g + 1] - tm.start[g];
    const int local = t - tm.start[g] * tiles_n;
    const int ni = local / mt, mi = local % mt;
    const int row0 = tm.off[g] + mi * BM;
    const int row_end = tm.off[g + 1];
    const int n0 = ni * BN;

    // source row of every tile row (gather through a_rows)
    for (int r = tid; r < BM; r += 256) {
      int lr = min(row0 + r, row_end - 1);
      int src = lr;
      if (args.a_rows) {
        int sr = args.a_rows[lr];
        src = sr < 0 ? 0 : sr / args.a_row_div;
      }
      row_src[r] = src;
    }
    __syncthreads();

    // ---- per-thread global pointers and LDS slots
    const uint8_t* a_ptr[NA];
    const uint8_t* b_ptr[NB];
    int a_lds[NA], b_lds[NB];
    bool a_on[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      int c = tid + i * 256;
      a_on[i] = c < A_PIECES;
      int row = (c >> 3) % BM, piece = c & 7;
      a_ptr[i] = args.A + (size_t)row_src[row] * K + piece * 16;
      a_lds[i] = row * 128 + ((piece ^ (row & 7)) << 4);
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      int c = tid + i * 256;
      int row = c >> 3, piece = c & 7;
      int grow = SWIGLU ? (row < BN ? n0 + row : N + n0 + row - BN) : n0 + row;
      b_ptr[i] = args.B + ((size_t)g * (SWIGLU ? 2 * N : N) + grow) * K + piece * 16;
      b_lds[i] = BM * 128 + row * 128 + ((piece ^ (row & 7)) << 4);
    }
    const float* sa_ptr = args.sA + (size_t)row_src[tid < BM ? tid : 0] * KB;
    const size_t nbk = (size_t)(SWIGLU ? 2 * N : N) / 128;
    const float* sbg_ptr = args.sB + ((size_t)g * nbk + n0 / 128) * KB;
    const float* sbu_ptr = SWIGLU ? args.sB + ((size_t)g * nbk + (N + n0) / 128) * KB : sbg_ptr;

    v4i ra[NA], rb[NB];
    float rsa = 0.f, rsb0 = 0.f, rsb1 = 0.f;
    auto fetch = [&](int kb) {
#pragma unroll
      for (int i = 0; i < NA; ++i)
        if (a_on[i]) ra[i] = *reinterpret_cast<const v4i*>(a_ptr[i] + (size_t)kb * 128);
#pragma unroll
      for (int i = 0; i < NB; ++i) rb[i] = *reinterpret_cast<const v4i*>(b_ptr[i] + (size_t)kb * 128);
      if (tid < BM) rsa = sa_ptr[kb];
      if (tid == 0) { rsb0 = sbg_ptr[kb]; rsb1 = sbu_ptr[kb]; }
    };

    v4f acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    fetch(0);
    for (int kb = 0; kb < KB; ++kb) {
      const int st = kb & 1;
      uint8_t* L = lds[st];
#pragma unroll
      for (int i = 0; i < NA; ++i)
        if (a_on[i]) *reinterpret_cast<v4i*>(L + a_lds[i]) = ra[i];
#pragma unroll
      for (int i = 0; i < NB; ++i) *reinterpret_cast<v4i*>(L + b_lds[i]) = rb[i];
      if (tid < BM) lds_sa[st][tid] = rsa;
      if (tid == 0) { lds_sb[st][0] = rsb0; lds_sb[st][1] = rsb1; }
      __syncthreads();
      if (kb + 1 < KB) fetch(kb + 1);

      // operands of this wave
      const int gsel = 2 * (lane >> 4);
      v8i af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        int row = wm * WTM + i * 16 + (lane & 15);
        const uint8_t* base = L + row * 128;
        v4i lo = *reinterpret_cast<const v4i*>(base + ((gsel ^ (row & 7)) << 4));
        v4i hi = *reinterpret_cast<const v4i*>(base + (((gsel + 1) ^ (row & 7)) << 4));
        af[i] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        int brow;
        if (SWIGLU) {
          const int half = j / (TN / 2), jj = j % (TN / 2);
          brow = half * BN + wn * WCOL + jj * 16 + (lane & 15);
        } else {
          brow = wn * WCOL + j * 16 + (lane & 15);
        }
        const uint8_t* base = L + BM * 128 + brow * 128;
        v4i lo = *reinterpret_cast<const v4i*>(base + ((gsel ^ (brow & 7)) << 4));
        v4i hi = *reinterpret_cast<const v4i*>(base + (((gsel + 1) ^ (brow & 7)) << 4));
        bfr[j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
      // promotion scales: sA of this lane's 4 rows in each row tile times sB
      const float sb0 = lds_sb[st][0], sb1 = lds_sb[st][1];
      v4f sa[TM];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        sa[i] = *reinterpret_cast<const v4f*>(&lds_sa[st][wm * WTM + i * 16 + (lane >> 4) * 4]);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const v4f s0 = sa[i] * sb0;
        const v4f s1 = sa[i] * sb1;
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const v4f zero = {0.f, 0.f, 0.f, 0.f};
          v4f p = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i], bfr[j], zero, 0, 0, 0,
                                                                  0, 0, 0);
          const v4f s = (SWIGLU && j >= TN / 2) ? s1 : s0;
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(s[r], p[r], acc[i][j][r]);
        }
      }
    }

    // ---- epilogue.  MFMA C layout: lane holds column lane%16, rows 4*(lane/16)+r.
    if constexpr (!SWIGLU) {
      uint16_t* C = static_cast<uint16_t*>(args.C);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = row0 + wm * WTM + i * 16 + (lane >> 4) * 4 + r;
          if (row < row_end) {
#pragma unroll
            for (int j = 0; j < TN; ++j) {
              const int col = n0 + wn * WCOL + j * 16 + (lane & 15);
              C[(size_t)row * N + col] = f32_to_bf16(acc[i][j][r]);
            }
          }
        }
    } else {
      constexpr int TH = TN / 2;
      float h[TM][TH][4];
      float rmax[TM][4];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float m = 0.f;
#pragma unroll
          for (int j = 0; j < TH; ++j) {
            h[i][j][r] = silu(acc[i][j][r]) * acc[i][j + TH][r];
            m = fmaxf(m, fabsf(h[i][j][r]));
          }
          rmax[i][r] = group_max<16>(m);  // across the 16 columns of the MFMA tile
        }
      if ((lane & 15) == 0) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            red[wn][wm * WTM + i * 16 + (lane >> 4) * 4 + r] = rmax[i][r];
      }
      __syncthreads();
      uint8_t* C = static_cast<uint8_t*>(args.C);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int trow = wm * WTM + i * 16 + (lane >> 4) * 4 + r;
          float m = red[0][trow];
#pragma unroll
          for (int w = 1; w < WN; ++w) m = fmaxf(m, red[w][trow]);
          const float s = block_scale(m);
          const int row = row0 + trow;
          if (row < row_end) {
#pragma unroll
            for (int j = 0; j < TH; ++j) {
              const int col = n0 + wn * WCOL + j * 16 + (lane & 15);
              C[(size_t)row * N + col] = (uint8_t)(e4m3x2(clamp448(h[i][j][r] / s), 0.f) & 0xFF);
            }
            if (wn == 0 && (lane & 15) == 0) args.sC[(size_t)row * (N / 128) + n0 / 128] = s;
          }
        }
    }
    __syncthreads();  // LDS (row_src, red, stages) is reused by the next tile
  }
}

static int g_num_cus = 0;

hipError_t launch_gemm_fp8(const uint8_t* A, const float* sA, const int32_t* a_rows, int a_row_div,
                           const uint8_t* B, const float* sB, const int32_t* offsets, int G,
                           int R_cap, int N, int K, bool swiglu, void* C, float* sC, int bm,
                           int num_cus, hipStream_t s) {
  GemmArgs a{A, sA, a_rows, a_row_div, B, sB, offsets, G, N, K, C, sC};
  const long tiles_n = N / 128;
  const long mtiles = R_cap / bm + G;
  long grid = std::min<long>(mtiles * tiles_n, (long)num_cus);
  if (grid >= 8) grid = grid / 8 * 8;
  if (grid < 1) grid = 1;
  dim3 gd((unsigned)grid), bd(256);
#define MOE_GEMM_CASE(BMV, SW)                                                   \
  hipLaunchKernelGGL((gemm_fp8_kernel<BMV, SW>), gd, bd, 0, s, a);
  if (swiglu) {
    switch (bm) {
      case 16: MOE_GEMM_CASE(16, true); break;
      case 32: MOE_GEMM_CASE(32, true); break;
      case 64: MOE_GEMM_CASE(64, true); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (bm) {
      case 16: MOE_GEMM_CASE(16, false); break;
      case 32: MOE_GEMM_CASE(32, false); break;
      case 64: MOE_GEMM_CASE(64, false); break;
      case 128: MOE_GEMM_CASE(128, false); break;
      default: return hipErrorInvalidValue;
    }
  }
#undef MOE_GEMM_CASE
  (void)g_num_cus;
  return hipGetLastError();
}

}  // namespace moe
