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
#include <type_traits>

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

// BM rows x 128 output columns per tile.  SWIGLU: B tile = 128 gate + 128 up rows.
//
// K loop: NS = 3 LDS stages filled by direct global->LDS DMA (16 bytes per lane), two
// K blocks in flight while the third is multiplied.  Every wave issues the same number
// of DMA instructions per stage (A rows, B rows, one 64-lane scale load), so one
// s_waitcnt vmcnt per stage plus a barrier publishes the stage to all waves.
template <int BM, bool SWIGLU>
__global__ __launch_bounds__(256, 1) void gemm_fp8_kernel(GemmArgs args) {
  constexpr int NS = 3;
  constexpr int BN = 128;                         // output columns per tile
  constexpr int BNB = SWIGLU ? 2 * BN : BN;       // B rows per tile
  constexpr int WM = (BM >= 128) ? 2 : 1;         // wave grid
  constexpr int WN = 4 / WM;
  constexpr int WTM = BM / WM;                    // rows per wave
  constexpr int TM = WTM / 16;                    // 16-row MFMA tiles per wave
  constexpr int WCOL = BN / WN;                   // output columns per wave
  constexpr int TN = (SWIGLU ? 2 : 1) * WCOL / 16;  // 16-col MFMA tiles per wave
  constexpr int AR = BM < 32 ? 32 : BM;           // A rows loaded (BM 16: two copies)
  constexpr int A_IN = AR / 32;                   // DMA instructions per wave: A
  constexpr int B_IN = BNB / 32;                  //                            B
  constexpr int PER = A_IN + B_IN + 1;            //                 + one scale load
  constexpr int A_BYTES = AR * 128, B_BYTES = BNB * 128;
  constexpr int SC_OFF = A_BYTES + B_BYTES;       // 4 x 256 B of scale slots
  constexpr int STAGE = SC_OFF + 1024;
  static_assert(TM >= 1 && WCOL % 16 == 0, "tile shape");
  static_assert(PER < 16, "vmcnt encoding");

  __shared__ TileMap tm;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NS][STAGE];
  __shared__ float red[SWIGLU ? WN : 1][SWIGLU ? BM : 1];
  __shared__ int row_src[128];

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

    // source row of every tile row (gather through a_rows); rows past the group's end
    // repeat its last row, their results are discarded
    if (tid < 128) {
      int lr = min(row0 + (tid % BM), row_end - 1);
      int src = lr;
      if (args.a_rows) {
        int sr = args.a_rows[lr];
        src = sr < 0 ? 0 : sr / args.a_row_div;
      }
      row_src[tid] = src;
    }
    __syncthreads();

    // ---- this lane's DMA sources.  A wave instruction fills 1024 LDS bytes = 8 rows
    // of 128 B; lane L lands at row L/8, slot L%8 and fetches global piece
    // (L%8) ^ (row%8), which realises the XOR swizzle read back below.
    const int lr8 = lane >> 3, slot = lane & 7, piece = slot ^ lr8;
    const uint8_t* a_src[A_IN];
#pragma unroll
    for (int i = 0; i < A_IN; ++i) {
      const int row = (wid * A_IN + i) * 8 + lr8;              // 0 .. AR-1
      a_src[i] = args.A + (size_t)row_src[row % BM] * K + piece * 16;
    }
    const size_t nbrows = SWIGLU ? 2 * (size_t)N : (size_t)N;
    const uint8_t* b_src[B_IN];
#pragma unroll
    for (int i = 0; i < B_IN; ++i) {
      const int row = (wid * B_IN + i) * 8 + lr8;              // 0 .. BNB-1
      const int grow = SWIGLU ? (row < BN ? n0 + row : N + n0 + row - BN) : n0 + row;
      b_src[i] = args.B + ((size_t)g * nbrows + grow) * K + piece * 16;
    }
    // scale DMA: wave 0 -> sA rows 0..63, wave 1 -> sA rows 64..127, wave 2 -> sB
    // (lanes < 32 gate block, >= 32 up block), wave 3 -> a spare copy of sB
    const size_t nbk = nbrows / 128;
    const float* sc_src;
    if (wid < 2) {
      sc_src = args.sA + (size_t)row_src[(wid * 64 + lane) % BM] * KB;
    } else {
      const int nb = (SWIGLU && lane >= 32) ? (N + n0) / 128 : n0 / 128;
      sc_src = args.sB + ((size_t)g * nbk + nb) * KB;
    }

    // wave-uniform LDS byte address of this wave's first DMA slot in stage 0
    const uint32_t m_wave = __builtin_amdgcn_readfirstlane(lds_addr(&lds[0][0]) +
                                                           (uint32_t)wid * (A_IN * 1024));
    const uint32_t mb_wave = __builtin_amdgcn_readfirstlane(lds_addr(&lds[0][0]) + A_BYTES +
                                                            (uint32_t)wid * (B_IN * 1024));
    const uint32_t ms_wave = __builtin_amdgcn_readfirstlane(lds_addr(&lds[0][0]) + SC_OFF +
                                                            (uint32_t)wid * 256);
    auto issue = [&](int st, int kb) {
      const uint32_t so = (uint32_t)st * STAGE;
#pragma unroll
      for (int i = 0; i < A_IN; ++i) dma16(a_src[i] + (size_t)kb * 128, m_wave + so + i * 1024);
#pragma unroll
      for (int i = 0; i < B_IN; ++i) dma16(b_src[i] + (size_t)kb * 128, mb_wave + so + i * 1024);
      dma4(sc_src + kb, ms_wave + so);
    };

    v4f acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    // operand fragments of one K block, double-buffered in registers: the block after
    // the current one is read from LDS while the current one is multiplied
    const int gsel = 2 * (lane >> 4);
    v8i af[2][TM], bfr[2][TN];
    v4f sa[2][TM];
    float sb0[2], sb1[2];
    // buffer indices are compile-time constants so the fragments stay in registers
    auto read_frags = [&](auto BUF, int stg) {
      constexpr int buf = decltype(BUF)::value;
      const uint8_t* L = lds[stg];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = wm * WTM + i * 16 + (lane & 15);
        const uint8_t* base = L + row * 128;
        const v4i lo = *reinterpret_cast<const v4i*>(base + ((gsel ^ (row & 7)) << 4));
        const v4i hi = *reinterpret_cast<const v4i*>(base + (((gsel + 1) ^ (row & 7)) << 4));
        af[buf][i] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
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
        const uint8_t* base = L + A_BYTES + brow * 128;
        const v4i lo = *reinterpret_cast<const v4i*>(base + ((gsel ^ (brow & 7)) << 4));
        const v4i hi = *reinterpret_cast<const v4i*>(base + (((gsel + 1) ^ (brow & 7)) << 4));
        bfr[buf][j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
      const float* lsa = reinterpret_cast<const float*>(L + SC_OFF);
      const float* lsb = reinterpret_cast<const float*>(L + SC_OFF + 512);
#pragma unroll
      for (int i = 0; i < TM; ++i)
        sa[buf][i] = *reinterpret_cast<const v4f*>(&lsa[wm * WTM + i * 16 + (lane >> 4) * 4]);
      sb0[buf] = lsb[0];
      sb1[buf] = lsb[32];
    };

    // Pipeline: stages kb+1 and kb+2 are in flight (DMA) while block kb is multiplied
    // from registers and block kb+1 is read from LDS into the other register set.  The
    // K loop is unrolled by two so the register set of every block is static.
    issue(0, 0);
    if (KB > 1) issue(1, 1);
    if (KB > 2) issue(2, 2);
    if (KB > 2) wait_vmcnt<2 * PER>(); else if (KB > 1) wait_vmcnt<PER>(); else wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    read_frags(std::integral_constant<int, 0>{}, 0);
    int st = 0;  // stage of block kb
    auto kstep = [&](int kb, auto CUR) {
      constexpr int cur = decltype(CUR)::value;
      const int st1 = st == NS - 1 ? 0 : st + 1;   // stage of block kb+1
      // block kb's fragments are in registers; every wave must be done reading stage
      // st before it is refilled, and block kb+1 must have landed in stage st1
      __builtin_amdgcn_s_waitcnt(0xC07F);          // lgkmcnt(0)
      if (kb + 2 < KB) wait_vmcnt<PER>(); else wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      if (kb + 3 < KB) issue(st, kb + 3);
      if (kb + 1 < KB) read_frags(std::integral_constant<int, cur ^ 1>{}, st1);

      const v4f zero = {0.f, 0.f, 0.f, 0.f};
      v4f s0[TM], s1[TM];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        s0[i] = sa[cur][i] * sb0[cur];
        s1[i] = sa[cur][i] * sb1[cur];
      }
      // MFMA t into one partial while the previous partial is promoted
      v4f p[2];
#pragma unroll
      for (int t = 0; t <= TM * TN; ++t) {
        if (t < TM * TN) {
          const int i = t / TN, j = t % TN;
          p[t & 1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[cur][i], bfr[cur][j],
                                                                     zero, 0, 0, 0, 0, 0, 0);
        }
        if (t > 0) {
          const int i = (t - 1) / TN, j = (t - 1) % TN;
          const v4f sc = (SWIGLU && j >= TN / 2) ? s1[i] : s0[i];
          const v4f q = p[(t - 1) & 1];
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(sc[r], q[r], acc[i][j][r]);
        }
      }
      st = st1;
    };
    int kb = 0;
    for (; kb + 1 < KB; kb += 2) {
      kstep(kb, std::integral_constant<int, 0>{});
      kstep(kb + 1, std::integral_constant<int, 1>{});
    }
    if (kb < KB) kstep(kb, std::integral_constant<int, 0>{});

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
