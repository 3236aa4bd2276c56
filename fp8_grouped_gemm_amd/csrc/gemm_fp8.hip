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
//   * 512 threads = 8 wave64s (two per SIMD) over a BM x BNB tile (BNB rows of B).
//     Prefill tiles are 128 x 256 with 64 x 64 per wave, so one weight byte brought
//     into LDS feeds 128 token rows and every fragment read from LDS feeds 4 MFMAs.  A SwiGLU tile
//     loads 128 gate rows and 128 up rows of B so the 1x128 requant block is complete
//     inside one workgroup.
//   * Operands reach LDS by direct global->LDS DMA into 3 buffers (two K blocks in
//     flight), in a 16-byte XOR swizzle (row stride 128 B) read back conflict-free.
//     Row groups past the end of the group are not fetched and waves whose rows are all
//     padding skip their MFMAs, so small groups cost little more than their weights.
//   * Persistent grid: workgroup b works on tiles v, v+P, v+2P, ... where
//     v = (b mod 8) * P/8 + b/8, so consecutive tiles -- the row tiles that share one
//     B column tile -- run on the same XCD and share its L2.
#include <type_traits>

#include "common.hpp"
#include "launch.hpp"
#include "tiles.hpp"
#include "dma.hpp"

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
  int mode, cap;  // GroupRows of the tile map and its C (masked) or M (dense)
};
}  // namespace

// Two tile classes share one persistent tile list: groups with at most BMS rows are
// cut into BMS-row tiles worked by 8 waves side by side (all SIMDs busy, the weight
// stream dominates), larger groups into 128-row tiles worked by 2 x 4 waves (a weight
// byte in LDS feeds 128 rows).  B tile: BNB rows (SWIGLU: BNB/2 gate + BNB/2 up rows ->
// BNB/2 output columns; plain: BNB output columns).  Eight waves, two per SIMD, so that
// one wave's MFMAs cover the other's LDS reads and promotion arithmetic.
template <int BMS, int BNB, bool SWIGLU>
__global__ __launch_bounds__(512, 1) void gemm_fp8_kernel(GemmArgs args) {
  constexpr int NT = 512, NW = 8;
  constexpr int NS = 3;
  constexpr int BMB = 128;                         // rows of a big-group tile
  constexpr int BN_OUT = SWIGLU ? BNB / 2 : BNB;   // output columns per tile
  constexpr int B_IN = BNB / 8 / NW;               // B DMA instructions per wave (8 rows each)
  constexpr int A_IN_MAX = BMB / 8 / NW;           // A DMA instructions per wave, at most
  constexpr int PER_MAX = A_IN_MAX + B_IN + 1;     // + one scale load
  constexpr int A_BYTES = BMB * 128, B_BYTES = BNB * 128;
  constexpr int SC_OFF = A_BYTES + B_BYTES;        // 4 x 256 B of scale slots
  constexpr int STAGE = SC_OFF + 1024;
  static_assert(!SWIGLU || BN_OUT == 128, "1x128 requant block");
  static_assert(B_IN >= 1 && A_IN_MAX >= 1 && PER_MAX < 16, "DMA split");

  __shared__ TileMap tm;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NS][STAGE];
  __shared__ float red[SWIGLU ? 512 : 1];          // SwiGLU row maxima [wn][row]
  __shared__ int row_src[128];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = args.G, K = args.K, N = args.N, KB = K / 128;
  const int tiles_n = N / BN_OUT;

  build_tile_map<BMS, BMB, NT>(tm, args.offsets, G, args.mode, args.cap);
  const int total = tm.start[G] * tiles_n;
  const int P = gridDim.x;
  const int b = blockIdx.x;
  const int v = (P % 8 == 0) ? (b % 8) * (P / 8) + b / 8 : b;
  const uint32_t lds0 = lds_addr(&lds[0][0]);
  const int lr8 = lane >> 3, slot = lane & 7;
  // 16-byte piece p of row r sits in slot p ^ swz(r) of the row's 128 LDS bytes; pairs
  // of rows share a 256-byte bank line, so the key changes every second row
  auto swz = [](int r) { return (r >> 1) & 7; };
  const int gsel = 2 * (lane >> 4);

  // one tile of class BM (WM waves along M)
  auto run_tile = [&](auto BMC, int g, int row0, int row_end, int n0) {
    constexpr int BM = decltype(BMC)::value;
    constexpr int WM = BM == BMB ? 2 : 1;
    constexpr int WN = NW / WM;
    constexpr int WTM = BM / WM;                   // rows per wave
    constexpr int TM = WTM / 16;                   // 16-row MFMA tiles per wave
    constexpr int WTN = BNB / WN;                  // B rows per wave
    constexpr int TN = WTN / 16;                   // 16-col MFMA tiles per wave
    constexpr int AR = BM < 32 ? 32 : BM;          // A rows in LDS (BM 16: rows repeat)
    constexpr int NA = AR / 8;                     // A DMA instructions (8 rows each)
    static_assert(TM >= 1 && TN >= 1 && (!SWIGLU || TN % 2 == 0), "tile shape");
    const int wm = wid / WN, wn = wid % WN;
    const int n_valid = min(row_end - row0, BM);   // >= 1

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
    // (L%8) ^ swz(row), which realises the XOR swizzle read back below.  A row group q
    // (rows 8q .. 8q+7) is fetched by wave q % 8.
    const uint8_t* a_src[A_IN_MAX];
#pragma unroll
    for (int i = 0; i < A_IN_MAX; ++i) {
      const int row = ((wid + NW * i) * 8 + lr8) % AR;
      a_src[i] = args.A + (size_t)row_src[row % BM] * K + (slot ^ swz(row)) * 16;
    }
    // row groups holding at least one real row; the rest are never fetched
    const int groups = min((min(n_valid, AR) + 7) / 8, NA);
    const int a_cnt = min(max((groups - wid + NW - 1) / NW, 0), A_IN_MAX);
    const bool has_sc = wid < 3;                    // waves 0/1: sA rows, wave 2: sB
    const int per = a_cnt + B_IN + (has_sc ? 1 : 0); // DMA instructions per stage
    const size_t nbrows = SWIGLU ? 2 * (size_t)N : (size_t)N;
    const uint8_t* b_src[B_IN];
#pragma unroll
    for (int i = 0; i < B_IN; ++i) {
      const int row = (wid * B_IN + i) * 8 + lr8;               // 0 .. BNB-1
      const int grow = SWIGLU ? (row < BN_OUT ? n0 + row : N + n0 + row - BN_OUT) : n0 + row;
      b_src[i] = args.B + ((size_t)g * nbrows + grow) * K + (slot ^ swz(row)) * 16;
    }
    // scale DMA: waves 0/1 -> sA rows 0..63 / 64..127; wave 2 -> sB, lanes < 32 the
    // first B column block of the tile, lanes >= 32 the second (SwiGLU: gate / up)
    const size_t nbk = nbrows / 128;
    const float* sc_src;
    if (wid < 2) {
      sc_src = args.sA + (size_t)row_src[(wid * 64 + lane) % BM] * KB;
    } else {
      int nb = n0 / 128;
      if (lane >= 32) nb = SWIGLU ? (N + n0) / 128 : min(n0 / 128 + 1, (int)nbk - 1);
      sc_src = args.sB + ((size_t)g * nbk + nb) * KB;
    }
    const uint32_t m_a = lds0 + (uint32_t)wid * 1024;
    const uint32_t m_b = lds0 + A_BYTES + (uint32_t)wid * (B_IN * 1024);
    const uint32_t m_s = lds0 + SC_OFF + (uint32_t)min(wid, 2) * 256;
    auto issue = [&](int st, int kb) {
      const uint32_t so = (uint32_t)st * STAGE;
#pragma unroll
      for (int i = 0; i < A_IN_MAX; ++i)
        if (i < a_cnt) dma16(a_src[i] + (size_t)kb * 128, m_a + so + i * (NW * 1024));
#pragma unroll
      for (int i = 0; i < B_IN; ++i) dma16(b_src[i] + (size_t)kb * 128, m_b + so + i * 1024);
      if (has_sc) dma4(sc_src + kb, m_s + so);
    };

    v4f acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    const bool active = wm * WTM < n_valid;          // wave has a real row
    // small tiles: 16-row blocks holding a real row; the rest are neither read nor
    // multiplied (their results are never stored).  Large tiles run every block (a
    // branch per block costs them more than the rare partial tile saves).
    const int tmv = BM == BMB ? TM : min(TM, max((n_valid - wm * WTM + 15) / 16, 0));

    // K loop: buffers hold blocks kb, kb+1, kb+2 (NS = 3); while block kb is
    // multiplied, kb+1 and kb+2 are in flight.  One barrier per block: it publishes
    // block kb and certifies every wave is done with block kb-1, whose buffer is refilled.
    issue(0, 0);
    if (KB > 1) issue(1, 1);
    int st = 0;
    for (int kb = 0; kb < KB; ++kb) {
      wait_vmcnt_upto<PER_MAX>(kb + 1 < KB ? per : 0);
      __builtin_amdgcn_s_barrier();
      if (kb + 2 < KB) issue(st == 0 ? 2 : st - 1, kb + 2);    // buffer (kb+2) % 3
      if (active) {
        const uint8_t* L = lds[st];
        const float* lsa = reinterpret_cast<const float*>(L + SC_OFF);
        const float* lsb = reinterpret_cast<const float*>(L + SC_OFF + 512);
        v8i af[TM];
        auto read_a = [&](int i) {
          const int row = wm * WTM + i * 16 + (lane & 15);
          const uint8_t* base = L + row * 128;
          const v4i lo = *reinterpret_cast<const v4i*>(base + ((gsel ^ swz(row)) << 4));
          const v4i hi = *reinterpret_cast<const v4i*>(base + (((gsel + 1) ^ swz(row)) << 4));
          af[i] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        };
        auto read_b = [&](int j) {
          int brow;
          if (SWIGLU) {
            const int half = j / (TN / 2), jj = j % (TN / 2);
            brow = half * BN_OUT + wn * (WTN / 2) + jj * 16 + (lane & 15);
          } else {
            brow = wn * WTN + j * 16 + (lane & 15);
          }
          const uint8_t* base = L + A_BYTES + brow * 128;
          const v4i lo = *reinterpret_cast<const v4i*>(base + ((gsel ^ swz(brow)) << 4));
          const v4i hi = *reinterpret_cast<const v4i*>(base + (((gsel + 1) ^ swz(brow)) << 4));
          return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        };
        // promotion scales: sA of this lane's 4 rows per row tile times sB of the
        // column block (plain: this wave's block; SwiGLU: gate for j < TN/2, up after)
        const float sbA = SWIGLU ? lsb[0] : lsb[wn * WTN >= 128 ? 32 : 0];
        const float sbB = lsb[32];
        v4f sa[TM];
#pragma unroll
        for (int i = 0; i < TM; ++i)
          sa[i] = *reinterpret_cast<const v4f*>(&lsa[wm * WTM + i * 16 + (lane >> 4) * 4]);
        // the A fragments stay in registers; B column tiles stream through two register
        // sets, the next one read while the current one is multiplied
        v8i bcur = read_b(0);
#pragma unroll
        for (int i = 0; i < TM; ++i)
          if (i < tmv) read_a(i);
        const v4f zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const v8i bnext = (j + 1 < TN) ? read_b(j + 1) : bcur;
          const float sb = (SWIGLU && j >= TN / 2) ? sbB : sbA;
          v4f pp[TM];
#pragma unroll
          for (int i = 0; i < TM; ++i)
            if (i < tmv)
              pp[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(af[i], bcur, zero, 0, 0,
                                                                      0, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < TM; ++i) {
            if (i >= tmv) continue;
            const v4f sc = sa[i] * sb;
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = fmaf(sc[r], pp[i][r], acc[i][j][r]);
          }
          bcur = bnext;
        }
      }
      st = st == NS - 1 ? 0 : st + 1;
    }

    // ---- epilogue.  MFMA C layout: lane holds column lane%16, rows 4*(lane/16)+r.  The
    // tile is staged through LDS (every DMA has landed, the stage buffers are free) so
    // that global stores are 16 contiguous bytes per lane.
    uint8_t* ot = &lds[0][0];
    if constexpr (!SWIGLU) {
      constexpr int OB = BNB * 2;                    // bytes per staged row
      __syncthreads();
      if (active) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int trow = wm * WTM + i * 16 + (lane >> 4) * 4 + r;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
              const int tcol = wn * WTN + j * 16 + (lane & 15);
              *reinterpret_cast<uint16_t*>(ot + trow * OB + tcol * 2) = f32_to_bf16(acc[i][j][r]);
            }
          }
      }
      __syncthreads();
      uint8_t* C = static_cast<uint8_t*>(args.C);
      constexpr int CPR = OB / 16;                   // 16-byte chunks per row
      for (int c = tid; c < n_valid * CPR; c += NT) {
        const int trow = c / CPR, ch = c % CPR;
        *reinterpret_cast<v4i*>(C + ((size_t)(row0 + trow) * N + n0) * 2 + ch * 16) =
            *reinterpret_cast<const v4i*>(ot + trow * OB + ch * 16);
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
            h[i][j][r] = silu_fast(acc[i][j][r]) * acc[i][j + TH][r];
            m = fmaxf(m, fabsf(h[i][j][r]));
          }
          rmax[i][r] = group_max<16>(m);  // across the 16 columns of the MFMA tile
        }
      if ((lane & 15) == 0) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            red[wn * BM + wm * WTM + i * 16 + (lane >> 4) * 4 + r] = rmax[i][r];
      }
      __syncthreads();
      if (active) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int trow = wm * WTM + i * 16 + (lane >> 4) * 4 + r;
            float m = red[trow];
#pragma unroll
            for (int w = 1; w < WN; ++w) m = fmaxf(m, red[w * BM + trow]);
            const float s = block_scale(m);
            const float inv = 1.0f / s;
#pragma unroll
            for (int j = 0; j < TH; ++j) {
              const int tcol = wn * (WTN / 2) + j * 16 + (lane & 15);
              ot[trow * 128 + tcol] = (uint8_t)(e4m3x2(clamp448(h[i][j][r] * inv), 0.f) & 0xFF);
            }
            const int row = row0 + trow;
            if (wn == 0 && (lane & 15) == 0 && row < row_end)
              args.sC[(size_t)row * (N / 128) + n0 / 128] = s;
          }
      }
      __syncthreads();
      uint8_t* C = static_cast<uint8_t*>(args.C);
      for (int c = tid; c < n_valid * 8; c += NT) {
        const int trow = c / 8, ch = c % 8;
        *reinterpret_cast<v4i*>(C + (size_t)(row0 + trow) * N + n0 + ch * 16) =
            *reinterpret_cast<const v4i*>(ot + trow * 128 + ch * 16);
      }
    }
    __syncthreads();  // LDS (row_src, red, stages) is reused by the next tile
  };

  for (int t = v; t < total; t += P) {
    // ---- locate the tile
    const int g = find_group(tm, G, t, tiles_n);
    const int mt = tm.start[g + 1] - tm.start[g];
    const int local = t - tm.start[g] * tiles_n;
    const int ni = local / mt, mi = local % mt;
    const int rows = group_rows(tm, g), r0 = group_row0(tm, g);
    const int n0 = ni * BN_OUT;
    if (rows <= BMS)
      run_tile(std::integral_constant<int, BMS>{}, g, r0 + mi * BMS, r0 + rows, n0);
    else
      run_tile(std::integral_constant<int, BMB>{}, g, r0 + mi * BMB, r0 + rows, n0);
  }
}

hipError_t launch_gemm_fp8(const uint8_t* A, const float* sA, const int32_t* a_rows, int a_row_div,
                           const uint8_t* B, const float* sB, const int32_t* offsets, int G,
                           int R_cap, int N, int K, bool swiglu, void* C, float* sC, int bm,
                           int num_cus, hipStream_t s, int rows_mode, int cap) {
  GemmArgs a{A, sA, a_rows, a_row_div, B, sB, offsets, G, N, K, C, sC, rows_mode, cap};
  const bool wide = !swiglu && N % 256 == 0;      // 256 output columns per plain tile
  const long tiles_n = swiglu ? N / 128 : (wide ? N / 256 : N / 128);
  const long mtiles = R_cap / (bm < 128 ? bm : 64) + G;
  long grid = std::min<long>(mtiles * tiles_n, (long)num_cus);
  if (grid >= 8) grid = grid / 8 * 8;
  if (grid < 1) grid = 1;
  dim3 gd((unsigned)grid), bd(512);
  // bm: tile rows of small groups (16, 32 or 64); groups above it use 128-row tiles
  const int bms = bm >= 64 ? 64 : bm;
#define MOE_GEMM_CASE(BMSV, BNBV, SW) \
  hipLaunchKernelGGL((gemm_fp8_kernel<BMSV, BNBV, SW>), gd, bd, 0, s, a)
  if (swiglu) {
    switch (bms) {
      case 16: MOE_GEMM_CASE(16, 256, true); break;
      case 32: MOE_GEMM_CASE(32, 256, true); break;
      case 64: MOE_GEMM_CASE(64, 256, true); break;
      default: return hipErrorInvalidValue;
    }
  } else if (wide) {
    switch (bms) {
      case 16: MOE_GEMM_CASE(16, 256, false); break;
      case 32: MOE_GEMM_CASE(32, 256, false); break;
      case 64: MOE_GEMM_CASE(64, 256, false); break;
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (bms) {
      case 16: MOE_GEMM_CASE(16, 128, false); break;
      case 32: MOE_GEMM_CASE(32, 128, false); break;
      case 64: MOE_GEMM_CASE(64, 128, false); break;
      default: return hipErrorInvalidValue;
    }
  }
#undef MOE_GEMM_CASE
  return hipGetLastError();
}

}  // namespace moe
