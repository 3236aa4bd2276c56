// Grouped GEMM with int4 block weights and bf16 activations (W4A16).
//
// Weights are the block-wise 4-bit codes of the DeepSeek-V4 lecture (tqpw.cn sec.
// 3.1): one fp32 scale per output channel and 128-wide K block.  The stored codes
// travel from HBM to LDS untouched (a quarter of the bytes of bf16).  Each wave then
// expands the codes of its own weight rows in registers, right before the MFMA that
// consumes them, to bf16(fl32(q * s7)) by a byte-permute table lookup (below): the
// table holds the eight magnitudes' bf16(fl32(m * s7)), each computed with one fp32
// rounding and the hardware round-to-nearest-even bf16 conversion, so the lookup gives
// exactly the dequantised weight.  The 32x32x16 bf16 MFMA accumulates in fp32;
// the expansion runs on the vector ALU beside it, software-pipelined one step ahead.
//
// Tile: 128 rows x 256 weight rows (plain: 256 output columns, the last column tile
// possibly half used; SwiGLU: 128 gate + 128 up rows for 128 output columns).  Eight
// waves (two per SIMD, so one wave's expansion runs beside the other's MFMAs) side by
// side over the weight rows, each with all 128 rows and 32 weight rows: plain, 32
// consecutive rows; SwiGLU, 16 gate rows and the 16 up rows of the same output columns,
// so that one MFMA tile holds both and a lane swap pairs them in the epilogue.
// Gathered activation rows, packed codes and scales arrive by direct global->LDS DMA in
// three stages, in the same persistent, XCD-aware tile order as the FP8 kernel.
#include <type_traits>

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

// Codes of one row and 128-wide K block, as stored: 64 little-endian 32-bit words, word
// p holding k = 8p .. 8p+7 -- byte b carries k = 8p+b in its low nibble and k = 8p+4+b
// in its high nibble, each nibble sign (bit 3) and magnitude (bits 0-2, at most 7).
//
// Expansion by table: bf16(fl32(m * s)) for the eight magnitudes m is built once per row
// and K block and split into its low bytes (l0: m 0-3, l1: m 4-7) and high bytes (h0,
// h1).  A byte permute then looks up four codes at once; the sign goes into bit 15
// (bf16 of fl32(-m s) is the negated bf16 of fl32(m s)).
struct Tab {
  uint32_t l0, l1, h0, h1;
};

__device__ __forceinline__ uint32_t bf16x2(float a, float b) {
  typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
  const v2bf v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ Tab make_tab(float s) {
  // entries m = 2i (low half) and 2i + 1 (high half); fl32(m * s) by one rounding
  const uint32_t p0 = bf16x2(0.0f, s);
  const uint32_t p1 = bf16x2(2.0f * s, 3.0f * s);
  const uint32_t p2 = bf16x2(4.0f * s, 5.0f * s);
  const uint32_t p3 = bf16x2(6.0f * s, 7.0f * s);
  // perm(hi, lo, sel): result byte i = byte sel_i of the 8 bytes lo (0-3), hi (4-7)
  Tab t;
  t.l0 = __builtin_amdgcn_perm(p1, p0, 0x06040200u);
  t.l1 = __builtin_amdgcn_perm(p3, p2, 0x06040200u);
  t.h0 = __builtin_amdgcn_perm(p1, p0, 0x07050301u);
  t.h1 = __builtin_amdgcn_perm(p3, p2, 0x07050301u);
  return t;
}

// one code word -> the 8 bf16 weights of k = 8p .. 8p+7, in k order
__device__ __forceinline__ v8bf expand8(uint32_t w, const Tab& t) {
  const uint32_t m03 = w & 0x07070707u;
  const uint32_t m47 = (w >> 4) & 0x07070707u;
  const uint32_t l03 = __builtin_amdgcn_perm(t.l1, t.l0, m03);
  const uint32_t l47 = __builtin_amdgcn_perm(t.l1, t.l0, m47);
  const uint32_t h03 = __builtin_amdgcn_perm(t.h1, t.h0, m03) | ((w << 4) & 0x80808080u);
  const uint32_t h47 = __builtin_amdgcn_perm(t.h1, t.h0, m47) | (w & 0x80808080u);
  const v4i r = {(int)__builtin_amdgcn_perm(h03, l03, 0x05010400u),
                 (int)__builtin_amdgcn_perm(h03, l03, 0x07030602u),
                 (int)__builtin_amdgcn_perm(h47, l47, 0x05010400u),
                 (int)__builtin_amdgcn_perm(h47, l47, 0x07030602u)};
  return __builtin_bit_cast(v8bf, r);
}
// wait for this wave's LDS reads, then for the whole workgroup (a stage is refilled
// right after the barrier, so no read of it may still be in flight)
__device__ __forceinline__ void w4_lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
}  // namespace

template <bool SWIGLU>
__global__ __launch_bounds__(512, 1) void gemm_w4a16_kernel(W4Args args) {
  constexpr int BM = 128, BNB = 256;                // tile rows, weight rows per tile
  constexpr int BNO = SWIGLU ? 128 : 256;           // output columns per tile
  constexpr int NS = 3;                             // DMA stages
  constexpr int ROWB = 256;                         // A bytes per row per K block
  constexpr int NW = 8, NT = 512;
  constexpr int WR = BNB / NW;                      // weight rows per wave: 32
  constexpr int A_IN = BM * ROWB / 1024 / NW;       // A DMA instructions per wave: 4
  constexpr int B_IN = WR * 64 / 1024;              // code DMA instructions per wave: 2
  constexpr int PER_MAX = A_IN + B_IN + 1;          // + the scales (even waves)
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
  const int hf = lane >> 5, l32 = lane & 31;       // 32x32x16 MFMA operand: row l32, k half hf
  // XOR keys of the 16-byte pieces of an A row (256 B) and of a code row (64 B).  The LDS
  // (64 four-byte banks) serves a 16-byte read for lanes {0-7, 16-23}, {8-15, 24-31},
  // {32-39, 48-55}, {40-47, 56-63} together; those 16 lanes read rows r..r+7 and
  // r+16..r+23 at one piece index, and the keys send them to 16 different bank groups.
  auto akey = [](int row) { return (row & 7) | ((row >> 1) & 8); };
  auto ckey = [](int r) { return ((r >> 2) & 1) | ((r >> 3) & 2); };
  const int G = args.G, K = args.K, N = args.N, KB = K / 128;
  const int NBtot = SWIGLU ? 2 * N : N;
  const int tiles_n = (N + BNO - 1) / BNO;
  build_tile_map<BM, BM, NT>(tm, args.offsets, G);
  const int total = tm.start[G] * tiles_n;
  const int P = gridDim.x, b = blockIdx.x;
  const int v = (P % 8 == 0) ? (b % 8) * (P / 8) + b / 8 : b;
  const uint32_t lds0 = lds_addr(&lds[0][0]);

  // weight row of tile row r = 32 * wave + s: plain n0 + r (past N: repeats row N-1,
  // unused); SwiGLU gate rows n0 + 16 * wave + s (s < 16) and the up rows of the same
  // columns, N + n0 + 16 * wave + s - 16 (s >= 16)
  auto wrow = [&](int r, int n0) {
    if (!SWIGLU) return min(n0 + r, N - 1);
    const int w = r >> 5, s = r & 31;
    return s < 16 ? n0 + 16 * w + s : N + n0 + 16 * w + s - 16;
  };

  // one tile whose real rows lie in its first TM 32-row blocks
  auto run_tile = [&](auto TMC, int g, int row0, int n_valid, int n0) {
    constexpr int TM = decltype(TMC)::value;
    const int ncols = min(BNO, N - n0);            // plain N % 256 == 128: last tile half
    const bool wactive = SWIGLU || wid * WR < ncols;  // else: repeated rows, not stored

    // A: an instruction fills 4 rows of 256 B; lane L lands at row L/16, slot L%16 and
    // fetches 16-byte piece (L%16) ^ akey(row), the XOR swizzle read back below.
    const uint8_t* a_src[A_IN];
#pragma unroll
    for (int i = 0; i < A_IN; ++i) {
      const int row = (wid * A_IN + i) * 4 + (lane >> 4);
      a_src[i] = reinterpret_cast<const uint8_t*>(args.A + (size_t)row_src[row] * K) +
                 (((lane & 15) ^ akey(row)) << 4);
    }
    const int a_cnt = min(max((n_valid - wid * A_IN * 4 + 3) / 4, 0), A_IN);
    // codes: an instruction fills 16 weight rows of 64 B (row L/4, slot L%4, holding
    // piece (L%4) ^ ckey(row)); every wave fetches its own 32 rows, and each even wave
    // the 64 scales of its rows and the next wave's (one row per lane)
    const bool scales = (wid & 1) == 0;
    const int per = a_cnt + B_IN + (scales ? 1 : 0);
    const uint8_t* b_src[B_IN];
#pragma unroll
    for (int i = 0; i < B_IN; ++i) {
      const int r = wid * WR + i * 16 + (lane >> 2);
      b_src[i] = args.B + ((size_t)g * NBtot + wrow(r, n0)) * (K / 2) +
                 (((lane & 3) ^ ckey(r)) << 4);
    }
    const float* s_src =
        args.s7 + ((size_t)g * NBtot + wrow(min(wid * WR + lane, BNB - 1), n0)) * KB;
    const uint32_t m_a = lds0 + (uint32_t)wid * (A_IN * 1024);
    const uint32_t m_b = lds0 + BR_OFF + (uint32_t)wid * (B_IN * 1024);
    const uint32_t m_s = lds0 + SC_OFF + (uint32_t)wid * (WR * 4);
    // piece q of the copies of block kb into stage st (this wave's A rows, then its codes,
    // then the scales); pieces this wave does not have are skipped, so a block is `per`
    // copies for every wave
    auto issue_piece = [&](int st, int kb, int q) {
      const uint32_t so = (uint32_t)st * STAGE;
      if (q < A_IN) {
        if (q < a_cnt) dma16(a_src[q] + (size_t)kb * ROWB, m_a + so + q * 1024);
      } else if (q < A_IN + B_IN) {
        dma16(b_src[q - A_IN] + (size_t)kb * 64, m_b + so + (q - A_IN) * 1024);
      } else if (scales) {
        dma4(s_src + kb, m_s + so);
      }
    };
    auto issue = [&](int st, int kb) {
#pragma unroll
      for (int q = 0; q < PER_MAX; ++q) issue_piece(st, kb, q);
    };

    v16f acc[TM];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;

    // K loop: block j lives in stage j % 3.  At step 6 of block j the workgroup waits for
    // block j + 1 and meets at a barrier, after which stage j % 3 is free, and the wave
    // reads block j + 1's codes, scale table and first operands while block j's last
    // MFMAs run, so the next block starts with its operands in registers.  Block j + 3
    // goes into the freed stage one copy per step over steps 0-6 of block j + 1 (a burst
    // of a wave's copies stalls it until the vector memory unit takes them); it is waited
    // for at step 6 of block j + 2.
    issue(0, 0);
    if (KB > 1) issue(1, 1);
    if (KB > 2) issue(2, 2);
    wait_vmcnt_upto<2 * PER_MAX>((KB > 1 ? per : 0) + (KB > 2 ? per : 0));   // block 0 landed
    w4_lds_barrier();

    v4i raw[2];
    Tab tab;
    auto read_codes = [&](const uint8_t* L) {
      const int r = wid * WR + l32;
      const uint8_t* src = L + BR_OFF + r * 64;
      raw[0] = *reinterpret_cast<const v4i*>(src + (((2 * hf) ^ ckey(r)) << 4));
      raw[1] = *reinterpret_cast<const v4i*>(src + (((2 * hf + 1) ^ ckey(r)) << 4));
      tab = make_tab(reinterpret_cast<const float*>(L + SC_OFF)[r]);
    };
    auto expand_step = [&](int kk) { return expand8((uint32_t)raw[kk >> 2][kk & 3], tab); };
    // MFMA step kk takes k = 64 hf + 8 kk + e from lane (l32, hf): code word 8 hf + kk of
    // the weight row and 16-byte piece 8 hf + kk of the A row, one k order for both.
    auto read_step = [&](const uint8_t* L, int kk, v8bf* af) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int row = i * 32 + l32;
        af[i] = *reinterpret_cast<const v8bf*>(L + row * ROWB +
                                               (((8 * hf + kk) ^ akey(row)) << 4));
      }
    };
    // software pipeline over the 8 steps: while the TM MFMAs of step kk run, the wave
    // reads the A fragments of step kk + 2 (a ring of four, so a read has two steps to
    // land) and expands the weights of step kk + 1.  The block's last LDS reads are made
    // at step 5, so the barrier that publishes block kb + 1 sits at step 6; steps 6 and 7
    // read block kb + 1's codes, scale table and first two A fragments.
    v8bf af[4][TM], bf[2];
    read_codes(lds[0]);
    read_step(lds[0], 0, af[0]);
    read_step(lds[0], 1, af[1]);
    bf[0] = expand_step(0);
    int st = 0;
    for (int kb = 0; kb < KB; ++kb) {
      const uint8_t* L = lds[st];
      const int stn = st == NS - 1 ? 0 : st + 1;
      const int stp = st == 0 ? NS - 1 : st - 1;   // the stage block kb - 1 freed
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int c = kk & 1;
        if (kk < PER_MAX && kb >= 1 && kb + 2 < KB) issue_piece(stp, kb + 2, kk);
        if (kk < 6) {
          read_step(L, kk + 2, af[(kk + 2) & 3]);
          bf[c ^ 1] = expand_step(kk + 1);
        } else if (kk == 6) {
          bf[1] = expand_step(7);                  // the last use of this block's codes
          if (kb + 1 < KB) {
            wait_vmcnt_upto<PER_MAX>(kb + 2 < KB ? per : 0);              // block kb+1 landed
            w4_lds_barrier();
            read_codes(lds[stn]);
            read_step(lds[stn], 0, af[0]);
          }
        } else if (kb + 1 < KB) {
          bf[0] = expand_step(0);                  // block kb + 1, codes read at step 6
          read_step(lds[stn], 1, af[1]);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kk & 3][i], bf[c], acc[i], 0, 0,
                                                           0);
        // issue order: each MFMA followed by a share of the next steps' LDS reads and
        // expansion (left alone, the scheduler sinks them to their uses)
#pragma unroll
        for (int m = 0; m < TM; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);              // MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);              // DS read
          __builtin_amdgcn_sched_group_barrier(0x002, 15 / TM + 1, 0);    // VALU
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      st = stn;
    }

    // epilogue through LDS (stage buffers are idle): 16-byte row-contiguous stores
    __syncthreads();
    uint8_t* ot = &lds[0][0];
    constexpr int OB = BNO * 2;
    // accumulator element r of lane (l32, hf): row 8 (r / 4) + 4 hf + r % 4, column l32.
    // SwiGLU: columns 0-15 are gate rows, 16-31 the up rows of the same outputs; lane
    // l32 < 16 takes the up value from lane l32 + 16.
    if (wactive) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int trow = i * 32 + (r >> 2) * 8 + hf * 4 + (r & 3);
          if (SWIGLU) {
            // the up value of lane l32 < 16 sits in lane l32 + 16: a row swap on the
            // VALU (the second result holds, in lanes 0-15 and 32-47, the values of
            // lanes 16-31 and 48-63)
            const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc[i][r]),
                                                             __float_as_uint(acc[i][r]), false,
                                                             false);
            const float up = __uint_as_float(sw[1]);
            if (l32 < 16) {
              const int tcol = wid * 16 + l32;
              const float hv = silu_fast(acc[i][r]) * up;   // rounded to bf16 next
              *reinterpret_cast<uint16_t*>(ot + trow * OB + tcol * 2) = f32_to_bf16(hv);
            }
          } else {
            const int tcol = wid * WR + l32;
            *reinterpret_cast<uint16_t*>(ot + trow * OB + tcol * 2) = f32_to_bf16(acc[i][r]);
          }
        }
    }
    __syncthreads();
    const int CPR = ncols / 8;                     // 16-byte chunks per output row
    uint8_t* C = reinterpret_cast<uint8_t*>(args.C);
    for (int c = tid; c < n_valid * CPR; c += NT) {
      const int trow = c / CPR, ch = c % CPR;
      *reinterpret_cast<v4i*>(C + ((size_t)(row0 + trow) * N + n0) * 2 + ch * 16) =
          *reinterpret_cast<const v4i*>(ot + trow * OB + ch * 16);
    }
    __syncthreads();
  };

  for (int t = v; t < total; t += P) {
    const int g = find_group(tm, G, t, tiles_n);
    const int mt = tm.start[g + 1] - tm.start[g];
    const int local = t - tm.start[g] * tiles_n;
    const int ni = local / mt, mi = local % mt;
    const int row0 = tm.off[g] + mi * BM, row_end = tm.off[g + 1];
    const int n_valid = min(row_end - row0, BM);   // >= 1
    if (tid < BM) {
      int lr = min(row0 + tid, row_end - 1), src = lr;
      if (args.a_rows) {
        int sr = args.a_rows[lr];
        src = sr < 0 ? 0 : sr / args.a_row_div;
      }
      row_src[tid] = src;
    }
    __syncthreads();
    if (n_valid <= 32)
      run_tile(std::integral_constant<int, 1>{}, g, row0, n_valid, ni * BNO);
    else if (n_valid <= 64)
      run_tile(std::integral_constant<int, 2>{}, g, row0, n_valid, ni * BNO);
    else
      run_tile(std::integral_constant<int, 4>{}, g, row0, n_valid, ni * BNO);
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
    hipLaunchKernelGGL(gemm_w4a16_kernel<true>, dim3((unsigned)grid), dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL(gemm_w4a16_kernel<false>, dim3((unsigned)grid), dim3(512), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
