// Grouped FP8 GEMM, 256 x 256 tiles, for the MFMA-bound part of a grouped GEMM.
//
// Same computation as gemm_fp8_kernel (MegaMoE walkthrough, discosf.com sec. 3.2:
// groups differ in M and share N and K; each 128-deep K block reduced by the FP8
// matrix core into a fresh fp32 partial and promoted with its two scales, the
// two-level accumulation of qidao123.com day 3), for the whole 256-row tiles of large
// groups.  Why a second kernel: in the 128 x 256 tiles of gemm_fp8_kernel every CU pulls
// 48 KB of operands per 128-deep block for 1024 cycles of matrix work, near what a CU's
// vector memory path takes in (about 40-45 B per cycle for 16-byte-per-lane loads); a
// 256 x 256 tile pulls 64 KB for 2048 cycles of matrix work.  Measured on MI355X it is
// nevertheless slower than the 128-row kernel, so callers get it only on request.
//
// gfx950 mapping
//   * 512 threads = 8 waves, two per SIMD, as a 2 x 4 grid: wave (wr, wc) computes tile
//     rows wr*128 .. +128 against weight rows wc*64 .. +64 (SwiGLU: gate rows wc*32 .. +32
//     and the up rows of the same output columns), 32 MFMA tiles of 16 x 16 per block,
//     128 accumulator registers.
//   * Both operands reach LDS by direct global->LDS DMA, two stages of 64 KB: the
//     activation rows (gathered through a_rows, 16-byte XOR swizzle as in
//     gemm_fp8_kernel), the tile's 16 fragment-major weight fragments (2 KB each, in the
//     order the MFMA takes them) and the rows' scales of the block.  The tile's two
//     weight-scale rows for every K block are copied to LDS once per tile.
//   * The barrier that publishes block kb+1 sits at step 28 of block kb's 32 MFMA steps
//     (the block's last LDS read of its own stage is at step 24); steps 29-31 refill each
//     weight fragment right after its last use and read block kb+1's first activation
//     fragment, so a block starts with its operands in registers.  The copies of block
//     kb+2 go out one piece per step after that barrier, into the stage it freed.  They
//     are issued as inline asm and the kernel waits for them itself (vmcnt(0) before each
//     publishing barrier): they are the only vector memory operations in the loop.
//   * Each MFMA's partial is promoted one step behind, after the next MFMA has been
//     issued, with the row scale times the weight-block scale.
//   * Tiles: only whole 256-row tiles, and only whole rounds of the grid (big_cut: the
//     rest goes to gemm_fp8_kernel, launched after this one with the same cut).  Runs of
//     two row tiles are walked column tile by column tile, so the 32 tiles one XCD holds
//     at a time share their K slices in that XCD's L2.
#include <algorithm>

#include "common.hpp"
#include "dma.hpp"
#include "launch.hpp"
#include "tiles.hpp"

namespace moe {

namespace {
struct BigArgs {
  const uint8_t* A;
  const float* sA;
  const int32_t* a_rows;
  int a_row_div;
  const uint8_t* Bf;  // fragment-major weights
  const int32_t* offsets;
  int G, N, K;
  void* C;
  float* sC;
  int mode, cap;      // GroupRows of the tile map and its C (masked) or M (dense)
  int rpr;            // row tiles per round (big_cut)
};

constexpr int BG_HALF = 128 * 128;   // one 128-row half of a stage's activation rows
constexpr int BG_B = 16 * 2048;      // the tile's 16 weight fragments
constexpr int kBigDmaPerBlock = 9;   // copy instructions per wave per K block (4 A, 4 B, 1 scale)

// Buffer descriptor of a raw byte buffer at base with no size limit (stride 0,
// 0xFFFFFFFF records): offsets are 32-bit.
__device__ __forceinline__ v4i big_rsrc(const void* base) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return v4i{(int)(uint32_t)a, (int)((a >> 32) & 0xFFFFu), -1, 0x00020000};
}
// global->LDS DMA through a buffer descriptor: lane L's SIZE bytes from
// base + voff + soff + OFS land at lds_dst + OFS + SIZE * L (the instruction's immediate
// offset moves both addresses).  Written as inline asm, so the compiler does not count
// it: the kernel waits for its copies itself (vmcnt(0) before each barrier that
// publishes a stage), and a compiler-inserted wait before a read of the other stage
// would stall the loop.
template <int SIZE, int OFS = 0>
__device__ __forceinline__ void big_dma(v4i rs, uint32_t voff, uint32_t soff, void* lds_dst) {
  static_assert((SIZE == 16 || SIZE == 4) && (OFS == 0 || OFS == 1024), "big_dma form");
  const uint32_t m = lds_addr(lds_dst);
  if constexpr (SIZE == 4)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                 :: "s"(m), "v"(voff), "s"(rs), "s"(soff) : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\t"
                 "buffer_load_dwordx4 %1, %2, %3 offen offset:%4 lds"
                 :: "s"(m), "v"(voff), "s"(rs), "s"(soff), "i"(OFS) : "memory", "m0");
}

__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ void big_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
}  // namespace

template <bool SWIGLU>
__global__ __launch_bounds__(512, 1) void gemm_fp8_big_kernel(BigArgs args,
                                                               const float* __restrict__ sB) {
  constexpr int NT = 512;
  constexpr int BN_OUT = SWIGLU ? 128 : 256;       // output columns per tile
  __shared__ int goff[kMaxGroups + 1];
  __shared__ int bpre[kMaxGroups + 1];
  __shared__ int row_src[kBigRows];
  __shared__ __attribute__((aligned(1024))) uint8_t a0[2 * BG_HALF];   // two 128-row halves
  __shared__ __attribute__((aligned(1024))) uint8_t a1[2 * BG_HALF];
  __shared__ __attribute__((aligned(1024))) uint8_t b0[BG_B];
  __shared__ __attribute__((aligned(1024))) uint8_t b1[BG_B];
  __shared__ __attribute__((aligned(1024))) float s0[kBigRows];
  __shared__ __attribute__((aligned(1024))) float s1[kBigRows];
  __shared__ float wsc[2][kGemmMaxKBlocks];       // the tile's two weight-scale rows
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wr = wid >> 2, wc = wid & 3;
  const int G = args.G, K = args.K, N = args.N, KB = K / 128;
  const int tiles_n = N / BN_OUT;
  const int R = SWIGLU ? 2 * N : N;                // weight rows per group
  const int R16 = R / 16, RB = R / 128;
  auto swz = [](int r) {                           // as gemm_fp8_kernel
    const int k = (r >> 1) & 3;
    return (k & 1) | ((k & 2) << 1);
  };

  // Loop-invariant LDS read addresses of this lane, per stage: its activation rows
  // (row 16 i + lane % 16 of the wave's half sits at +2048 i: the swizzle depends on
  // lane % 16 only), its weight fragments (fixed offsets from the first) and its row
  // scales (+64 i bytes).
  const int l15 = lane & 15;
  const int a_lo = l15 * 128 + (((2 * (lane >> 4)) ^ swz(l15)) << 4);
  const int a_hi = a_lo ^ 16;                      // the next 16-byte K piece
  const int fb = SWIGLU ? 2 * wc : 4 * wc;         // first weight fragment of the wave
  // (an offset into one object per stage: a select between objects would hide from the
  // compiler which stage a read touches, and it would wait for the copies into the other)
  const uint8_t* const la_lo[2] = {a0 + wr * BG_HALF + a_lo, a1 + wr * BG_HALF + a_lo};
  const uint8_t* const la_hi[2] = {a0 + wr * BG_HALF + a_hi, a1 + wr * BG_HALF + a_hi};
  const uint8_t* const lb[2] = {b0 + fb * 2048 + lane * 16, b1 + fb * 2048 + lane * 16};
  const float* const ls[2] = {s0 + wr * 128 + l15, s1 + wr * 128 + l15};
  // fragment j of the wave relative to its first (SwiGLU: two gate then two up fragments)
  auto fofs = [](int j) { return SWIGLU ? (j < 2 ? j : 8 + (j - 2)) : j; };

  // group rows and the prefix of their whole 256-row tiles
  const int mode = args.mode, cap = args.cap;
  for (int i = tid; i <= G; i += NT) {
    if (mode == kRowsOffsets) goff[i] = args.offsets[i];
    else if (mode == kRowsMasked) goff[i] = i < G ? min(max(args.offsets[i], 0), cap) : 0;
    else goff[i] = i == 0 ? 0 : cap;
  }
  __syncthreads();
  auto grow0 = [&](int g) { return mode == kRowsMasked ? g * cap : goff[g]; };
  auto grows = [&](int g) { return mode == kRowsMasked ? goff[g] : goff[g + 1] - goff[g]; };
  group_prefix<NT>(bpre, G, [&](int g) { return grows(g) / kBigRows; });
  const int cut = big_cut(bpre[G], args.rpr);
  const int ntiles = cut * tiles_n;
  const int P = gridDim.x, b = blockIdx.x;
  const int v = (P % 8 == 0) ? (b % 8) * (P / 8) + b / 8 : b;
  const v4i rs_a = big_rsrc(args.A), rs_s = big_rsrc(args.sA);

  auto run_tile = [&](int g, int row0, int n0) {
    if (tid < kBigRows) {
      const int lr = row0 + tid;
      int src = lr;
      if (args.a_rows) {
        const int sr = args.a_rows[lr];
        src = sr < 0 ? 0 : sr / args.a_row_div;
      }
      row_src[tid] = src;
    }
    // the weight-block scales of the tile's two 128-row weight blocks (plain: columns
    // n0 .. +128 and +128 .. +256; SwiGLU: the gate and the up block) for every K block
    for (int t = tid; t < 2 * KB; t += NT) {
      const int h = t >= KB ? 1 : 0, kbt = t - h * KB;
      const int wrow = SWIGLU ? (h ? (N + n0) / 128 : n0 / 128) : n0 / 128 + h;
      wsc[h][kbt] = sB[((size_t)g * RB + wrow) * KB + kbt];
    }
    __syncthreads();

    // ---- copies of one block.  Activations: instruction q of a wave fills rows
    // 8 (wid + 8 q) .. +8 (lane L: row L/8, slot L%8, global piece (L%8) ^ swz(row)).
    // Weights: instruction q copies half q%2 of fragment 2 wid + q/2 (the K step and the
    // fragment in the scalar offset).  Row scales: one 64-row quarter per wave (waves 4-7
    // repeat waves 0-3: same bytes, same place).
    uint32_t a_voff[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = (wid + 8 * q) * 8 + (lane >> 3), slot = lane & 7;
      a_voff[q] = (uint32_t)row_src[row] * (uint32_t)K + ((slot ^ swz(row)) << 4);
    }
    const v4i rs_b = big_rsrc(args.Bf + (size_t)g * R16 * (size_t)KB * 2048);
    uint32_t b_soff[2];
#pragma unroll
    for (int f2 = 0; f2 < 2; ++f2) {
      const int f = 2 * wid + f2;
      const int nb = SWIGLU ? (f < 8 ? n0 / 16 + f : N / 16 + n0 / 16 + (f - 8)) : n0 / 16 + f;
      b_soff[f2] = (uint32_t)__builtin_amdgcn_readfirstlane(nb * KB * 2048);
    }
    const uint32_t b_voff = lane * 16;
    const uint32_t s_voff = (uint32_t)row_src[(wid & 3) * 64 + lane] * (uint32_t)KB * 4u;
    // piece q (0-8) of the copies of block kb into stage S
    auto dma_piece = [&](auto S, int kb, int q) {
      constexpr int st = decltype(S)::value % 2;
      uint8_t* ah = (st == 0 ? a0 : a1) + (q >> 1) * BG_HALF + (wid + 8 * (q & 1)) * 1024;
      uint8_t* bd = (st == 0 ? b0 : b1) + 2 * wid * 2048 + ((q - 4) >> 1) * 2048;
      const uint32_t kbw = (uint32_t)kb * 2048u;
      switch (q) {
        case 0: case 1: case 2: case 3:
          big_dma<16>(rs_a, a_voff[q], (uint32_t)kb * 128u, ah);
          break;
        case 4: case 6:
          big_dma<16, 0>(rs_b, b_voff, b_soff[(q - 4) >> 1] + kbw, bd);
          break;
        case 5: case 7:                            // the fragment's second half
          big_dma<16, 1024>(rs_b, b_voff, b_soff[(q - 4) >> 1] + kbw, bd);
          break;
        default:
          big_dma<4>(rs_s, s_voff, (uint32_t)kb * 4u, (st == 0 ? s0 : s1) + (wid & 3) * 64);
      }
      asm volatile("" ::: "memory");
    };
    auto dma = [&](auto S, int kb) {
#pragma unroll
      for (int q = 0; q < kBigDmaPerBlock; ++q) dma_piece(S, kb, q);
    };

    // the wave's weight-scale row (a wave's columns lie in one 128-row weight block)
    const float* wsA = wsc[SWIGLU ? 0 : (wc >> 1)];
    const float* wsB = wsc[SWIGLU ? 1 : (wc >> 1)];

    v4f acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
    const v4f zero = {0.f, 0.f, 0.f, 0.f};

    auto rd_a = [&](int st, int i) {
      const v4i lo = *reinterpret_cast<const v4i*>(la_lo[st] + i * 2048);
      const v4i hi = *reinterpret_cast<const v4i*>(la_hi[st] + i * 2048);
      return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };
    auto rd_b = [&](int st, int j) {
      const v4i lo = *reinterpret_cast<const v4i*>(lb[st] + fofs(j) * 2048);
      const v4i hi = *reinterpret_cast<const v4i*>(lb[st] + fofs(j) * 2048 + 1024);
      return v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    };

    // operands in registers: the block's 4 weight fragments, a ring of 2 activation
    // fragments with their row scales, the block's weight scales
    v8i bf[4], af[2];
    float sa[2], wA, wB;
    v4f pp[2];

    // One block in stage S.  Its last activation fragment is read at step 24; at step 28
    // the workgroup waits for the copies of block kb + 1 (into the other stage) and
    // meets at a barrier, after which no wave reads stage S any more, so the copies of
    // block kb + 2 go out into it.  Steps 29-31 read block kb + 1's first activation
    // fragment and refill each weight fragment right after its last use, so the next
    // block starts with its operands in registers.  (The last block reads the idle
    // stage in the same way; those values are not used.)
    auto body = [&](auto S, int kb) {
      constexpr int st = decltype(S)::value % 2, nx = st ^ 1;
      const bool has_next = kb + 1 < KB, has_next2 = kb + 2 < KB;
      const int kbn = has_next ? kb + 1 : kb;
      float wAn = 0.f, wBn = 0.f;
      float cpA = 0.f, cpB = 0.f;                  // scales of the previous row fragment
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float cA = sa[i & 1] * wA, cB = SWIGLU ? sa[i & 1] * wB : cA;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int s = i * 4 + j;
          if (s == 28 && has_next) {
            wait_vmcnt<0>();
            big_barrier();
          }
          // The copies of a block go out one piece at a time (a burst of them stalls the
          // issuing wave until the vector memory unit takes them): pieces 0 and 1 of block
          // kb + 2 after the barrier at step 28, pieces 2-8 of block kb + 1 at steps 0, 2,
          // .., 12 (block 1 went out whole before the loop).  All land before step 28.
          if ((s == 28 || s == 30) && has_next2)
            dma_piece(std::integral_constant<int, st>{}, kb + 2, (s - 28) / 2);
          if (s <= 12 && (s & 1) == 0 && kb >= 1 && has_next)
            dma_piece(std::integral_constant<int, nx>{}, kb + 1, 2 + s / 2);
          // weights as the A operand: a lane holds four consecutive output columns of
          // one output row (the transposed 16x16 tile)
          pp[s & 1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af[i & 1], zero, 0,
                                                                        0, 0, 0, 0, 0);
          if (s > 0) {
            const int ip = (s - 1) >> 2, jp = (s - 1) & 3;
            // the previous partial is promoted after this MFMA has been issued (it then
            // runs under this one instead of waiting for its own result)
            asm volatile("" : "+v"(pp[(s - 1) & 1]) : "v"(pp[s & 1]));
            const float c = j == 0 ? ((SWIGLU && jp >= 2) ? cpB : cpA)
                                   : ((SWIGLU && jp >= 2) ? cB : cA);
#pragma unroll
            for (int r = 0; r < 4; ++r)
              acc[ip][jp][r] = fmaf(c, pp[(s - 1) & 1][r], acc[ip][jp][r]);
            // the promotion happens here, not sunk below the block's last MFMA (which
            // would hold all 32 partials at once)
            asm volatile("" : "+v"(acc[ip][jp]));
          }
          if (j == 0 && i < 7) {                   // next activation fragment of this block
            af[(i + 1) & 1] = rd_a(st, i + 1);
            sa[(i + 1) & 1] = ls[st][(i + 1) * 16];
          }
          if (i == 7 && j == 1) {                  // block kb + 1: first activation fragment
            af[0] = rd_a(nx, 0);
            sa[0] = ls[nx][0];
            wAn = wsA[kbn];
            wBn = SWIGLU ? wsB[kbn] : wAn;
          }
          if (i == 7 && j >= 1) bf[j - 1] = rd_b(nx, j - 1);
          // nothing moves across steps (the scheduler would otherwise hoist every
          // fragment read of the block and run out of registers)
          __builtin_amdgcn_sched_barrier(0);
        }
        cpA = cA;
        cpB = cB;
      }
      bf[3] = rd_b(nx, 3);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[7][3][r] = fmaf(cpB, pp[1][r], acc[7][3][r]);
      wA = wAn;
      wB = wBn;
    };

    // prologue: blocks 0 and 1 (KB is even, so at least 2) into the two stages
    dma(std::integral_constant<int, 0>{}, 0);
    dma(std::integral_constant<int, 1>{}, 1);
    wait_vmcnt<kBigDmaPerBlock>();                 // block 0 landed
    big_barrier();
#pragma unroll
    for (int j = 0; j < 4; ++j) bf[j] = rd_b(0, j);
    af[0] = rd_a(0, 0);
    sa[0] = ls[0][0];
    wA = wsA[0];
    wB = SWIGLU ? wsB[0] : wA;
    for (int kb = 0; kb < KB; kb += 2) {           // KB is even (checked by the launcher)
      body(std::integral_constant<int, 0>{}, kb);
      body(std::integral_constant<int, 1>{}, kb + 1);
    }
    // every wave is done with both stages (the epilogue stages its output in them)
    big_barrier();

    // ---- epilogue, one 128-row half at a time through the (idle) weight stages: rows of
    // 256 bytes whose 16-byte chunks are XOR-swizzled by row
    auto chunk_at = [](uint8_t* base, int row, int chunk) {
      return base + row * 256 + ((chunk ^ (row & 15)) << 4);
    };
    // the thread index seen through an opaque copy: the epilogue's addresses are then
    // computed here, not hoisted out of the tile loop and held through the K loop
    const int et = opaque(tid), el = et & 63;
    // the outputs in registers first (bf16 pairs, or fp32 silu(gate) * up), so that the
    // accumulators die before the staging stores
    constexpr int JO = SWIGLU ? 2 : 4;
    v4f out[8][JO];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < JO; ++j) {
        if constexpr (SWIGLU) {
#pragma unroll
          for (int r = 0; r < 4; ++r) out[i][j][r] = silu_fast(acc[i][j][r]) * acc[i][j + 2][r];
        } else {
          out[i][j][0] = __uint_as_float((uint32_t)f32_to_bf16(acc[i][j][0]) |
                                         ((uint32_t)f32_to_bf16(acc[i][j][1]) << 16));
          out[i][j][1] = __uint_as_float((uint32_t)f32_to_bf16(acc[i][j][2]) |
                                         ((uint32_t)f32_to_bf16(acc[i][j][3]) << 16));
        }
      }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if constexpr (!SWIGLU) {
        // bf16: columns 0-127 in b0, 128-255 in b1
        if (wr == half) {
          uint8_t* buf = wc < 2 ? b0 : b1;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int row = i * 16 + (el & 15);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int col = (wc & 1) * 64 + j * 16 + (el >> 4) * 4;
              *reinterpret_cast<uint2*>(chunk_at(buf, row, col >> 3) + (col & 7) * 2) =
                  make_uint2(__float_as_uint(out[i][j][0]), __float_as_uint(out[i][j][1]));
            }
          }
        }
        __syncthreads();
        uint8_t* C = static_cast<uint8_t*>(args.C);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const int c = et + k * NT;                // 16-byte chunk: 32 per row
          const int row = c >> 5, cc = c & 31;
          const v4i val = *reinterpret_cast<const v4i*>(chunk_at(cc < 16 ? b0 : b1, row, cc & 15));
          *reinterpret_cast<v4i*>(C + ((size_t)(row0 + half * 128 + row) * N + n0) * 2 + cc * 16) =
              val;
        }
        __syncthreads();
      } else {
        // fp32 h = silu(gate) * up: output columns 0-63 in b0, 64-127 in b1
        if (wr == half) {
          uint8_t* buf = wc < 2 ? b0 : b1;
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int row = i * 16 + (el & 15);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
              const int col = (wc & 1) * 32 + j * 16 + (el >> 4) * 4;   // within buf
              *reinterpret_cast<v4f*>(chunk_at(buf, row, col >> 2)) = out[i][j];
            }
          }
        }
        __syncthreads();
        // four threads per row, each a quarter (32 columns) of the row's 1x128 block
        const int row = et >> 2, part = et & 3;
        uint8_t* buf = part < 2 ? b0 : b1;
        float hv[32];
        float m = 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const v4f x = *reinterpret_cast<const v4f*>(chunk_at(buf, row, (part & 1) * 8 + q));
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            hv[q * 4 + e] = x[e];
            m = fmaxf(m, fabsf(x[e]));
          }
        }
        m = fmaxf(m, __shfl_xor(m, 1, 64));
        m = fmaxf(m, __shfl_xor(m, 2, 64));
        // the activation quantiser's rule: s = fl32(amax / 448), q = e4m3(fl32(h / s))
        const float sc = block_scale(m);
        uint32_t w[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
          w[q] = e4m3x4(clamp448(hv[4 * q] / sc), clamp448(hv[4 * q + 1] / sc),
                        clamp448(hv[4 * q + 2] / sc), clamp448(hv[4 * q + 3] / sc));
        const int grow = row0 + half * 128 + row;
        uint8_t* C = static_cast<uint8_t*>(args.C) + (size_t)grow * N + n0 + part * 32;
        *reinterpret_cast<v4i*>(C) = v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
        *reinterpret_cast<v4i*>(C + 16) = v4i{(int)w[4], (int)w[5], (int)w[6], (int)w[7]};
        if (part == 0) args.sC[(size_t)grow * (N / 128) + n0 / 128] = sc;
        __syncthreads();
      }
    }
  };

  for (int t = v; t < ntiles; t += P) {
    // runs of GMB row tiles, walked column tile by column tile
    constexpr int GMB = 2;
    const int chunk = t / (GMB * tiles_n);
    const int rows_c = min(GMB, cut - chunk * GMB);
    const int idx = t - chunk * GMB * tiles_n;
    const int rt = chunk * GMB + idx % rows_c, ct = idx / rows_c;
    const int g = find_group(bpre, G, rt, 1);
    const int gu = __builtin_amdgcn_readfirstlane(g);
    const int r0 = __builtin_amdgcn_readfirstlane(grow0(gu) + (rt - bpre[gu]) * kBigRows);
    const int n0 = __builtin_amdgcn_readfirstlane(ct * BN_OUT);
    run_tile(gu, r0, n0);
  }
}

int big_rows_per_round(int N, bool swiglu, int num_cus) {
  const int tiles_n = swiglu ? N / 128 : N / 256;
  return std::max(1, num_cus / std::max(1, tiles_n));
}

hipError_t launch_gemm_fp8_big(const uint8_t* A, const float* sA, const int32_t* a_rows,
                               int a_row_div, const uint8_t* Bf, const float* sB,
                               const int32_t* offsets, int G, int N, int K, bool swiglu, void* C,
                               float* sC, int num_cus, hipStream_t s, int rows_mode, int cap) {
  if (K / 128 > kGemmMaxKBlocks || (K / 128) % 2 != 0) return hipErrorInvalidValue;
  const int rpr = big_rows_per_round(N, swiglu, num_cus);
  BigArgs a{A, sA, a_rows, a_row_div, Bf, offsets, G, N, K, C, sC, rows_mode, cap, rpr};
  int grid = num_cus;
  if (grid >= 8) grid = grid / 8 * 8;
  if (swiglu)
    hipLaunchKernelGGL(gemm_fp8_big_kernel<true>, dim3(grid), dim3(512), 0, s, a, sB);
  else
    hipLaunchKernelGGL(gemm_fp8_big_kernel<false>, dim3(grid), dim3(512), 0, s, a, sB);
  return hipGetLastError();
}

}  // namespace moe
