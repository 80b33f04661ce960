// gemm_mx_kernel.h -- the FP8 block-scaled GEMM kernels for the MI355X (gfx950):
// the scale-panel packing pre-pass and the persistent GEMM kernel.
//
// The operation (CMU "TIRx" blog, section "Evaluation", "Kernel
// performance": FP8 block-scaled matrix multiplication, groups of inputs
// sharing scale factors; the page gives no element encoding, group size or
// scale format): D = A @ B.T with E4M3 elements, one E8M0 power-of-two scale
// per 32 consecutive K values of each row of A and of B (the OCP
// microscaling layout, which the gfx950 matrix cores apply themselves), FP32
// accumulation, one rounding to BF16.  Both operands are K-major, as
// TileFoundry's schedule tutorial (section 4) requires of fp8e4m3 operands.
//
// The kernel is the FP16 kernel's design (dense_gemm.hip) with FP8 data:
//   * 256 x 256 output tiles, four waves of 128 x 128, persistent grid in
//     the grouped XCD-aware order;
//   * a 128-deep K stage is 128 bytes per row, so the LDS layout, its XOR
//     swizzle and the LDS-DMA loader are those of the FP16 kernel's 64-deep
//     stage; two stages in a ring;
//   * v_mfma_scale_f32_16x16x128_f8f6f4: each lane holds 32 bytes of a row
//     (k = 16q .. 16q+15 and 64 + 16q .. 64 + 16q + 15 for lane group q) and
//     the E8M0 scale of block q of its row (a lane group's scale covers the
//     32 consecutive k of block q: measured on the GPU), selected by op_sel
//     from a register holding four scales;
//   * the scales of each stage arrive in LDS with the data: a pre-pass packs
//     them per tile and stage into a 1 KiB panel ordered so that each lane's
//     four-scale words are consecutive across the wave (conflict-free 4-byte
//     LDS reads);
//   * each stage runs as two halves of 32 MFMAs (A fragments 0-3, then
//     4-7), so that all fragments fit in 128 VGPRs: the first half reads A
//     fragments 4-7, the second half (after the stage barrier) reads the next
//     stage's A fragments 0-3, scales and, as each frees, B fragments;
//   * split-K, as in the FP16 kernel, for the tiles of a last, partial wave
//     (all tiles when there are fewer than CUs): parts over ranges of K
//     stages write FP32 partial tiles that split_reduce.h sums in part order
//     and rounds to BF16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "cdna_ops.h"
#include "tile_config.h"
#include "tile_sched.h"

namespace dg {

namespace mx {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// (BM, BN, BKE, GROUP, SC_BYTES and MX_SMALL_K_MAX: tile_config.h)
constexpr int THREADS = 256;
constexpr int WT = 128;                    // wave tile
constexpr int MI = 8, NI = 8;              // 16 x 16 blocks per wave
constexpr int OP_BYTES = BM * BKE;         // 32 KiB per operand per stage
constexpr int SLOT = 2 * OP_BYTES + 2 * SC_BYTES;
constexpr int LDS = 2 * SLOT;              // 132 KiB
constexpr int DMA = OP_BYTES / (THREADS * 16);  // 8 loads per thread per operand
constexpr int HALF_PAIRS = 16;             // MFMA pairs per half stage
constexpr int BARQ = 2;                    // pairs of the second half before its barrier
// (the next stage's read step 2j, B fragment j, runs at pair BARQ + 2j and
// must follow the fragment's last MFMA pair 2j + 1; 3 and 4 measured no faster)
static_assert(BARQ >= 2, "B fragment reads would overtake their last MFMAs");

struct MxParams {
  const uint8_t* A;
  const uint8_t* B;
  const uint8_t* PSA;  // packed scales: [tile row][stage][1 KiB panel]
  const uint8_t* PSB;  // packed scales: [tile column][stage][1 KiB panel]
  uint16_t* D;
  int M, N, K;
  int lda, ldb, ldd;
  int tiles_m, tiles_n, group_m, num_tasks, num_xcds;
  int d_vec;
  int nks;   // K stages
  int koff;  // leading pad of the first stage (K elements)
  // split-K (the SPLIT kernel): tasks below full_tasks are whole tiles; the
  // rest are (tile, part) pairs over the last `tiles` tiles of the order.
  // Task full_tasks + u is part u / tiles of tile full_tasks + u % tiles; the
  // part covers K stages [part * split_steps, min(nks, (part + 1) *
  // split_steps)) and writes its FP32 partial tile (row-major 256 x 256) to
  // ws at index part * tiles + u % tiles (split_reduce.h sums them)
  int full_tasks, splits, split_steps, tiles;
  float* ws;
};

// Panel layout: byte ((w*2 + h)*64 + s*16 + l16)*4 + b holds the scale of
// row w*128 + 16 (4 h + b) + l16 of the tile for block s of the stage: lane
// l = 16 s + l16 of wave row (or column) w finds the scales of its fragments
// 4h .. 4h+3 in the word at ((w*2 + h)*64 + l)*4, and the 64 lanes of a
// wave read 256 consecutive bytes.
struct PackArgs {
  const uint8_t* S[2];  // SA, SB
  int rows[2];          // M, N
  int ld[2];            // ldsa, ldsb
  int tiles[2];         // tile rows of A, tile columns of B
};

// One launch packs both operands.  Workgroup (g, c) takes tile g (A's tile
// rows first, then B's tile columns) and the 4 stages of chunk c: it copies
// the tile's 256 rows x 16 scale bytes of those stages into LDS, four
// threads per row (4-byte reads where the rows allow it), then writes each
// stage's panel, one 4-byte word per thread (each panel a contiguous 1 KiB).
// Rows past the matrix and blocks outside [0, K/32) get scale 1 (their data
// is zero, and zero times a finite scale stays zero).
constexpr int PACK_STAGES = 4;
__global__ __launch_bounds__(256) void scale_pack(PackArgs a, int nb, int nks, int koff,
                                                  uint8_t* __restrict__ P) {
  __shared__ uint32_t rowbuf[BM][PACK_STAGES];  // 4 scale bytes (one stage) per word
  int tile = blockIdx.x;
  const int op = tile >= a.tiles[0] ? 1 : 0;
  const size_t out0 = (size_t)tile * nks * SC_BYTES;  // panels of earlier tiles
  if (op) tile -= a.tiles[0];
  const int ks0 = blockIdx.y * PACK_STAGES;
  const int c0 = ks0 * (BKE / GROUP) - koff / GROUP;  // first block of the chunk
  const int t = threadIdx.x;
  const uint8_t* S = a.S[op];
  const int ld = a.ld[op], rows = a.rows[op];
  // whole words of the row are read in place when the row starts, the
  // stride and the chunk's first block are 4-byte aligned and the chunk
  // lies inside [0, nb)
  const bool words = (((uintptr_t)S | (uintptr_t)ld | (uintptr_t)c0) & 3) == 0 && c0 >= 0 &&
                     c0 + 4 * PACK_STAGES <= nb;
  const int j = t & 3;  // stage j of the chunk: blocks c0 + 4 j .. +3
#pragma unroll
  for (int pass = 0; pass < BM / 64; ++pass) {
    const int r = pass * 64 + (t >> 2);
    const int row = tile * BM + r;
    uint32_t v = 0x7F7F7F7Fu;
    if (row < rows) {
      const uint8_t* src = S + (int64_t)row * ld + c0 + 4 * j;
      if (words) {
        v = *(const uint32_t*)src;
      } else {
        v = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int blk = c0 + 4 * j + b;
          v |= (uint32_t)(blk >= 0 && blk < nb ? src[b] : (uint8_t)127) << (8 * b);
        }
      }
    }
    rowbuf[r][j] = v;
  }
  __syncthreads();
  const int l16 = t & 15, s = (t >> 4) & 3, h = (t >> 6) & 1, w = t >> 7;
  const int kn = min(PACK_STAGES, nks - ks0);
  for (int k = 0; k < kn; ++k) {
    uint32_t word = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b)
      word |= ((rowbuf[w * WT + 16 * (4 * h + b) + l16][k] >> (8 * s)) & 0xFFu) << (8 * b);
    *(uint32_t*)(P + out0 + (size_t)(ks0 + k) * SC_BYTES + 4 * t) = word;
  }
}

struct Frags {
  i32x8 lo[4];  // A fragments 0-3
  i32x8 hi[4];  // A fragments 4-7
  i32x8 b[8];
};

// fn(integral_constant<int, i>) for i = B .. E-1 (indices usable as
// constant expressions, which the MFMA's op_sel operands must be)
template <int B, int E, typename Fn>
__device__ __forceinline__ void static_for(Fn&& fn) {
  if constexpr (B < E) {
    fn(std::integral_constant<int, B>{});
    static_for<B + 1, E>(fn);
  }
}

// v_mfma_scale_f32_16x16x128_f8f6f4 with E4M3 operands, accumulating in
// place, the scale of srcA taken from byte X of its scale register and that
// of srcB from byte Y (op_sel holds the low bit of each byte index, op_sel_hi
// the high bit).  Written as asm for the same reason as the 16 x 16 x 32
// MFMA of the FP16 kernel: with all 256 accumulator registers live, the
// compiler's builtin form keeps some accumulators out of place and copies
// them around every MFMA.  The compiler inserts no wait states for these
// MFMAs: the kernel orders accumulator reset and result reads itself, and
// their source registers are written by LDS reads only.
template <int X, int Y>
__device__ __forceinline__ void mx_mfma(f32x4& c, const i32x8& a, const i32x8& b, uint32_t sa,
                                        uint32_t sb);
#define DG_MX_MFMA(X, Y, XL, YL, XH, YH)                                                      \
  template <>                                                                                 \
  __device__ __forceinline__ void mx_mfma<X, Y>(f32x4 & c, const i32x8& a, const i32x8& b,   \
                                                uint32_t sa, uint32_t sb) {                   \
    asm("v_mfma_scale_f32_16x16x128_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[" #XL "," #YL      \
        ",0] op_sel_hi:[" #XH "," #YH ",0]"                                                   \
        : "+a"(c)                                                                             \
        : "v"(a), "v"(b), "v"(sa), "v"(sb));                                                  \
  }
DG_MX_MFMA(0, 0, 0, 0, 0, 0)
DG_MX_MFMA(0, 1, 0, 1, 0, 0)
DG_MX_MFMA(0, 2, 0, 0, 0, 1)
DG_MX_MFMA(0, 3, 0, 1, 0, 1)
DG_MX_MFMA(1, 0, 1, 0, 0, 0)
DG_MX_MFMA(1, 1, 1, 1, 0, 0)
DG_MX_MFMA(1, 2, 1, 0, 0, 1)
DG_MX_MFMA(1, 3, 1, 1, 0, 1)
DG_MX_MFMA(2, 0, 0, 0, 1, 0)
DG_MX_MFMA(2, 1, 0, 1, 1, 0)
DG_MX_MFMA(2, 2, 0, 0, 1, 1)
DG_MX_MFMA(2, 3, 0, 1, 1, 1)
DG_MX_MFMA(3, 0, 1, 0, 1, 0)
DG_MX_MFMA(3, 1, 1, 1, 1, 0)
DG_MX_MFMA(3, 2, 1, 0, 1, 1)
DG_MX_MFMA(3, 3, 1, 1, 1, 1)
#undef DG_MX_MFMA

// One 16 x 16 block of D^T = B A^T over 128 k: srcA is B's fragment J (its
// scales: byte J % 4 of sb[J / 4]), srcB is A's fragment I (byte I % 4 of
// sa[I / 4]); each lane ends up holding one row of D, four columns.
template <int I, int J>
__device__ __forceinline__ void mfma_mx(f32x4 (&acc)[MI][NI], const i32x8& bf, const i32x8& af,
                                        const u32x2& sa, const u32x2& sb) {
  mx_mfma<J % 4, I % 4>(acc[I][J], bf, af, sb[J / 4], sa[I / 4]);
}
// MFMA t (0..31) of a half stage: B fragment t / 4 against A fragment
// base + i, with i running forwards under even B fragments and backwards
// under odd ones, so that each MFMA changes one operand only.
template <int T>
constexpr int snake_i() { return ((T / 4) & 1) ? 3 - T % 4 : T % 4; }

template <bool SPLIT>
__global__ __launch_bounds__(THREADS) void gemm_mx_kernel(MxParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[LDS];
  const uint32_t lds0 = lds_addr(smem);

  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int nk = p.nks;
  const int slot0 = xcd_slot(blockIdx.x, gridDim.x, p.num_xcds);

  for (int task = slot0; task < p.num_tasks; task += gridDim.x) {
    int tm, tn;
    const bool part = SPLIT && task >= p.full_tasks;
    const int u = task - p.full_tasks;
    const int split = part ? u / p.tiles : 0;
    tile_of_task(part ? p.full_tasks + u % p.tiles : task, p.tiles_m, p.tiles_n, p.group_m, &tm,
                 &tn);
    // this task's K stages (ring slots count from kbeg)
    const int kbeg = split * p.split_steps;
    const int kend = part ? min(nk, kbeg + p.split_steps) : nk;
    const int m0 = tm * BM, n0 = tn * BN;
    const int vm = min(BM, p.M - m0), vn = min(BN, p.N - n0);

    const int lane = opaque_tid() & 63;
    const int l16 = lane & 15, lq = lane >> 4;

    f32x4 acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j) acc[i][j] = (f32x4){};
    fence();

    // Fragment read offsets: lane (l16, lq) reads logical chunks lq and lq+4
    // of row 16 f + l16 (the swizzle depends on the row's low four bits).
    const int sw = swz_k(l16);
    const int fa0 = (wm * WT + l16) * 128 + ((lq ^ sw) << 4);
    const int fa1 = (wm * WT + l16) * 128 + (((lq + 4) ^ sw) << 4);
    const int fb0 = OP_BYTES + (wn * WT + l16) * 128 + ((lq ^ sw) << 4);
    const int fb1 = OP_BYTES + (wn * WT + l16) * 128 + (((lq + 4) ^ sw) << 4);
    const int fsa = 2 * OP_BYTES + wm * 512 + lane * 4;  // fragments 0-3; 4-7 at +256
    const int fsb = 2 * OP_BYTES + SC_BYTES + wn * 512 + lane * 4;

    // Loader (the FP16 kernel's, in bytes): load i of this thread covers tile
    // row (8 wave + i) * 8 + lane / 8 and the logical chunk the swizzle puts
    // at physical chunk lane % 8.
    uint32_t a_off[DMA], b_off[DMA];
    int kc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) kc[h] = (lane & 7) ^ swz_k(h * 8 + (lane >> 3));
#pragma unroll
    for (int i = 0; i < DMA; ++i) {
      const int r = (8 * wave + i) * 8 + (lane >> 3);
      a_off[i] = r < vm ? (uint32_t)(r * p.lda + kc[i & 1] * 16) : OOB;
      b_off[i] = r < vn ? (uint32_t)(r * p.ldb + kc[i & 1] * 16) : OOB;
    }
    struct Stage {
      i32x4 ra, rb, rs;  // A, B and scale-panel descriptors
      uint32_t base;     // LDS slot
      uint32_t wbase;    // this wave's first 1 KiB of the slot's A tile
      int k0;            // first k of the stage (negative only for the first)
    };
    auto stage_setup = [&](int ks, int slot) {
      Stage st;
      const int k0 = ks * BKE - p.koff;
      const bool live = ks < kend;
      st.k0 = k0;
      st.base = lds0 + slot * SLOT;
      st.wbase = st.base + (8 * wave) * 1024;
      st.ra = make_rsrc((uint64_t)(uintptr_t)(p.A + (int64_t)m0 * p.lda) + k0,
                        live ? (uint32_t)((vm - 1) * p.lda + p.K - k0) : 0u);
      st.rb = make_rsrc((uint64_t)(uintptr_t)(p.B + (int64_t)n0 * p.ldb) + k0,
                        live ? (uint32_t)((vn - 1) * p.ldb + p.K - k0) : 0u);
      // even waves load the A panel, odd waves the B panel (each panel is
      // written twice with the same bytes: every wave issues the same
      // instruction stream, with no branch to split the loop body)
      const uint8_t* panel = (wave & 1) == 0 ? p.PSA + ((int64_t)tm * nk + ks) * SC_BYTES
                                             : p.PSB + ((int64_t)tn * nk + ks) * SC_BYTES;
      st.rs = make_rsrc((uint64_t)(uintptr_t)panel, live ? (uint32_t)SC_BYTES : 0u);
      return st;
    };
    // load i of a stage: 0..7 A, 8..15 B, 16 a scale panel
    auto load = [&](const Stage& st, int i, bool masked) {
      if (i < 2 * DMA) {
        const int op = i / DMA, j = i % DMA;
        const uint32_t off = op == 0 ? a_off[j] : b_off[j];
        const bool in = !masked || st.k0 + kc[j & 1] * 16 >= 0;
        dma16_at(op == 0 ? st.ra : st.rb, in ? off : OOB, st.wbase, op * OP_BYTES + j * 1024);
      } else {
        dma16_at(st.rs, (uint32_t)(lane * 16), st.base + (wave & 1) * SC_BYTES, 2 * OP_BYTES);
      }
      fence();
    };

    auto read_a = [&](int slot, int f) {
      const char* base = smem + slot * SLOT;
      const u32x4 x = *(const u32x4*)(base + fa0 + f * 2048);
      const u32x4 y = *(const u32x4*)(base + fa1 + f * 2048);
      return (i32x8){(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
    };
    auto read_b = [&](int slot, int f) {
      const char* base = smem + slot * SLOT;
      const u32x4 x = *(const u32x4*)(base + fb0 + f * 2048);
      const u32x4 y = *(const u32x4*)(base + fb1 + f * 2048);
      return (i32x8){(int)x[0], (int)x[1], (int)x[2], (int)x[3], (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
    };
    auto read_s = [&](int slot, int off) { return *(const uint32_t*)(smem + slot * SLOT + off); };

    // Ring: stage ks in slot (ks - kbeg) % 2; entering step ks, stage ks has landed,
    // stage ks+1 is in flight, and F.lo, F.b, sa[0], sb hold stage ks.  Each
    // scale word (four fragments' scales) is read straight into the register
    // the MFMAs use, after that register's last use by the stage before: no
    // copies between stages.
    Frags F;
    u32x2 sa, sb;
    // the reads of stage ks+1 issued during stage ks's second half, in the
    // order issued (the prologue issues the same sequence, so the loop head
    // sees one pattern of outstanding reads)
    auto read_next = [&](int slot, int step) {
      switch (step) {
        case 0: F.b[0] = read_b(slot, 0); break;
        case 1: F.lo[0] = read_a(slot, 0); break;
        case 2: F.b[1] = read_b(slot, 1); break;
        case 3: F.lo[1] = read_a(slot, 1); break;
        case 4: F.b[2] = read_b(slot, 2); break;
        case 5: F.lo[2] = read_a(slot, 2); break;
        case 6: F.b[3] = read_b(slot, 3); break;
        case 7: F.lo[3] = read_a(slot, 3); break;
        case 8: F.b[4] = read_b(slot, 4); break;
        case 9: sa[0] = read_s(slot, fsa); break;
        case 10: F.b[5] = read_b(slot, 5); break;
        case 11: sb[0] = read_s(slot, fsb); break;
        case 12: F.b[6] = read_b(slot, 6); break;
        case 13: F.b[7] = read_b(slot, 7); break;
        default: sb[1] = read_s(slot, fsb + 256); break;
      }
      fence();
    };
    {
      const Stage s0 = stage_setup(kbeg, 0);
#pragma unroll
      for (int i = 0; i < 2 * DMA + 1; ++i) load(s0, i, true);
      const Stage s1 = stage_setup(kbeg + 1, 1);
#pragma unroll
      for (int i = 0; i < DMA; ++i) load(s1, i, true);
      load(s1, 2 * DMA, true);
      wait_vm_barrier<DMA + 1>();  // stage 0 has landed
#pragma unroll
      for (int step = 0; step < 15; ++step) read_next(0, step);
    }

    for (int ks = kbeg; ks < kend; ++ks) {
      const int slot = (ks - kbeg) & 1;
      // stage ks+1's B tile, into the other slot (free since the last
      // barrier): issued over the first half's first DMA pairs
      const Stage sn1 = stage_setup(ks + 1, slot ^ 1);
      // first half: A fragments 0-3 against B fragments 0-7 (pair q: B
      // fragment 2q / 4, two A fragments in snake order); A fragments 4-7 of
      // this stage are read in between
      static_for<0, HALF_PAIRS>([&](auto qc) {
        constexpr int q = decltype(qc)::value;
        if constexpr (q % 4 == 1) F.hi[q / 4] = read_a(slot, 4 + q / 4);
        if constexpr (q == 3) sa[1] = read_s(slot, fsa + 256);  // A fragments 4-7
        mfma_mx<snake_i<2 * q>(), (2 * q) / 4>(acc, F.b[(2 * q) / 4], F.lo[snake_i<2 * q>()], sa, sb);
        mfma_mx<snake_i<2 * q + 1>(), (2 * q + 1) / 4>(acc, F.b[(2 * q + 1) / 4],
                                                       F.lo[snake_i<2 * q + 1>()], sa, sb);
        fence();
        if constexpr (q < DMA) load(sn1, DMA + q, false);
      });
      // second half: A fragments 4-7.  After BARQ pairs, the barrier: stage
      // ks+1 has landed for every wave and every wave is done reading stage
      // ks; then stage ks+1's A fragments 0-3 and scales are read, each B
      // fragment once its last MFMA of this stage has issued, and stage ks's
      // slot is refilled with stage ks+2's A tile and scales (its B tile
      // during the next stage's first half: the refill loads are split over
      // two halves rather than bunched into one).
      const Stage sn = stage_setup(ks + 2, slot);
      static_for<0, HALF_PAIRS>([&](auto qc) {
        constexpr int q = decltype(qc)::value;
        if constexpr (q == BARQ) {
          wait_vm_barrier<0>();
          fence();
        }
        // stage ks+1's reads: B fragment j (and sb[0]) only after its last
        // MFMA of this stage (pairs 2j, 2j+1; sb[0] serves pairs 0-7)
        if constexpr (q >= BARQ && q <= 14) read_next(slot ^ 1, q - BARQ);
        mfma_mx<4 + snake_i<2 * q>(), (2 * q) / 4>(acc, F.b[(2 * q) / 4], F.hi[snake_i<2 * q>()], sa, sb);
        mfma_mx<4 + snake_i<2 * q + 1>(), (2 * q + 1) / 4>(acc, F.b[(2 * q + 1) / 4],
                                                           F.hi[snake_i<2 * q + 1>()], sa, sb);
        fence();
        if constexpr (q >= BARQ) {
          // stage ks+2's A tile and scale panel (its B tile follows in the
          // next stage's first half)
          constexpr int n = HALF_PAIRS - BARQ, tot = DMA + 1;
          static_for<((q - BARQ) * tot) / n, ((q - BARQ + 1) * tot) / n>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            load(sn, i < DMA ? i : 2 * DMA, false);
          });
        }
      });
      // the remaining reads (B fragment 7 and sb[1] last: free after the
      // last pair)
      static_for<15 - BARQ, 15>([&](auto sc) { read_next(slot ^ 1, decltype(sc)::value); });
    }

    wait_vm_barrier<0>();  // every wave is done with the ring; reuse it for staging
    // wait states between the last MFMAs and the reads of their results
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    fence();

    if constexpr (SPLIT) {
      if (part) {
        // FP32 partial tile, row-major 256 x 256: lane holds row l16 of each
        // 16-row block and columns j*16 + 4*lq .. +3 (16 contiguous bytes);
        // 16 x 16 blocks wholly outside D are skipped (nothing reads them)
        float* w = p.ws + (size_t)(split * p.tiles + u % p.tiles) * (BM * BN) +
                   (size_t)(wm * WT + l16) * BN + wn * WT + 4 * lq;
#pragma unroll
        for (int i = 0; i < MI; ++i) {
          if (wm * WT + i * 16 >= vm) break;
#pragma unroll
          for (int j = 0; j < NI; ++j) {
            if (wn * WT + j * 16 >= vn) break;
            *(float4*)(w + i * 16 * BN + j * 16) =
                make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        continue;
      }
    }

    // Epilogue (the FP16 kernel's): per 32-row band, round to BF16, stage the
    // band's 32 x 128 outputs of this wave in LDS, store 16-byte row chunks.
    char* stg = smem + wave * (32 * 256);
    const bool interior = p.d_vec && vm == BM && vn == BN;
#pragma unroll
    for (int band = 0; band < MI / 2; ++band) {
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int i = 2 * band + half;
        const int row = half * 16 + l16;
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          u32x2 v;
          v[0] = pack2<__bf16>(acc[i][j][0], acc[i][j][1]);
          v[1] = pack2<__bf16>(acc[i][j][2], acc[i][j][3]);
          const int chunk = 2 * j + (lq >> 1);
          *(u32x2*)(stg + row * 256 + ((chunk ^ (row & 15)) << 4) + (lq & 1) * 8) = v;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      const int row0 = m0 + wm * WT + band * 32;
      const int col0 = n0 + wn * WT;
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int rr = t * 4 + (lane >> 4);
        const int cc = lane & 15;
        const u32x4 v = *(const u32x4*)(stg + rr * 256 + ((cc ^ (rr & 15)) << 4));
        const int row = row0 + rr;
        const int col = col0 + cc * 8;
        if (interior) {
          __builtin_nontemporal_store(v, (u32x4*)(p.D + (int64_t)row * p.ldd + col));
        } else if (row < p.M && col < p.N) {
          uint16_t* dst = p.D + (int64_t)row * p.ldd + col;
          if (p.d_vec && col + 8 <= p.N) {
            __builtin_nontemporal_store(v, (u32x4*)dst);
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (col + e < p.N) dst[e] = (uint16_t)(v[e >> 1] >> ((e & 1) * 16));
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_lds_barrier();
  }
}

}  // namespace mx
}  // namespace dg
