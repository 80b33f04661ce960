// gemm_kernel.h -- the FP16/BF16 tiled GEMM kernels for the MI355X (gfx950):
// the persistent GEMM kernel and the operand repack (the split-K reduction
// is in split_reduce.h).
//
// Kernel structure (one persistent workgroup per CU):
//   * a persistent loop over output tiles in the grouped, XCD-aware order of
//     tile_sched.h ("TIRx GEMM on Blackwell", V6: persistent CTAs pulling
//     tiles; TileFoundry schedule tutorial, sections 2-3: persistent CTAs and
//     the grouped traversal);
//   * per K step, 16-byte LDS-DMA loads of the A and B tiles into LDS rings
//     (three slots for one operand, two for the other: all 160 KiB) while
//     the previous stage feeds the matrix cores ("TIRx GEMM on Blackwell",
//     V5: shared-memory stages so loading the next K tile overlaps the MMA
//     of the current one);
//   * an XOR swizzle of 16-byte chunks inside each LDS row, so both the
//     row-wise tile writes and the column-wise MFMA fragment reads spread over
//     all banks (the role of the 128-byte swizzle in the TIRx and TileFoundry
//     shared-memory layouts);
//   * v_mfma_f32_16x16x32_{f16,bf16} with FP32 accumulators; four waves each
//     own a 128 x 128 quarter of a 256 x 256 tile (128 x 64 of a 256 x 128
//     tile for narrow A @ B.T outputs; 64 rows of a 128-row tile where M <=
//     128) and read the shared A and B stages
//     ("TIRx GEMM on Blackwell", V8/V9: larger tiles and several consumers
//     reusing one staged operand tile);
//   * an epilogue that rounds to the output type, stages each wave's rows in
//     LDS and writes whole 16-byte row chunks (TileFoundry tutorial, section 5:
//     the output tile is staged in shared memory before the store);
//   * ragged M, N and K handled by masking: out-of-range loads read zeros
//     through the buffer descriptor's range check, out-of-range stores are
//     skipped (the pages' shapes all divide the tiles; this is our reading);
//   * split-K for the last, partial wave of tiles (the parts' FP32 tiles
//     summed by split_reduce.h), and a repack of operands the 16-byte loads
//     cannot read in place (chosen by the host side, dense_gemm.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cdna_ops.h"
#include "tile_config.h"
#include "tile_sched.h"

namespace dg {

// ---- tile configuration (Layout, BM, BN, BK, WAVES, THREADS: tile_config.h)
constexpr int SLOTS3 = 3;            // LDS ring depth of the early operand (below)
constexpr int SLOTS2 = 2;            // LDS ring depth of the other operand
constexpr int MK = 32;               // K depth of one MFMA (16 x 16 x 32)
constexpr int SUB = BK / MK;         // MFMA k-substeps per stage
// Tile rows TM: 256 (BM), or 128 for products with M <= 128 (half the
// MFMA work of a 256-row tile that would be half padding).  A wave tile is
// TM / 2 rows (MI 16-row MFMA blocks); the A tile of a stage is TM rows of
// 128 B, loaded in TM / 32 16-byte loads per thread.
template <int TM>
constexpr int wave_rows() { return TM / 2; }
template <int TM>
constexpr int a_loads() { return TM * BK * 2 / (THREADS * 16); }
// MFMA pairs of the last substep issued before its barrier: the reads of
// that substep's fragments (issued during the previous substep) complete
// meanwhile, so the barrier's LDS wait costs nothing
constexpr int BAR_PAIR = 2;

static_assert(BK == 64 && BM == 256 && BN == 256, "swizzles below assume these sizes");
static_assert(SUB == 2, "the ring schedule below has two substeps per stage");

struct Params {
  const uint16_t* A;
  const uint16_t* B;
  uint16_t* D;
  int M, N, K;
  int lda, ldb, ldd;
  int tiles_m, tiles_n, group_m, num_tasks, num_xcds;
  int d_vec;  // D rows are 16-byte aligned (16-byte stores allowed)
  // split-K (the SPLIT kernels): tasks below full_tasks are whole tiles;
  // the rest are (tile, part) pairs over the last `tiles` tiles of the
  // order.  Task full_tasks + u is part u / tiles of tile full_tasks +
  // u % tiles; the part covers K steps [part * split_steps, min(nk, (part +
  // 1) * split_steps)) and writes its FP32 partial tile (row-major TM x TN,
  // TM and TN the tile's rows and width) to ws at index part * tiles + u %
  // tiles
  int full_tasks, splits, split_steps, tiles;
  float* ws;
};

template <int MA, int NB>
struct Frags {
  u32x4 a[MA];
  u32x4 b[NB];
};

// Tile width TN: 256 (four 128 x 128 wave tiles), or for A @ B.T 128 (four
// 128 x 64 wave tiles): for outputs at most 128 wide (half the work of a
// half-padded 256-wide tile), and for twice the tiles where 256-wide ones
// would leave half the CUs idle, at more operand traffic per FLOP.  Tile
// rows TM: 256, or 128 where M <= 128 (four 64-row wave tiles).
template <typename T, int LAYOUT, bool SPLIT, int TN, int TM>
__global__ __launch_bounds__(THREADS) void gemm_kernel(Params p) {
  static_assert(TN == BN || (TN == BN / 2 && LAYOUT == NT), "tile widths 256, and 128 for A @ B.T");
  static_assert(TM == BM || TM == BM / 2, "tile rows 256 or 128");
  constexpr int WTM = wave_rows<TM>();             // wave tile rows
  constexpr int MI = WTM / 16;                     // 16 x 16 blocks per wave, M direction
  constexpr int A_BYTES = TM * BK * 2;             // bytes of an A tile (TM rows x 128 B)
  constexpr int DMA_PER_OPERAND = a_loads<TM>();   // 16-byte loads per thread (A)
  constexpr int WTN = TN / 2;                      // wave tile columns
  constexpr int NI = WTN / 16;                     // 16 x 16 blocks per wave, N direction
  constexpr int PAIRS = MI * NI / 2;               // MFMA pairs per substep
  constexpr int B_TILE = TN * BK * 2;              // bytes of a B tile
  constexpr int DMA_B = B_TILE / (THREADS * 16);   // 16-byte loads per thread (B)
  // The operand with the three-slot ring, whose loads are issued a substep
  // earlier (0 = A, 1 = B): B for A @ B, whose row-major tile (64 rows of
  // 512 B, far apart in memory) is the costlier one to load (measured: 1.4%
  // faster than A there); A for A @ B.T (the two are alike).
  constexpr int EARLY = LAYOUT == NN ? 1 : 0;
  constexpr int DMA_E = EARLY == 0 ? DMA_PER_OPERAND : DMA_B;   // loads of the early tile
  constexpr int DMA_L = EARLY == 0 ? DMA_B : DMA_PER_OPERAND;   // and of the other
  constexpr int E_BYTES = EARLY == 0 ? A_BYTES : B_TILE;
  constexpr int L_BYTES = EARLY == 0 ? B_TILE : A_BYTES;
  constexpr int RING2 = SLOTS3 * E_BYTES;            // the two-slot ring follows the other
  constexpr int LDS_BYTES = RING2 + SLOTS2 * L_BYTES;  // all 160 KiB for 256-wide tiles
  using Frags = dg::Frags<MI, NI>;
  __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];
  const uint32_t lds0 = lds_addr(smem);

  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int wm = wave >> 1;  // wave tile row (0..1)
  const int wn = wave & 1;   // wave tile column (0..1)

  const int nk = (p.K + BK - 1) / BK;
  const int slot0 = xcd_slot(blockIdx.x, gridDim.x, p.num_xcds);

  for (int task = slot0; task < p.num_tasks; task += gridDim.x) {
    int tm, tn;
    const bool part = SPLIT && task >= p.full_tasks;
    const int u = task - p.full_tasks;
    const int tile = part ? p.full_tasks + u % p.tiles : task;
    const int split = part ? u / p.tiles : 0;
    tile_of_task(tile, p.tiles_m, p.tiles_n, p.group_m, &tm, &tn);
    // this task's K steps
    const int kbeg = split * p.split_steps;
    const int kend = part ? min(nk, kbeg + p.split_steps) : nk;
    const int m0 = tm * TM;
    const int n0 = tn * TN;
    const int vm = min(TM, p.M - m0);  // valid rows of the A tile
    const int vn = min(TN, p.N - n0);  // valid columns of D in this tile

    // MFMA operand layout (16 x 16 x 32): lane l holds row l % 16 of a
    // 16-row fragment and k = 8 (l / 16) .. +7 of the substep's 32
    const int lane = opaque_tid() & 63;
    const int l16 = lane & 15;
    const int lq = lane >> 4;

    // Accumulators start at zero.  The compiler places the zeroing just
    // before the K loop, after the prologue's barrier and fragment reads: at
    // least 30 instructions separate each register's reset from the first
    // (asm, so unguarded) MFMA that reads it, far more than the wait states
    // the hardware needs.  (Pinning it earlier, under the first loads, made
    // the register allocator spill.)
    f32x4 acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j) acc[i][j] = (f32x4){};
    fence();

    // Loader roles.  K-contiguous tiles: each wave instruction fills 1 KiB =
    // 8 rows of 128 B; wave w's instruction i of an operand with L loads per
    // thread covers rows (L w + i) * 8 ... +7, lane -> row lane/8 of the
    // group and a logical chunk by the swizzle (which depends on the row's
    // low four bits, i.e. on i's parity, L being even).
    // NN B tile: each wave instruction fills 2 k rows of 512 B.
    const int nn_row_lo = lane >> 5;

    // Fragment read offsets (bytes within a stage).  Fragment f of a
    // K-contiguous tile (16 rows) sits 16 * 128 bytes after fragment 0: the
    // swizzle depends only on the row's low four bits.
    int fa[SUB], fb[SUB], fbn[NI];
#pragma unroll
    for (int s = 0; s < SUB; ++s) {
      fa[s] = (wm * WTM + l16) * 128 + (((4 * s + lq) ^ swz_k(l16)) << 4);
      fb[s] = (wn * WTN + l16) * 128 + (((4 * s + lq) ^ swz_k(l16)) << 4);
    }
    {
      // transposing reads (NN B): in 16-lane block lq, lane i supplies row
      // k = 8 lq + i / 4 (+ 4 for the second read, + 32 per substep) and the
      // four columns n = wn*128 + 16 j + 4 (i % 4) .. +3, so that it receives
      // column 16 j + i at four consecutive k
      const int klane = 8 * lq + (l16 >> 2);
      // swz_n of every row this lane reads (the +4 and +32 row offsets of the
      // reads leave bits 0-1 and 3-4 of k unchanged)
      const int fl = swz_n(klane);
#pragma unroll
      for (int j = 0; j < NI; ++j)
        fbn[j] = klane * 512 + (((wn * 16 + 2 * j + ((lane & 3) >> 1)) ^ fl) << 4) + (lane & 1) * 8;
    }

    // Per-lane load offsets, fixed for the tile; the buffer descriptor of
    // each K step is rebased on that step (scalar work), so a load needs no
    // vector arithmetic.  Rows beyond M (A) or N (NT B) get an offset past
    // every range and read zeros.
    //
    // K steps: step s covers k = s*BK - koff .. +BK-1.  koff pads the first
    // step at its front so that the last one ends exactly at K8 (K rounded
    // up to 8; where K8 > K the operand is a zero-padded copy, or for the NN
    // B the descriptor ends at row K-1).  Only the first step reaches outside
    // [0, K8) -- below 0 -- so only its loads, issued in the prologue, need
    // per-lane masks.
    const int K8 = (p.K + 7) & ~7;
    const int koff = (BK - (K8 & (BK - 1))) & (BK - 1);
    uint32_t a_off[DMA_PER_OPERAND], b_off[DMA_B];
    int kc[2];  // logical chunk of this lane for even / odd instruction index
#pragma unroll
    for (int h = 0; h < 2; ++h) kc[h] = (lane & 7) ^ swz_k(h * 8 + (lane >> 3));
#pragma unroll
    for (int i = 0; i < DMA_PER_OPERAND; ++i) {
      const int r = (DMA_PER_OPERAND * wave + i) * 8 + (lane >> 3);
      a_off[i] = r < vm ? (uint32_t)(r * p.lda * 2 + kc[i & 1] * 16) : OOB;
    }
    if (LAYOUT == NT) {
#pragma unroll
      for (int i = 0; i < DMA_B; ++i) {
        const int r = (DMA_B * wave + i) * 8 + (lane >> 3);
        b_off[i] = r < vn ? (uint32_t)(r * p.ldb * 2 + kc[i & 1] * 16) : OOB;
      }
    } else {
#pragma unroll
      for (int i = 0; i < DMA_B; ++i) {
        const int k = 2 * (8 * wave + i) + nn_row_lo;
        const int c = (lane & 31) ^ swz_n(k);
        b_off[i] = (uint32_t)(k * p.ldb * 2 + c * 16);
      }
    }

    // LDS-DMA loads of K step ks into slot `slot` of its ring: the A tile (half 0)
    // or the B tile (half 1), issued one load at a time.  The descriptor
    // starts at the step's first column (K-contiguous tiles) or row (NN B)
    // and ends with the tile's last valid row, rounded up to a whole 8-element
    // chunk (where K or N is not a multiple of 8 the operand is a zero-padded
    // copy).  Steps at or past kend get an empty range: the slot is
    // zero-filled and the loop keeps a fixed pattern of loads in flight.
    struct Half {
      i32x4 r;
      uint32_t base;
      int k0;  // the step's first k (negative only for the first step)
    };
    // (Ranges are computed in 32 bits, which the argument check guarantees
    // suffice; 64-bit forms made the compiler branch inside the loop.)
    auto half_setup = [&](int ks, int slot, int half) {
      Half h;
      const int k0 = ks * BK - koff;
      const bool live = ks < kend;
      h.k0 = k0;
      h.base = lds0 + (half == EARLY ? 0 : RING2) + slot * (half == 0 ? A_BYTES : B_TILE) +
               ((half == 0 ? DMA_PER_OPERAND : DMA_B) * wave) * 1024;
      if (half == 0 || LAYOUT == NT) {
        // columns k0 .. K8 of the tile's rows
        const uint64_t src = half == 0 ? (uint64_t)(uintptr_t)(p.A + (int64_t)m0 * p.lda)
                                       : (uint64_t)(uintptr_t)(p.B + (int64_t)n0 * p.ldb);
        const int span = half == 0 ? (vm - 1) * p.lda : (vn - 1) * p.ldb;
        const uint32_t bytes = (uint32_t)(span + K8 - k0) * 2u;
        h.r = make_rsrc(src + 2 * (int64_t)k0, live ? bytes : 0u);
      } else {
        // rows k0 .. min(k0 + BK, K) - 1 of B, columns n0 .. N (rounded up to 8)
        const int rows = min(BK, p.K - k0);
        const uint32_t bytes = (uint32_t)((rows - 1) * p.ldb + ((p.N - n0 + 7) & ~7)) * 2u;
        h.r = make_rsrc((uint64_t)(uintptr_t)(p.B + n0) + 2 * (int64_t)k0 * p.ldb, live ? bytes : 0u);
      }
      return h;
    };
    // One load of a refill.  MASKED (prologue only): chunks or rows before
    // k = 0 read zeros.
    auto refill_one = [&](const Half& h, int half, int i, bool masked) {
      if (half == 0 || LAYOUT == NT) {
        const uint32_t off = half == 0 ? a_off[i] : b_off[i];
        dma16_at(h.r, !masked || h.k0 + (kc[i & 1] << 3) >= 0 ? off : OOB, h.base, i * 1024);
      } else {
        const int k = 2 * (8 * wave + i) + nn_row_lo;
        dma16_at(h.r, !masked || h.k0 + k >= 0 ? b_off[i] : OOB, h.base, i * 1024);
      }
      fence();
    };
    auto refill_stage = [&](int ks, int slot) {
      const Half ha = half_setup(ks, slot, 0);  // A and B slots agree for stages 0 and 1
      const Half hb = half_setup(ks, slot, 1);
#pragma unroll
      for (int i = 0; i < DMA_PER_OPERAND; ++i) refill_one(ha, 0, i, true);
#pragma unroll
      for (int i = 0; i < DMA_B; ++i) refill_one(hb, 1, i, true);
    };

    // Fragment reads of k-substep s of the stage in slot `slot`, one LDS
    // instruction at a time: item f < MI reads A fragment f; the rest read the
    // B fragments (NT: one ds_read_b128 each; NN: two transposing reads each).
    constexpr int READS = MI + (LAYOUT == NT ? NI : 2 * NI);
    auto read_item = [&](int es, int ls, int s, Frags& F, int f) {
      const char* abase = smem + (EARLY == 0 ? es * A_BYTES : RING2 + ls * A_BYTES);
      const char* bbase = smem + (EARLY == 1 ? es * B_TILE : RING2 + ls * B_TILE);
      if (f < MI) {
        F.a[f] = *(const u32x4*)(abase + fa[s] + f * 2048);
      } else if (LAYOUT == NT) {
        const int j = f - MI;
        F.b[j] = *(const u32x4*)(bbase + fb[s] + j * 2048);
      } else {
        const int j = (f - MI) >> 1, h = (f - MI) & 1;
        const u32x2 v = read_tr(bbase + fbn[j] + (s * 32 + 4 * h) * 512);
        F.b[j][2 * h] = v[0];
        F.b[j][2 * h + 1] = v[1];
      }
    };
    // All reads of a substep in item order.  The fences keep that order: the
    // loop head then sees the same sequence of outstanding reads from the
    // prologue as from the loop's back edge, and waits only for the ones the
    // first MFMAs need.
    auto read_frags = [&](int es, int ls, int s, Frags& F) {
#pragma unroll
      for (int f = 0; f < READS; ++f) {
        read_item(es, ls, s, F, f);
        fence();
      }
    };
    // the share of `total` items due before step q of `steps`, spread evenly
    auto share = [](int q, int steps, int total, auto&& item) {
#pragma unroll
      for (int f = (q * total) / steps; f < ((q + 1) * total) / steps; ++f) item(f);
    };

    // Operand order (B fragment first) leaves each lane holding one row of D
    // and four consecutive columns.  Consecutive MFMAs share a B fragment, so
    // the next substep's reads (A fragments first, then B) arrive in the
    // order its MFMAs need them; the A fragments run forwards under even B
    // fragments and backwards under odd ones, so each MFMA changes one
    // operand only.
    auto mfma_pair = [&](const Frags& F, int q) {
#pragma unroll
      for (int t = 2 * q; t < 2 * q + 2; ++t) {
        const int j = t / MI, i = (j & 1) ? MI - 1 - t % MI : t % MI;
        mfma16<T>(acc[i][j], F.b[j], F.a[i]);
      }
    };

    // The rings: stage ks (counted from the task's first step) keeps its
    // EARLY operand's tile in slot ks % 3 of the three-slot ring and the
    // other's in slot ks % 2 of the two-slot ring.  Entering step ks, stage
    // ks has landed, stage ks+1 is in flight, and F0 holds substep 0 of
    // stage ks.  Substep 0 runs its 64 MFMAs in pairs with the reads of
    // substep 1 spread between them (spread, not bunched: a burst of reads
    // fills the LDS command queue and stalls the MFMA issue behind it), and
    // with the loads of stage ks+2's EARLY tile: its slot held stage ks-1,
    // which every wave finished reading before the last barrier.  Substep 1
    // runs BAR_PAIR pairs, then the barrier: stage ks+1 has landed for every
    // wave (only the 8 EARLY loads just issued may be in flight: loads
    // complete in order) and every wave is done reading stage ks, so the rest
    // of substep 1 interleaves the reads of stage ks+1's first substep with
    // the loads of stage ks+2's other tile into stage ks's two-ring slot.
    // The third slot spreads a stage's loads over the whole step instead of
    // its second half, halving the requests in flight at a time (measured:
    // 3-4% faster on the large and ragged shapes).
    Frags F0, F1;
    refill_stage(kbeg, 0);
    refill_stage(kbeg + 1, 1);
    wait_vm_barrier<DMA_PER_OPERAND + DMA_B>();
    read_frags(0, 0, 0, F0);

    int es = 0;  // early-ring slot of stage ks
    for (int ks = kbeg; ks < kend; ++ks) {
      const int ls = (ks - kbeg) & 1;           // two-slot-ring slot of stage ks
      const int es1 = es == 2 ? 0 : es + 1;     // early-ring slot of stage ks+1
      const int es2 = es1 == 2 ? 0 : es1 + 1;   // early-ring slot of stage ks+2
      Half he;
#pragma unroll
      for (int q = 0; q < PAIRS; ++q) {
        share(q, PAIRS, READS, [&](int f) { read_item(es, ls, 1, F1, f); });
        mfma_pair(F0, q);
        fence();
        // (the descriptor's scalar work goes behind the first MFMAs)
        if (q == 0) he = half_setup(ks + 2, es2, EARLY);
        // stages from the third on start at k >= 0: no masks
        share(q, PAIRS, DMA_E, [&](int i) { refill_one(he, EARLY, i, false); });
      }
      const Half hl = half_setup(ks + 2, ls, 1 - EARLY);
#pragma unroll
      for (int q = 0; q < PAIRS; ++q) {
        if (q == BAR_PAIR) {
          wait_vm_barrier<DMA_E>();
          fence();
        }
        if (q >= BAR_PAIR)
          share(q - BAR_PAIR, PAIRS - BAR_PAIR, READS, [&](int f) { read_item(es1, ls ^ 1, 0, F0, f); });
        mfma_pair(F1, q);
        fence();
        if (q >= BAR_PAIR)
          share(q - BAR_PAIR, PAIRS - BAR_PAIR, DMA_L,
                [&](int i) { refill_one(hl, 1 - EARLY, i, false); });
      }
      es = es1;
    }

    wait_vm_barrier<0>();  // every wave is done with the ring; reuse it for staging
    // wait states between the last MFMAs and the first reads of their results
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    fence();

    if (part) {
      // FP32 partial tile, row-major 256 x 256: lane holds row l16 of each
      // 16-row block and columns j*16 + 4*lq .. +3 (16 contiguous bytes);
      // 16 x 16 blocks wholly outside D are skipped (nothing reads them)
      float* w = p.ws + (size_t)(split * p.tiles + u % p.tiles) * (TM * TN) +
                 (size_t)(wm * WTM + l16) * TN + wn * WTN + 4 * lq;
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        if (wm * WTM + i * 16 >= vm) break;
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          if (wn * WTN + j * 16 >= vn) break;
          *(float4*)(w + i * 16 * TN + j * 16) =
              make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      continue;
    }

    // Epilogue: per 32-row band (two 16-row blocks), round, stage the band's
    // 32 x WTN outputs of this wave in LDS (rows of CH 16-byte chunks,
    // swizzled by row), then store 16-byte row chunks.  Each phase is issued
    // whole before the next (all conversions into registers of their own,
    // all LDS writes, all read-backs, then the stores), so that their
    // latencies overlap instead of adding up per chunk.
    constexpr int CH = WTN / 8;       // 16-byte chunks per staged row
    constexpr int RPI = 64 / CH;      // rows per wave instruction of the read-back
    constexpr int NR = 32 / RPI;      // read-back instructions per band
    char* stg = smem + wave * (32 * CH * 16);
    const bool interior = p.d_vec && vm == TM && vn == TN;
#pragma unroll
    for (int band = 0; band < MI / 2; ++band) {
      // lane holds row half*16 + l16 of the band, columns j*16 + 4*lq + 0..3
      // of each block j: 16-byte chunk 2j + lq/2, its lower or upper 8 bytes
      u32x2 v[2][NI];
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          v[half][j][0] = pack2<T>(acc[2 * band + half][j][0], acc[2 * band + half][j][1]);
          v[half][j][1] = pack2<T>(acc[2 * band + half][j][2], acc[2 * band + half][j][3]);
        }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int row = half * 16 + l16;
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          const int chunk = 2 * j + (lq >> 1);
          *(u32x2*)(stg + row * (CH * 16) + ((chunk ^ (row & (CH - 1))) << 4) + (lq & 1) * 8) =
              v[half][j];
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      const int row0 = m0 + wm * WTM + band * 32;
      const int col0 = n0 + wn * WTN;
      const int cc = lane % CH;
      u32x4 r[NR];
#pragma unroll
      for (int t = 0; t < NR; ++t) {
        const int rr = t * RPI + lane / CH;
        r[t] = *(const u32x4*)(stg + rr * (CH * 16) + ((cc ^ (rr & (CH - 1))) << 4));
      }
      __builtin_amdgcn_sched_barrier(0);
      // D is written once and not read again here: non-temporal stores
      // (measured 0.3-1% faster, 4.7% on the large FP8 product)
      if (interior) {
        // the whole tile is inside D and its rows are 16-byte aligned
#pragma unroll
        for (int t = 0; t < NR; ++t) {
          const int rr = t * RPI + lane / CH;
          __builtin_nontemporal_store(r[t], (u32x4*)(p.D + (int64_t)(row0 + rr) * p.ldd + col0 + cc * 8));
        }
      } else {
#pragma unroll
        for (int t = 0; t < NR; ++t) {
          const int rr = t * RPI + lane / CH;
          const int row = row0 + rr;
          const int col = col0 + cc * 8;
          if (row < p.M && col < p.N) {
            uint16_t* dst = p.D + (int64_t)row * p.ldd + col;
            if (p.d_vec && col + 8 <= p.N) {
              __builtin_nontemporal_store(r[t], (u32x4*)dst);
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e)
                if (col + e < p.N) dst[e] = (uint16_t)(r[t][e >> 1] >> ((e & 1) * 16));
            }
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // staging reads done before the next tile refills the ring; the stores
    // drain while the next tile's first loads are in flight
    wait_lds_barrier();
  }
}

// Copy of a rows x cols matrix of 16-bit elements (any leading dimension,
// 2-byte alignment) into a dense, 16-byte aligned rows x dcols matrix
// (dcols = cols rounded up to 8), zero-filling columns cols .. dcols-1: the
// layout the tiled kernel's 16-byte chunk loads need.  Each thread handles
// 8-element chunks of the destination, striding over the grid.
constexpr int64_t REPACK_MAX_BLOCKS = 1 << 16;
__global__ __launch_bounds__(256) void repack(const uint16_t* __restrict__ src, int64_t rows,
                                              int64_t cols, int64_t ld, uint16_t* __restrict__ dst,
                                              int64_t dcols) {
  const int64_t chunks = dcols / 8, total = rows * chunks;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gid < total; gid += stride) {
    const int64_t r = gid / chunks;
    const int64_t c0 = (gid % chunks) * 8;
    const uint16_t* s = src + r * ld + c0;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t lo = c0 + 2 * e < cols ? s[2 * e] : 0u;
      const uint32_t hi = c0 + 2 * e + 1 < cols ? s[2 * e + 1] : 0u;
      w[e] = lo | (hi << 16);
    }
    *(u32x4*)(dst + r * dcols + c0) = (u32x4){w[0], w[1], w[2], w[3]};
  }
}

}  // namespace dg
