// gemm_mx_small_kernel.h -- the FP8 block-scaled small-output kernel for the
// MI355X (gfx950): D = A @ B.T with E4M3 elements, one E8M0 scale per 32 K
// values of each row, FP32 accumulation and one rounding to BF16 (the
// operation of gemm_mx_kernel.h; CMU "TIRx" blog, section "Evaluation",
// "Kernel performance"), for products with M <= 128 and K <= MX_SMALL_K_MAX
// that plan.cpp's mx_small_output gives it.
//
// The FP16 small-output kernel's decomposition (gemm_small_kernel.h) with
// FP8 data and three tile shapes: one workgroup of eight waves per TR x TC
// tile of D, 16 x 16, 32 x 16 or 32 x 32 (the plan takes 16 x 16 for one
// 16-row tile row, else the largest whose tiles still number at least the
// CUs).  Wave w takes the 128-deep K chunks w, w + 8, ... (128 bytes per
// row, the FP16 kernel's 64-deep LDS row and swizzle), streamed through a
// two-slot LDS ring of its own, each slot TR rows of A then TC rows of B;
// one scaled MFMA per 16 x 16 block of the tile and chunk (lane group q
// holds 32 bytes of its row, logical 16-byte chunks q and q + 4, and the
// scale of the chunk's block q, as in the tiled kernel).  The tile's scale
// bytes (TR rows of A and TC of B, K / 32 each) are staged in LDS once,
// before the K loop, read as they are stored (any leading dimension; scale
// 1 outside the rows and blocks).  The waves' FP32 blocks are added in wave
// order, rounded to BF16 and stored.  Every output's sum is the same
// sequence of MFMAs whatever the tile shape, so the three shapes give the
// same bits.
//
// A 32-row tile reads each chunk of B once for two 16-row blocks, a
// 32-column one each chunk of A once for two column blocks: against 16 x 16
// tiles, half the LDS-DMA bytes per MFMA at 32 x 32 (measured, one box,
// both in row order: 128 x 4096 x 4096 19.3 -> 12.1 us, 64 x 4096 x 8192
// 16.8 -> 10.2).
//
// Tile order: the launch's workgroups are dealt to the XCDs round-robin;
// the tiles are laid out XCD by XCD (tile_sched.h's xcd_slot) with the tile
// row varying fastest, so that the tiles of one column strip, which read
// the same rows of B, run together on one XCD and share them in its L2
// (measured: 32 x 8192 x 8192 in 16 x 16 tiles 24.4 us in row order, 16.0
// in this one; in 32 x 32 tiles 18.8 and 12.9).
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

struct MxSmallParams {
  const uint8_t* A;
  const uint8_t* B;
  const uint8_t* SA;
  const uint8_t* SB;
  uint16_t* D;
  int M, N, K;  // K a multiple of 32, at most MX_SMALL_K_MAX
  int lda, ldb, ldsa, ldsb, ldd;
  int tiles_m, tiles_n;  // tiles of the launch's shape in M and N
  int num_xcds;
  int d_vec;  // D rows are 8-byte aligned (4-element stores allowed)
};

// TMB x TNB blocks of 16 x 16 per tile.
template <int TMB, int TNB>
__global__ __launch_bounds__(SMALL_THREADS) void gemm_mx_small(MxSmallParams p) {
  constexpr int RING = 2;                          // chunks in flight per wave
  constexpr int TR = SMALL_TILE * TMB, TC = SMALL_TILE * TNB;
  constexpr int SLOT = (TR + TC) * BKE;            // one chunk: TR rows of A, TC of B
  constexpr int NBMAX = MX_SMALL_K_MAX / GROUP;
  constexpr int SROWS = TR > TC ? TR : TC;
  constexpr int BLOCKS = TMB * TNB;
  constexpr int LOADS = 2 * (TMB + TNB);           // LDS-DMA loads per chunk, 8 rows each
  static_assert(BLOCKS <= SMALL_WAVES, "one wave per block in the final sum");
  static_assert(SMALL_WAVES * BLOCKS * 64 * 16 <= SMALL_WAVES * RING * SLOT,
                "the waves' partial blocks fit in the rings they replace");
  __shared__ __attribute__((aligned(1024))) char ring[SMALL_WAVES * RING * SLOT];
  __shared__ uint8_t scales[2][SROWS][NBMAX];

  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int lane = (int)threadIdx.x & 63;
  const int l16 = lane & 15, lq = lane >> 4;
  const int tile = xcd_slot((int)blockIdx.x, (int)gridDim.x, p.num_xcds);
  const int tm = tile % p.tiles_m, tn = tile / p.tiles_m;
  const int m0 = tm * TR, n0 = tn * TC;
  const int vm = min(TR, p.M - m0), vn = min(TC, p.N - n0);
  const int nb = p.K / GROUP;

  // Loads (as in the FP16 small-output kernel, in bytes): load i of an
  // operand fills rows 8 i .. 8 i + 7 of its tile's 128-byte chunk rows,
  // lane L row 8 i + L / 8 and the logical 16-byte chunk the swizzle stores
  // at physical chunk L % 8; rows past M or N and bytes past K read zeros.
  // (the descriptors are workgroup-uniform: read through readfirstlane so
  // that the compiler keeps them in the scalar registers the loads take)
  i32x4 ra = make_rsrc((uint64_t)(uintptr_t)(p.A + (int64_t)m0 * p.lda),
                       (uint32_t)((vm - 1) * p.lda + p.K));
  i32x4 rb = make_rsrc((uint64_t)(uintptr_t)(p.B + (int64_t)n0 * p.ldb),
                       (uint32_t)((vn - 1) * p.ldb + p.K));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ra[i] = __builtin_amdgcn_readfirstlane(ra[i]);
    rb[i] = __builtin_amdgcn_readfirstlane(rb[i]);
  }
  uint32_t aoff[2 * TMB], boff[2 * TNB];
  int kca[2 * TMB], kcb[2 * TNB];
#pragma unroll
  for (int i = 0; i < 2 * TMB; ++i) {
    const int r = 8 * i + (lane >> 3);
    kca[i] = (lane & 7) ^ swz_k(r);
    aoff[i] = r < vm ? (uint32_t)(r * p.lda + kca[i] * 16) : OOB;
  }
#pragma unroll
  for (int j = 0; j < 2 * TNB; ++j) {
    const int r = 8 * j + (lane >> 3);
    kcb[j] = (lane & 7) ^ swz_k(r);
    boff[j] = r < vn ? (uint32_t)(r * p.ldb + kcb[j] * 16) : OOB;
  }
  const uint32_t wring = lds_addr(ring) + wave * (RING * SLOT);
  auto issue = [&](int t) {
    const int c = wave + SMALL_WAVES * t;
    const uint32_t base = wring + (t % RING) * SLOT;
#pragma unroll
    for (int i = 0; i < 2 * TMB; ++i)
      dma16_at(ra, c * BKE + kca[i] * 16 < p.K ? aoff[i] + c * BKE : OOB, base, i * 1024);
#pragma unroll
    for (int j = 0; j < 2 * TNB; ++j)
      dma16_at(rb, c * BKE + kcb[j] * 16 < p.K ? boff[j] + c * BKE : OOB, base, TR * BKE + j * 1024);
  };
  const int chunks = (p.K + BKE - 1) / BKE;
  const int per_wave = (chunks + SMALL_WAVES - 1) / SMALL_WAVES;

  // The tile's scales by LDS-DMA where every scale row starts 4-byte aligned,
  // K / 32 is a multiple of 4 and a tile's rows span less than 2^31 bytes:
  // waves 0-3 copy A's TR rows (TR / 4 each), waves 4-7 B's TC rows, one
  // 256-byte row of `scales` per instruction (lane L: blocks 4 L .. 4 L + 3;
  // rows past M or N and blocks past K / 32 read zeros, whose data is zero
  // too).  Issued before the ring's first chunks, so that each wave then
  // waits for these loads only.
  const int64_t sld = p.ldsa > p.ldsb ? p.ldsa : p.ldsb;
  const bool sdma = nb > 0 && (nb & 3) == 0 &&
                    ((((uintptr_t)p.SA | (uintptr_t)p.SB) & 3) == 0) &&
                    (((p.ldsa | p.ldsb) & 3) == 0) &&
                    (SROWS - 1) * sld + nb < ((int64_t)1 << 31);
  if (sdma) {
    const int op = wave >> 2;
    const int vr = op ? vn : vm;
    const int ld = op ? p.ldsb : p.ldsa;
    i32x4 rs = make_rsrc((uint64_t)(uintptr_t)(op ? p.SB + (int64_t)n0 * p.ldsb
                                                  : p.SA + (int64_t)m0 * p.ldsa),
                         (uint32_t)((vr - 1) * ld + nb));
#pragma unroll
    for (int i = 0; i < 4; ++i) rs[i] = __builtin_amdgcn_readfirstlane(rs[i]);
    auto rows = [&](auto per) {  // this wave's `per` rows of its operand
      const int r0 = per * (wave & 3);
      const uint32_t sbase = lds_addr(&scales[op][r0][0]);
#pragma unroll
      for (int i = 0; i < per; ++i) {
        const int row = r0 + i;
        dma4_at(rs, row < vr && 4 * lane < nb ? (uint32_t)(row * ld + 4 * lane) : OOB, sbase,
                i * NBMAX);
      }
    };
    if (op == 0)
      rows(std::integral_constant<int, TR / 4>());
    else
      rows(std::integral_constant<int, TC / 4>());
  }
  if (per_wave > 0)
    for (int t = 0; t < RING; ++t) issue(t);

  // Otherwise the tile's scales are loaded as bytes, while the first chunks
  // load.  Thread t takes operand t / 256 (A, then B), rows (t / 16) % 16 +
  // 16 s of the tile (s below TMB or TNB) and blocks t % 16 + 16 j: per row,
  // its PER bytes are loaded first (the wait for them also waits for the
  // first chunks), every load unconditional (from an address inside the
  // matrix: row 0 of the tile for rows past M or N, block 0 for blocks past
  // K / 32), so that all of them are in flight at once, then stored (scale 1
  // for rows past M or N; blocks past K / 32 are never read).  The shares
  // follow from shifts of t: index arithmetic with K / 32 as divisor
  // measured ~1.5 us per call.  (With K = 0 there are no scales, and the
  // scale pointers may be null.)
  static_assert(SMALL_THREADS == 2 * SMALL_TILE * 16 && NBMAX % 16 == 0, "one thread per 16 blocks");
  if (sdma) {
    // this wave's scale rows have landed; the ring's first two chunks may
    // still be in flight
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(LOADS * RING) : "memory");
  } else if (nb > 0) {
    constexpr int PER = NBMAX / 16;
    const int t = (int)threadIdx.x;
    const int op = t >> 8, r16 = (t >> 4) & 15, b0 = t & 15;
    const int vr = op ? vn : vm;
    const int passes = op ? TNB : TMB;
    for (int s = 0; s < passes; ++s) {
      const int row = SMALL_TILE * s + r16;
      const bool rin = row < vr;
      const uint8_t* src = op ? p.SB + (int64_t)(n0 + (rin ? row : 0)) * p.ldsb
                              : p.SA + (int64_t)(m0 + (rin ? row : 0)) * p.ldsa;
      int v[PER];
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int b = b0 + 16 * j;
        v[j] = src[b < nb ? b : 0];
      }
      // Every loaded value is stored (blocks past K / 32 with scale 1; they
      // are never read): a load whose value went unused would stay pending,
      // as far as the compiler knows, into the K loop, where it would then
      // wait for all loads in flight (the ring's included) at every chunk.
#pragma unroll
      for (int j = 0; j < PER; ++j) {
        const int b = b0 + 16 * j;
        scales[op][row][b] = (uint8_t)(rin && b < nb ? v[j] : 127);  // 127: scale 1
      }
    }
  }
  __syncthreads();

  // Fragment reads: lane (l16, lq) reads row l16 of a 16-row block, logical
  // chunks lq and lq + 4.
  const int sw = swz_k(l16);
  const int fr0 = l16 * BKE + ((lq ^ sw) << 4);
  const int fr1 = l16 * BKE + (((lq + 4) ^ sw) << 4);
  f32x4 acc[TMB][TNB];
#pragma unroll
  for (int i = 0; i < TMB; ++i)
#pragma unroll
    for (int j = 0; j < TNB; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if (per_wave > 0) {
    for (int t = 0; t < per_wave; ++t) {
      asm volatile("s_waitcnt vmcnt(%0)" : : "n"(LOADS * (RING - 1)) : "memory");
      const char* slot = ring + (wave * RING + t % RING) * SLOT;
      const int blk = (wave + SMALL_WAVES * t) * (BKE / GROUP) + lq;
      i32x8 af[TMB], bf[TNB];
      int sa[TMB], sb[TNB];
#pragma unroll
      for (int i = 0; i < TMB; ++i) {
        const u32x4 x = *(const u32x4*)(slot + i * SMALL_TILE * BKE + fr0);
        const u32x4 y = *(const u32x4*)(slot + i * SMALL_TILE * BKE + fr1);
        af[i] = i32x8{(int)x[0], (int)x[1], (int)x[2], (int)x[3],
                      (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
        sa[i] = blk < nb ? scales[0][SMALL_TILE * i + l16][blk] : 127;
      }
#pragma unroll
      for (int j = 0; j < TNB; ++j) {
        const u32x4 x = *(const u32x4*)(slot + (TR + j * SMALL_TILE) * BKE + fr0);
        const u32x4 y = *(const u32x4*)(slot + (TR + j * SMALL_TILE) * BKE + fr1);
        bf[j] = i32x8{(int)x[0], (int)x[1], (int)x[2], (int)x[3],
                      (int)y[0], (int)y[1], (int)y[2], (int)y[3]};
        sb[j] = blk < nb ? scales[1][SMALL_TILE * j + l16][blk] : 127;
      }
      // srcA the B fragment (its scale sb), srcB the A fragment (sa): each
      // lane ends up holding one row of D, four columns; E4M3 operands
#pragma unroll
      for (int i = 0; i < TMB; ++i)
#pragma unroll
        for (int j = 0; j < TNB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af[i], acc[i][j], 0, 0,
                                                                       0, sb[j], 0, sa[i]);
      // the slot's reads are done (the MFMAs took their data): refill it
      asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
      issue(t + RING);
    }
    // no LDS-DMA write may land after the wave ends
    asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
  }

  // The waves' blocks, through the rings' LDS (once every wave is done with
  // its ring): block b of wave w at part[w][b]; wave b adds block b's eight
  // in wave order.  Lane (l16, lq) of block (i, j): D row m0 + 16 i + l16,
  // columns n0 + 16 j + 4 lq .. +3.
  __syncthreads();
  f32x4(*part)[BLOCKS][64] = reinterpret_cast<f32x4(*)[BLOCKS][64]>(ring);
#pragma unroll
  for (int i = 0; i < TMB; ++i)
#pragma unroll
    for (int j = 0; j < TNB; ++j) part[wave][i * TNB + j][lane] = acc[i][j];
  __syncthreads();
  if (wave >= BLOCKS) return;
  f32x4 s = part[0][wave][lane];
#pragma unroll
  for (int w = 1; w < SMALL_WAVES; ++w) s += part[w][wave][lane];
  const int row = m0 + SMALL_TILE * (wave / TNB) + l16;
  const int col = n0 + SMALL_TILE * (wave % TNB) + 4 * lq;
  if (row >= p.M || col >= p.N) return;
  u32x2 v;
  v[0] = pack2<__bf16>(s[0], s[1]);
  v[1] = pack2<__bf16>(s[2], s[3]);
  uint16_t* dst = p.D + (int64_t)row * p.ldd + col;
  if (p.d_vec && col + 4 <= p.N) {
    *(u32x2*)dst = v;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (col + e < p.N) dst[e] = (uint16_t)(v[e >> 1] >> ((e & 1) * 16));
  }
}

}  // namespace mx
}  // namespace dg
