// gemm_small_kernel.h -- the small-output kernel for the MI355X (gfx950):
// D = A @ B.T or D = A @ B (FP16 or BF16) with M <= 128, such as a 128 x
// 128 output, whose one 256 x 128 tile would leave almost every CU idle, a
// single row of 16 x 16 tiles (M <= 16) of any width, or a few rows of
// A @ B.T tiles over a short enough K.  (Which products run it:
// small_output in plan.cpp.)
//
// The product is the one of gemm_kernel.h (FP32 accumulation of the K
// blocks' partial products, one rounding to the output type; TileFoundry's
// schedule tutorial, section 1).  What changes is the decomposition:
//   * the output is cut into 16 x 16 tiles, one workgroup each (64 for a
//     128 x 128 output), so that many CUs stream the operands at once; for
//     A @ B.T also 32 x 16 or 32 x 32 tiles (the plan takes the largest
//     whose tiles still number at least the CUs, 16 x 16 for one 16-row tile
//     row): a 32-row tile reads each chunk of B once for two row blocks, a
//     32-column one each chunk of A once for two column blocks, and every
//     block's sum is the same sequence of MFMAs whatever the tile shape;
//   * inside a workgroup, eight waves split K: wave w takes the 64-deep K
//     chunks w, w + 8, w + 16, ..., each wave accumulating its own FP32
//     blocks with v_mfma_f32_16x16x32, two accumulators per 16 x 16 block
//     (one per 32-deep half of a chunk);
//   * each wave streams its chunks through a ring of its own in LDS: the
//     LDS-DMA loads of gemm_kernel.h (eight lanes per 128-byte row segment,
//     the same XOR swizzle), two chunks in flight, each wave waiting only
//     for its own loads (no barrier in the K loop).  (Fragments loaded
//     straight into registers put 16 rows under every 16 lanes of a load:
//     measured, that held a CU to ~37 GB/s.)
//   * the eight waves' blocks are summed through LDS in wave order, a fixed
//     order (results are reproducible), then rounded and stored;
//   * the tiles are dealt to the XCDs in runs (tile_sched.h's xcd_slot):
//     for A @ B.T with the tile row varying fastest, so that the tiles that
//     read the same rows of B run on one XCD and share them in its L2 (one
//     tile row: consecutive strips of B per XCD; measured 16 x 8192 x 8192
//     25.3 -> 20.8 us and 1 x 16384 x 4096 22.7 -> 19.7 against row order).
// Where tiles reach past M or N, or chunks past K, the loads read zeros
// (offsets past the buffer's range) and the stores are masked.
//
// A @ B (B row-major K x N): a chunk's B tile is 64 k rows of 32 bytes (the
// tile's 16 columns), still two 16-byte loads per lane, read into MFMA
// fragments (eight consecutive k of one column per lane) by transposing LDS
// reads, as the tiled kernel's A @ B does.  Four tiles side by side share
// B's 128-byte lines, so its tiles go to the XCDs row by row: tiles that
// share lines run on one XCD and share its L2.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cdna_ops.h"
#include "tile_config.h"
#include "tile_sched.h"

namespace dg {

// (SMALL_TILE, SMALL_WAVES and the planning limits: tile_config.h)

struct SmallParams {
  const uint16_t* A;
  const uint16_t* B;
  uint16_t* D;
  int M, N;
  int K;     // (A @ B: rows of B)
  int K8;    // K rounded up to 8 (A, and B for A @ B.T, hold zeros in [K, K8))
  int N8;    // (A @ B) N rounded up to 8: B's columns that may be read
  int lda, ldb, ldd;
  int tiles_m, tiles_n;  // tiles of the launch's shape in M and N
  int num_xcds;          // XCDs of the device, for the tile order
  int d_vec;     // D rows are 8-byte aligned (4-element stores allowed)
};

// LDS position of row k of a chunk's A @ B tile (64 rows of 32 bytes): the
// 128-byte half flips where bit 3 of k is set, so that the transposing
// reads of the two 16-lane blocks of a half-wave (rows 8 apart) fall in
// different banks.
__device__ __forceinline__ int nn_row_pos(int k) { return (32 * k) ^ (((k >> 3) & 1) << 7); }

// c += b-fragment rows x a-fragment columns over 32 k, through the builtin:
// with only two accumulators live the compiler keeps them in place, and it
// adds the wait states between the dependent MFMAs of a chain itself.
template <typename T>
__device__ __forceinline__ f32x4 mfma16_chain(f32x4 c, u32x4 b, u32x4 a);
template <>
__device__ __forceinline__ f32x4 mfma16_chain<_Float16>(f32x4 c, u32x4 b, u32x4 a) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, b),
                                                 __builtin_bit_cast(f16x8, a), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4 mfma16_chain<__bf16>(f32x4 c, u32x4 b, u32x4 a) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b),
                                                  __builtin_bit_cast(bf16x8, a), c, 0, 0, 0);
}

// TMB x TNB blocks of 16 x 16 per tile (A @ B: one).
template <typename T, int LAYOUT, int TMB, int TNB>
__global__ __launch_bounds__(SMALL_THREADS) void gemm_small(SmallParams p) {
  static_assert(LAYOUT == NT || (TMB == 1 && TNB == 1), "A @ B takes 16 x 16 tiles");
  // Chunks in flight per wave.  Two (72 KiB of LDS per workgroup with 16 x
  // 16 tiles, so two workgroups fit a CU) measured faster than four (136
  // KiB, one per CU) on every shape tried: 4.4 against 4.9 us at 128 x 128
  // x 4096, 22.7 against 24.3 at 1 x 16384 x 4096, 11.6 against 12.3 at 128
  // x 128 x 16384.
  constexpr int RING = 2;
  constexpr int TR = SMALL_TILE * TMB, TC = SMALL_TILE * TNB;
  constexpr int SLOT = (TR + TC) * 128;  // one chunk: TR rows of A, then the B tile, 128 B each
  constexpr int BLOCKS = TMB * TNB;
  constexpr int LOADS = 2 * (TMB + TNB);  // LDS-DMA loads per chunk, 8 rows each
  static_assert(BLOCKS <= SMALL_WAVES, "one wave per block in the final sum");
  static_assert(SMALL_WAVES * BLOCKS * 64 * 16 <= SMALL_WAVES * RING * SLOT,
                "the waves' partial blocks fit in the rings they replace");
  __shared__ __attribute__((aligned(1024))) char ring[SMALL_WAVES * RING * SLOT];

  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int lane = (int)threadIdx.x & 63;
  const int l16 = lane & 15, lq = lane >> 4;
  // Tile order (tile_sched.h's xcd_slot deals the XCDs runs of consecutive
  // slots): A @ B.T with the tile row varying fastest, so that the tiles of
  // a column strip, which read the same rows of B, run on one XCD (with one
  // tile row: consecutive strips of B per XCD); A @ B row by row, so that
  // the four tiles side by side that share B's 128-byte lines run on one XCD.
  const int tile = xcd_slot((int)blockIdx.x, (int)gridDim.x, p.num_xcds);
  const int tm = LAYOUT == NT ? tile % p.tiles_m : tile / p.tiles_n;
  const int tn = LAYOUT == NT ? tile / p.tiles_m : tile % p.tiles_n;
  const int m0 = tm * TR, n0 = tn * TC;
  const int vm = min(TR, p.M - m0), vn = min(TC, p.N - n0);

  // Loads: descriptors over the tile's valid rows and columns [0, K8).
  // Load instruction i of an operand fills rows 8 i .. 8 i + 7 of its TR
  // (or TC) x 128 B tile: lane L takes row 8 i + L / 8 and the logical
  // 16-byte chunk the swizzle stores at physical chunk L % 8.  Rows past M
  // or N and chunks at or past K8 get an offset past the range: zeros.
  const i32x4 ra = make_rsrc((uint64_t)(uintptr_t)(p.A + (int64_t)m0 * p.lda),
                             (uint32_t)(((vm - 1) * p.lda + p.K8) * 2));
  const i32x4 rb = make_rsrc((uint64_t)(uintptr_t)(p.B + (int64_t)n0 * p.ldb),
                             (uint32_t)(((vn - 1) * p.ldb + p.K8) * 2));
  uint32_t aoff[2 * TMB], boff[2 * TNB];
  int kca[2 * TMB], kcb[2 * TNB];
#pragma unroll
  for (int i = 0; i < 2 * TMB; ++i) {
    const int r = 8 * i + (lane >> 3);
    kca[i] = (lane & 7) ^ swz_k(r);
    aoff[i] = r < vm ? (uint32_t)((r * p.lda + kca[i] * 8) * 2) : OOB;
  }
#pragma unroll
  for (int j = 0; j < 2 * TNB; ++j) {
    const int r = 8 * j + (lane >> 3);
    kcb[j] = (lane & 7) ^ swz_k(r);
    boff[j] = r < vn ? (uint32_t)((r * p.ldb + kcb[j] * 8) * 2) : OOB;
  }
  // A @ B: load i of the B tile fills LDS bytes 1024 i .. +1023 of it; lane
  // L's 16 bytes there hold row kn[i] (nn_row_pos inverted), column chunk
  // L % 2 of the tile (columns n0 + 8 (L % 2) .. +7); chunks at or past N8
  // read zeros.  The offsets are relative to the chunk's first row (the
  // descriptor is rebased per chunk, so they stay small).
  int kn[2];
  uint32_t bnoff[2];
  const bool ncol = n0 + 8 * (lane & 1) < p.N8;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int b = 1024 * i + 16 * lane;
    kn[i] = (b >> 5) ^ (((b >> 8) & 1) << 2);
    bnoff[i] = ncol ? (uint32_t)((kn[i] * p.ldb + 8 * (lane & 1)) * 2) : OOB;
  }
  const uint32_t wring = lds_addr(ring) + wave * (RING * SLOT);
  // chunk t of this wave (K chunk wave + 8 t) into ring slot t % RING
  auto issue = [&](int t) {
    const int c = wave + SMALL_WAVES * t;
    const uint32_t base = wring + (t % RING) * SLOT;
    if constexpr (LAYOUT == NT) {
#pragma unroll
      for (int i = 0; i < 2 * TMB; ++i)
        dma16_at(ra, c * 64 + kca[i] * 8 < p.K8 ? aoff[i] + c * 128 : OOB, base, i * 1024);
#pragma unroll
      for (int j = 0; j < 2 * TNB; ++j)
        dma16_at(rb, c * 64 + kcb[j] * 8 < p.K8 ? boff[j] + c * 128 : OOB, base,
                 TR * 128 + j * 1024);
    } else {
      // B rows c*64 .. of the tile's columns, the range ending with the
      // last row of B (none for chunks past K); the descriptor is
      // wave-uniform: readfirstlane keeps it in the scalar registers the
      // load takes
      const int k0 = c * 64;
      const int rows = min(64, p.K - k0);
      const uint64_t a = (uint64_t)(uintptr_t)(p.B + (int64_t)k0 * p.ldb + n0);
      i32x4 rbn = make_rsrc(a, rows > 0 ? (uint32_t)(((rows - 1) * p.ldb + (p.N8 - n0)) * 2) : 0u);
#pragma unroll
      for (int e = 0; e < 4; ++e) rbn[e] = __builtin_amdgcn_readfirstlane(rbn[e]);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        dma16_at(ra, c * 64 + kca[i] * 8 < p.K8 ? aoff[i] + c * 128 : OOB, base, i * 1024);
        dma16_at(rbn, kn[i] < rows ? bnoff[i] : OOB, base, 2048 + i * 1024);
      }
    }
  };
  // Fragment reads: lane (l16, lq) reads row l16, logical chunk 4 s + lq
  // (half s of the chunk).
  const int fr0 = l16 * 128 + ((lq ^ swz_k(l16)) << 4);
  const int fr1 = l16 * 128 + (((4 + lq) ^ swz_k(l16)) << 4);
  // A @ B, transposing reads: for half s and read h, lane (l16, lq) supplies
  // row 32 s + 8 lq + l16 / 4 + 4 h, columns 4 (l16 % 4) .. +3, and receives
  // column l16 at four consecutive k (8 lq + 4 h .. +3 of the half)
  int ft[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) ft[h] = nn_row_pos(8 * lq + (l16 >> 2) + 4 * h) + 8 * (l16 & 3);

  // Every wave runs the same number of chunks (chunks past K load zeros and
  // add nothing), so that the count of loads in flight is the same at every
  // wait: RING - 1 later chunks of LOADS loads each.  Each 16 x 16 block
  // (i, j) of the tile has two accumulators, one per 32-deep half of a chunk.
  const int chunks = (p.K8 + 63) / 64;
  const int per_wave = (chunks + SMALL_WAVES - 1) / SMALL_WAVES;
  f32x4 acc0[TMB][TNB], acc1[TMB][TNB];
#pragma unroll
  for (int i = 0; i < TMB; ++i)
#pragma unroll
    for (int j = 0; j < TNB; ++j) acc0[i][j] = acc1[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if (per_wave > 0) {  // (K = 0: no loads at all, D is zero)
    for (int t = 0; t < RING; ++t) issue(t);
    for (int t = 0; t < per_wave; ++t) {
      asm volatile("s_waitcnt vmcnt(%0)" : : "n"(LOADS * (RING - 1)) : "memory");
      const char* slot = ring + (wave * RING + t % RING) * SLOT;
      u32x4 a0[TMB], a1[TMB], b0[TNB], b1[TNB];
#pragma unroll
      for (int i = 0; i < TMB; ++i) {
        a0[i] = *(const u32x4*)(slot + i * 2048 + fr0);
        a1[i] = *(const u32x4*)(slot + i * 2048 + fr1);
      }
      if constexpr (LAYOUT == NT) {
#pragma unroll
        for (int j = 0; j < TNB; ++j) {
          b0[j] = *(const u32x4*)(slot + (TR + SMALL_TILE * j) * 128 + fr0);
          b1[j] = *(const u32x4*)(slot + (TR + SMALL_TILE * j) * 128 + fr1);
        }
      } else {
        // (row 32 s + k of the tile: nn_row_pos adds 1024 s, bit 3 of k
        // unchanged)
        const u32x2 x0 = read_tr(slot + 2048 + ft[0]);
        const u32x2 x1 = read_tr(slot + 2048 + ft[1]);
        const u32x2 y0 = read_tr(slot + 2048 + 1024 + ft[0]);
        const u32x2 y1 = read_tr(slot + 2048 + 1024 + ft[1]);
        b0[0] = (u32x4){x0[0], x0[1], x1[0], x1[1]};
        b1[0] = (u32x4){y0[0], y0[1], y1[0], y1[1]};
      }
#pragma unroll
      for (int i = 0; i < TMB; ++i)
#pragma unroll
        for (int j = 0; j < TNB; ++j) {
          acc0[i][j] = mfma16_chain<T>(acc0[i][j], b0[j], a0[i]);
          acc1[i][j] = mfma16_chain<T>(acc1[i][j], b1[j], a1[i]);
        }
      // the slot's reads are done (the MFMAs took their data): refill it
      asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory");
      issue(t + RING);
    }
    // no LDS-DMA write may land after the wave ends
    asm volatile("s_waitcnt vmcnt(0)" : : : "memory");
  }

  // The waves' blocks, through the rings' LDS (once every wave is done with
  // its ring): block b of wave w at part[w][b]; wave b adds block b's eight
  // in wave order.  Lane (l16, lq) of block (i, j) holds D row m0 + 16 i +
  // l16, columns n0 + 16 j + 4 lq .. +3.
  __syncthreads();
  f32x4(*part)[BLOCKS][64] = reinterpret_cast<f32x4(*)[BLOCKS][64]>(ring);
#pragma unroll
  for (int i = 0; i < TMB; ++i)
#pragma unroll
    for (int j = 0; j < TNB; ++j) part[wave][i * TNB + j][lane] = acc0[i][j] + acc1[i][j];
  __syncthreads();
  if (wave >= BLOCKS) return;
  f32x4 s = part[0][wave][lane];
#pragma unroll
  for (int w = 1; w < SMALL_WAVES; ++w) s += part[w][wave][lane];
  const int row = m0 + SMALL_TILE * (wave / TNB) + l16;
  const int col = n0 + SMALL_TILE * (wave % TNB) + 4 * lq;
  if (row >= p.M || col >= p.N) return;
  u32x2 v;
  v[0] = pack2<T>(s[0], s[1]);
  v[1] = pack2<T>(s[2], s[3]);
  uint16_t* dst = p.D + (int64_t)row * p.ldd + col;
  if (p.d_vec && col + 4 <= p.N) {
    *(u32x2*)dst = v;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (col + e < p.N) dst[e] = (uint16_t)(v[e >> 1] >> ((e & 1) * 16));
  }
}

}  // namespace dg
