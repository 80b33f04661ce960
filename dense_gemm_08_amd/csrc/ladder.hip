// ladder.hip -- the optimisation steps of "TIRx GEMM on Blackwell" (its
// sections V3 to V9, "the journey"), rebuilt one idea at a time for gfx950,
// to measure what each idea buys on this hardware.  D = A @ B.T in FP16 only
// (the page's workload), on shapes that divide the tiles.  These kernels are
// deliberately plain: each level adds one mechanism to the level before and
// nothing else; the library's own kernel (dense_gemm.hip) is the last level.
//
//   level 1 (V3)  one 128 x 128 tile per workgroup, all tiles launched at
//                 once; per K step the threads copy A and B through registers
//                 into LDS, then compute (load and compute do not overlap)
//   level 2 (V4)  the copy engine: LDS-DMA loads (buffer_load ... lds) move
//                 the tiles instead of the threads (the role of TMA)
//   level 3 (V5)  two LDS stages: the loads of step k+1 are in flight while
//                 step k is computed
//   level 4 (V6)  persistent workgroups, one per CU, walking the tiles in the
//                 grouped order with the XCD remap (tile_sched.h)
//   level 5 (V8/V9) a 256 x 256 tile per workgroup: each staged A and B tile
//                 now feeds two wave rows / columns (the pages reach the same
//                 reuse with a 2-CTA cluster and a second consumer)
//   level 6       the library kernel: the same tile with the fine-grained
//                 schedule (reads and loads spread between MFMA pairs, one
//                 barrier per stage, descriptors rebased per step)
//   level 7 (V7)  level 4 with warp specialization: a fifth wave issues every
//                 LDS-DMA load while the four computing waves only read LDS
//                 and run MFMAs, the stages handed over by two workgroup
//                 barriers per step (the page's producer warp and its
//                 full/empty barriers; numbered last to keep levels 1-6)
//   level 8       level 5 with v_mfma_f32_32x32x16_f16 in place of the
//                 16 x 16 x 32 MFMA (four 32 x 32 blocks per wave direction,
//                 four 16-deep substeps per stage): the same tile, loads,
//                 LDS layout and schedule, so the two levels differ only in
//                 the MFMA shape (not a step of the page; the comparison
//                 behind the library kernel's choice of 16 x 16 x 32)
//   level 9       level 5 with eight waves (two per SIMD) of 128 x 64 in
//                 place of four of 128 x 128: while one wave of a SIMD waits
//                 (barrier, LDS) the other can issue MFMAs, at 1.5 times the
//                 LDS fragment reads (a comparison, not a page step)
//
// The library kernel does not specialize: with 256 x 256 tiles one wave per
// SIMD holds 256 accumulator registers, leaving no room for a fifth wave,
// and LDS-DMA loads are issued asynchronously by the computing waves
// themselves.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cdna_ops.h"
#include "dense_gemm.h"
#include "tile_sched.h"

namespace dg {

// current device's CU and XCD counts, checked to be a gfx950 (dense_gemm.hip)
dense_gemm_status device_topology(int* cus, int* xcds);

namespace ladder {

constexpr int BK = 64;  // K depth of one stage (128-byte rows)

struct LParams {
  const uint16_t* A;
  const uint16_t* B;
  uint16_t* D;
  int M, N, K;
  int lda, ldb, ldd;
  int tiles_m, tiles_n, num_tiles;
  int num_xcds;  // XCDs of the device (the scheduler's L2 remap)
};

template <int TILE, bool DMA, int STAGES, bool PERSIST, int MF = 16, int NW = 4>
__global__ __launch_bounds__(NW * 64) void ladder_kernel(LParams p) {
  static_assert(MF == 16 || MF == 32, "16 x 16 x 32 or 32 x 32 x 16 MFMAs");
  static_assert(NW == 4 || (NW == 8 && MF == 16), "2 x 2 waves, or 2 x 4 with 16 x 16 x 32");
  constexpr int W = TILE / 2;                 // wave tile rows (2 wave rows)
  constexpr int WN = TILE / (NW / 2);         // wave tile columns (NW / 2 wave columns)
  constexpr int MI = W / 16, NI = WN / 16;    // 16 x 16 MFMA blocks per wave
  constexpr int MB = W / 32;                  // 32 x 32 MFMA blocks per wave and direction
  constexpr int OPB = TILE * BK * 2;          // bytes of one operand tile per stage
  constexpr int STB = 2 * OPB;                // A tile, then B tile
  constexpr int LOADS = OPB / (NW * 64 * 16);  // 16-byte loads per thread per operand
  __shared__ __attribute__((aligned(1024))) char smem[STAGES * STB];
  const uint32_t lds0 = lds_addr(smem);

  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int wm = wave / (NW / 2), wn = wave % (NW / 2);
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15, lq = lane >> 4;
  const int nk = p.K / BK;

  const int first = PERSIST ? xcd_slot(blockIdx.x, gridDim.x, p.num_xcds) : blockIdx.x;
  const int stride = PERSIST ? gridDim.x : p.num_tiles;
  for (int t = first; t < p.num_tiles; t += stride) {
    int tm, tn;
    if (PERSIST) {
      tile_of_task(t, p.tiles_m, p.tiles_n, p.tiles_m < 8 ? p.tiles_m : 8, &tm, &tn);
    } else {
      tm = t / p.tiles_n;
      tn = t % p.tiles_n;
    }
    const uint16_t* a0 = p.A + (int64_t)tm * TILE * p.lda;
    const uint16_t* b0 = p.B + (int64_t)tn * TILE * p.ldb;

    // (only one of the two accumulator sets is used: the compiler drops the
    // other, MF being a template argument)
    f32x4 acc[MI][NI];
    f32x16 acc32[MB][MB];
    if (MF == 16) {
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NI; ++j) acc[i][j] = (f32x4){};
    } else {
#pragma unroll
      for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int j = 0; j < MB; ++j) acc32[i][j] = (f32x16){};
    }
    fence();

    // Load i of this thread covers tile row r = (LOADS*wave + i)*8 + lane/8
    // and the logical 16-byte chunk that the swizzle puts at physical chunk
    // lane % 8, so each wave instruction fills 1 KiB of LDS contiguously.
    auto row_of = [&](int i) { return (LOADS * wave + i) * 8 + (lane >> 3); };
    auto chunk_of = [&](int i) { return (lane & 7) ^ swz_k(row_of(i)); };
    const i32x4 ra = make_rsrc((uint64_t)(uintptr_t)a0, (uint32_t)(((int64_t)(TILE - 1) * p.lda + p.K) * 2));
    const i32x4 rb = make_rsrc((uint64_t)(uintptr_t)b0, (uint32_t)(((int64_t)(TILE - 1) * p.ldb + p.K) * 2));
    auto load = [&](int ks, int slot) {
      const int k0 = ks * BK;
      if (DMA) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
          const int r = row_of(i), c = chunk_of(i);
          const uint32_t m0 = lds0 + slot * STB + (LOADS * wave + i) * 1024;
          dma16(ra, (uint32_t)((r * p.lda + k0 + c * 8) * 2), m0);
          dma16(rb, (uint32_t)((r * p.ldb + k0 + c * 8) * 2), m0 + OPB);
        }
      } else {
        u32x4 va[LOADS], vb[LOADS];
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
          const int r = row_of(i), c = chunk_of(i);
          va[i] = *(const u32x4*)(a0 + (int64_t)r * p.lda + k0 + c * 8);
          vb[i] = *(const u32x4*)(b0 + (int64_t)r * p.ldb + k0 + c * 8);
        }
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
          char* dst = smem + slot * STB + (LOADS * wave + i) * 1024 + lane * 16;
          *(u32x4*)dst = va[i];
          *(u32x4*)(dst + OPB) = vb[i];
        }
      }
    };
    // Two 32-deep substeps (four 16-deep ones for 32 x 32 x 16 MFMAs): read
    // the wave's A and B fragments, then its MFMAs.
    auto compute = [&](int slot) {
      const char* base = smem + slot * STB;
      if (MF == 32) {
        // lane l holds row l % 32 of a 32-row fragment and k = 8 (l / 32) ..
        // +7 of the substep's 16: chunk 2 s + l / 32 of the 128-byte row
        const int r32 = lane & 31, h = lane >> 5;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int off = (((2 * s + h) ^ swz_k(r32)) << 4);
          u32x4 a[MB], b[MB];
#pragma unroll
          for (int i = 0; i < MB; ++i) a[i] = *(const u32x4*)(base + (wm * W + i * 32 + r32) * 128 + off);
#pragma unroll
          for (int j = 0; j < MB; ++j)
            b[j] = *(const u32x4*)(base + OPB + (wn * W + j * 32 + r32) * 128 + off);
#pragma unroll
          for (int j = 0; j < MB; ++j)
#pragma unroll
            for (int i = 0; i < MB; ++i) mfma32_f16(acc32[i][j], b[j], a[i]);
        }
        return;
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int off = (((4 * s + lq) ^ swz_k(l16)) << 4);
        u32x4 a[MI], b[NI];
#pragma unroll
        for (int i = 0; i < MI; ++i) a[i] = *(const u32x4*)(base + (wm * W + i * 16 + l16) * 128 + off);
#pragma unroll
        for (int j = 0; j < NI; ++j) b[j] = *(const u32x4*)(base + OPB + (wn * WN + j * 16 + l16) * 128 + off);
#pragma unroll
        for (int j = 0; j < NI; ++j)
#pragma unroll
          for (int i = 0; i < MI; ++i) mfma16<_Float16>(acc[i][j], b[j], a[i]);
      }
    };

    if (STAGES == 1) {
      for (int ks = 0; ks < nk; ++ks) {
        load(ks, 0);
        if (DMA)
          wait_vm_barrier<0>();  // the DMA loads have landed
        else
          wait_lds_barrier();    // the threads' LDS writes are done
        compute(0);
        wait_lds_barrier();  // every wave is done reading before the next load
      }
    } else {
      load(0, 0);
      for (int ks = 0; ks < nk; ++ks) {
        if (ks + 1 < nk) {
          load(ks + 1, (ks + 1) & 1);
          wait_vm_barrier<2 * LOADS>();  // step ks has landed; step ks+1 in flight
        } else {
          wait_vm_barrier<0>();
        }
        compute(ks & 1);
        wait_lds_barrier();  // slot ks & 1 is refilled by the next iteration's load
      }
    }

    // wait states between the last MFMAs and the reads of their results
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    fence();
    if (MF == 32) {
      // lane l holds row l % 32 of each 32 x 32 block and, for g = 0..3, the
      // four columns 8 g + 4 (l / 32) .. +3 in accumulators 4 g .. 4 g + 3
      const int r32 = lane & 31, h = lane >> 5;
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const int row = tm * TILE + wm * W + i * 32 + r32;
#pragma unroll
        for (int j = 0; j < MB; ++j)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int col = tn * TILE + wn * W + j * 32 + 8 * g + 4 * h;
            u32x2 v;
            v[0] = pack2<_Float16>(acc32[i][j][4 * g], acc32[i][j][4 * g + 1]);
            v[1] = pack2<_Float16>(acc32[i][j][4 * g + 2], acc32[i][j][4 * g + 3]);
            *(u32x2*)(p.D + (int64_t)row * p.ldd + col) = v;
          }
      }
      continue;
    }
    // lane holds row l16 of each 16-row block and 4 consecutive columns
#pragma unroll
    for (int i = 0; i < MI; ++i) {
      const int row = tm * TILE + wm * W + i * 16 + l16;
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const int col = tn * TILE + wn * WN + j * 16 + 4 * lq;
        u32x2 v;
        v[0] = pack2<_Float16>(acc[i][j][0], acc[i][j][1]);
        v[1] = pack2<_Float16>(acc[i][j][2], acc[i][j][3]);
        *(u32x2*)(p.D + (int64_t)row * p.ldd + col) = v;
      }
    }
  }
}

// Level 7: 128 x 128 tiles, two LDS stages, persistent grouped order (as
// level 4), and five waves: waves 0-3 compute (2 x 2, 64 x 64 each), wave 4
// loads.  Per K step every wave passes two barriers: "full" (the producer
// has waited for step ks's loads; the consumers may read its slot) and
// "empty" (the consumers are done reading step ks; the producer may refill
// that slot with step ks+2).  Both roles pass the same barriers in the same
// order, tile after tile, so no wave waits on a barrier the others skip.
constexpr int PTILE = 128;
constexpr int PTHREADS = 5 * 64;
__global__ __launch_bounds__(PTHREADS) void ladder_producer_kernel(LParams p) {
  constexpr int W = PTILE / 2;
  constexpr int MI = W / 16, NI = W / 16;
  constexpr int OPB = PTILE * BK * 2;         // 16 KiB per operand tile per stage
  constexpr int STB = 2 * OPB;
  constexpr int PLOADS = OPB / (64 * 16);     // 16 loads per operand by the producer
  __shared__ __attribute__((aligned(1024))) char smem[2 * STB];
  const uint32_t lds0 = lds_addr(smem);

  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const bool producer = wave == 4;
  const int wm = (wave >> 1) & 1, wn = wave & 1;
  const int lane = threadIdx.x & 63;
  const int l16 = lane & 15, lq = lane >> 4;
  const int nk = p.K / BK;

  for (int t = xcd_slot(blockIdx.x, gridDim.x, p.num_xcds); t < p.num_tiles; t += gridDim.x) {
    int tm, tn;
    tile_of_task(t, p.tiles_m, p.tiles_n, p.tiles_m < 8 ? p.tiles_m : 8, &tm, &tn);
    const uint16_t* a0 = p.A + (int64_t)tm * PTILE * p.lda;
    const uint16_t* b0 = p.B + (int64_t)tn * PTILE * p.ldb;
    const i32x4 ra = make_rsrc((uint64_t)(uintptr_t)a0, (uint32_t)(((int64_t)(PTILE - 1) * p.lda + p.K) * 2));
    const i32x4 rb = make_rsrc((uint64_t)(uintptr_t)b0, (uint32_t)(((int64_t)(PTILE - 1) * p.ldb + p.K) * 2));
    // producer: load i of an operand covers rows 8 i .. 8 i + 7 (lane / 8)
    // and the logical chunk the swizzle puts at physical chunk lane % 8
    // operand op (0: A, 1: B) of step ks into slot
    auto load = [&](int ks, int slot, int op) {
      const int k0 = ks * BK;
#pragma unroll
      for (int i = 0; i < PLOADS; ++i) {
        const int r = i * 8 + (lane >> 3), c = (lane & 7) ^ swz_k(r);
        const uint32_t m0 = lds0 + slot * STB + op * OPB + i * 1024;
        dma16(op == 0 ? ra : rb, (uint32_t)((r * (op == 0 ? p.lda : p.ldb) + k0 + c * 8) * 2), m0);
      }
    };

    f32x4 acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NI; ++j) acc[i][j] = (f32x4){};
    fence();

    if (producer) {
      load(0, 0, 0);
      load(0, 0, 1);
    }
    for (int ks = 0; ks < nk; ++ks) {
      if (producer) {
        // step ks+1 goes into the slot step ks-1 left at the last "empty"
        // barrier: its A tile before the wait for step ks, its B tile after
        // (at most 48 loads in flight, within the wave's vmcnt range)
        if (ks + 1 < nk) {
          load(ks + 1, (ks + 1) & 1, 0);
          asm volatile("s_waitcnt vmcnt(%0)" : : "n"(PLOADS) : "memory");  // step ks landed
          load(ks + 1, (ks + 1) & 1, 1);
        } else {
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
      }
      wait_lds_barrier();  // "full": step ks is in its slot
      if (!producer) {
        const char* base = smem + (ks & 1) * STB;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int off = (((4 * s + lq) ^ swz_k(l16)) << 4);
          u32x4 a[MI], b[NI];
#pragma unroll
          for (int i = 0; i < MI; ++i) a[i] = *(const u32x4*)(base + (wm * W + i * 16 + l16) * 128 + off);
#pragma unroll
          for (int j = 0; j < NI; ++j)
            b[j] = *(const u32x4*)(base + OPB + (wn * W + j * 16 + l16) * 128 + off);
#pragma unroll
          for (int j = 0; j < NI; ++j)
#pragma unroll
            for (int i = 0; i < MI; ++i) mfma16<_Float16>(acc[i][j], b[j], a[i]);
        }
      }
      wait_lds_barrier();  // "empty": every consumer is done reading step ks
    }

    if (!producer) {
      // wait states between the last MFMAs and the reads of their results
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
      fence();
#pragma unroll
      for (int i = 0; i < MI; ++i) {
        const int row = tm * PTILE + wm * W + i * 16 + l16;
#pragma unroll
        for (int j = 0; j < NI; ++j) {
          const int col = tn * PTILE + wn * W + j * 16 + 4 * lq;
          u32x2 v;
          v[0] = pack2<_Float16>(acc[i][j][0], acc[i][j][1]);
          v[1] = pack2<_Float16>(acc[i][j][2], acc[i][j][3]);
          *(u32x2*)(p.D + (int64_t)row * p.ldd + col) = v;
        }
      }
    }
  }
}

static dense_gemm_status launch_producer(const LParams& p0, int cus, hipStream_t stream) {
  LParams p = p0;
  p.tiles_m = p.M / PTILE;
  p.tiles_n = p.N / PTILE;
  p.num_tiles = p.tiles_m * p.tiles_n;
  const int grid = p.num_tiles < cus ? p.num_tiles : cus;
  hipLaunchKernelGGL(ladder_producer_kernel, dim3((unsigned)grid), dim3(PTHREADS), 0, stream, p);
  return hipGetLastError() == hipSuccess ? DENSE_GEMM_OK : DENSE_GEMM_LAUNCH_FAILED;
}

template <int TILE, bool DMA, int STAGES, bool PERSIST, int MF = 16, int NW = 4>
static dense_gemm_status launch(const LParams& p0, int cus, hipStream_t stream) {
  LParams p = p0;
  p.tiles_m = p.M / TILE;
  p.tiles_n = p.N / TILE;
  p.num_tiles = p.tiles_m * p.tiles_n;
  const int grid = PERSIST ? (p.num_tiles < cus ? p.num_tiles : cus) : p.num_tiles;
  hipLaunchKernelGGL((ladder_kernel<TILE, DMA, STAGES, PERSIST, MF, NW>), dim3((unsigned)grid),
                     dim3(NW * 64), 0, stream, p);
  return hipGetLastError() == hipSuccess ? DENSE_GEMM_OK : DENSE_GEMM_LAUNCH_FAILED;
}

}  // namespace ladder
}  // namespace dg

using namespace dg;

extern "C" dense_gemm_status gemm_nt_f16_ladder(int level, int64_t M, int64_t N, int64_t K,
                                                const void* A, int64_t lda, const void* B,
                                                int64_t ldb, void* D, int64_t ldd,
                                                hipStream_t stream) {
  if (level < 1 || level > 9) return DENSE_GEMM_BAD_ARG;
  if (level == 6) return gemm_nt_f16(M, N, K, A, lda, B, ldb, D, ldd, stream);
  const int64_t tile = level == 5 || level >= 8 ? 256 : 128;
  if (M <= 0 || N <= 0 || K <= 0 || M % tile || N % tile || K % ladder::BK) return DENSE_GEMM_BAD_ARG;
  if (M >= ((int64_t)1 << 31) || N >= ((int64_t)1 << 31) || K >= ((int64_t)1 << 31))
    return DENSE_GEMM_BAD_ARG;
  if (!A || !B || !D) return DENSE_GEMM_NULL_PTR;
  if (lda < K || ldb < K || ldd < N) return DENSE_GEMM_BAD_LD;
  if (((uintptr_t)A | (uintptr_t)B | (uintptr_t)D) & 15 || (lda | ldb | ldd) & 7)
    return DENSE_GEMM_MISALIGNED;
  if (lda >= ((int64_t)1 << 31) || ldb >= ((int64_t)1 << 31)) return DENSE_GEMM_TOO_LARGE;
  if (((tile - 1) * lda + K) * 2 >= ((int64_t)1 << 31) || ((tile - 1) * ldb + K) * 2 >= ((int64_t)1 << 31))
    return DENSE_GEMM_TOO_LARGE;
  // 32-bit row pitch of D and tile numbers
  if (ldd >= ((int64_t)1 << 31) || (M / tile) * (N / tile) >= ((int64_t)1 << 31))
    return DENSE_GEMM_TOO_LARGE;
  int cus = 0, xcds = 1;
  const dense_gemm_status st = device_topology(&cus, &xcds);
  if (st != DENSE_GEMM_OK) return st;
  ladder::LParams p{(const uint16_t*)A, (const uint16_t*)B, (uint16_t*)D, (int)M, (int)N, (int)K,
                    (int)lda, (int)ldb, (int)ldd, 0, 0, 0, xcds};
  switch (level) {
    case 1: return ladder::launch<128, false, 1, false>(p, cus, stream);
    case 2: return ladder::launch<128, true, 1, false>(p, cus, stream);
    case 3: return ladder::launch<128, true, 2, false>(p, cus, stream);
    case 4: return ladder::launch<128, true, 2, true>(p, cus, stream);
    case 7: return ladder::launch_producer(p, cus, stream);
    case 8: return ladder::launch<256, true, 2, true, 32>(p, cus, stream);
    case 9: return ladder::launch<256, true, 2, true, 16, 8>(p, cus, stream);
    default: return ladder::launch<256, true, 2, true>(p, cus, stream);
  }
}
