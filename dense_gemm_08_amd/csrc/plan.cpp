// plan.cpp -- host-side planning of the GEMM calls: the FP16/BF16 argument
// check, the persistent tile scheduler's helpers, the launch plans (kernel,
// tile shape, split-K) of the FP16/BF16 and FP8 products and the workspace
// a call needs.  Plain C++ with no device
// code, so it also builds with the host sanitizers (tests/host_fuzz.cpp).
#include "plan.h"

#include <stdint.h>

#include "tile_sched.h"

namespace dg {

// Tile rows per group of the grouped order.  The workgroups resident on one
// XCD take consecutive tasks, i.e. a block of group_m tile rows by a few
// tile columns that shares its A and B panels in that XCD's L2; 8 rows made
// that block closest to square for the grids measured (32 workgroups per
// XCD at 4096^3: an 8 x 4 block of 12 panels).
int choose_group_m(int64_t tiles_m) { return (int)(tiles_m < 8 ? tiles_m : 8); }

}  // namespace dg

using namespace dg;

extern "C" {

const char* dense_gemm_status_string(int status) {
  switch (status) {
    case DENSE_GEMM_OK: return "ok";
    case DENSE_GEMM_INVALID_DIM: return "invalid dimension (negative M, N or K)";
    case DENSE_GEMM_NULL_PTR: return "null pointer";
    case DENSE_GEMM_BAD_LD: return "leading dimension below its minimum";
    case DENSE_GEMM_MISALIGNED: return "operand pointer not aligned to its 2-byte elements";
    case DENSE_GEMM_TOO_LARGE: return "problem too large for 32-bit tile offsets";
    case DENSE_GEMM_LAUNCH_FAILED: return "kernel launch failed";
    case DENSE_GEMM_NO_DEVICE: return "no gfx950 device current";
    case DENSE_GEMM_BAD_ARG: return "bad argument";
    case DENSE_GEMM_NO_MEMORY: return "no device memory for the workspace";
    case DENSE_GEMM_WORKSPACE_TOO_SMALL:
      return "workspace smaller than the call needs (see the workspace size query)";
    case DENSE_GEMM_SCRATCH_TOO_SMALL:
      return "the call needs more scratch memory than the 64 MiB the no-allocation entry "
             "point holds per device (use dense_gemm_ex with a larger workspace)";
    default: return "unknown status";
  }
}

dense_gemm_status dense_gemm_validate(int layout, int64_t M, int64_t N, int64_t K, const void* A,
                                      int64_t lda, const void* B, int64_t ldb, const void* D,
                                      int64_t ldd) {
  if (layout != NT && layout != NN) return DENSE_GEMM_BAD_ARG;
  if (M < 0 || N < 0 || K < 0) return DENSE_GEMM_INVALID_DIM;
  if (M == 0 || N == 0) return DENSE_GEMM_OK;
  if (M >= kMaxDim || N >= kMaxDim || K >= kMaxDim) return DENSE_GEMM_TOO_LARGE;
  // task numbers are 32-bit: the tile count at the narrower tile width
  if (((M + BM - 1) / BM) * ((N + BN / 2 - 1) / (BN / 2)) >= kMaxDim) return DENSE_GEMM_TOO_LARGE;
  if (D == nullptr) return DENSE_GEMM_NULL_PTR;
  if (K > 0 && (A == nullptr || B == nullptr)) return DENSE_GEMM_NULL_PTR;
  if (ldd < N) return DENSE_GEMM_BAD_LD;
  if (K > 0) {
    if (lda < K) return DENSE_GEMM_BAD_LD;
    if (layout == NT ? ldb < K : ldb < N) return DENSE_GEMM_BAD_LD;
  }
  if (((uintptr_t)D & 1) != 0) return DENSE_GEMM_MISALIGNED;
  if (K > 0) {
    if (((uintptr_t)A & 1) != 0 || ((uintptr_t)B & 1) != 0) return DENSE_GEMM_MISALIGNED;
    // (leading dimensions first: the spans below must not overflow)
    if (lda >= kMaxDim || ldb >= kMaxDim) return DENSE_GEMM_TOO_LARGE;
    // 32-bit buffer offsets: the span one tile's descriptor covers, for the
    // operand as given or as its repacked copy (leading dimension K8 or N8)
    const int64_t K8 = (K + 7) & ~(int64_t)7, N8 = (N + 7) & ~(int64_t)7;
    const int64_t lda_k = lda > K8 ? lda : K8;
    const int64_t ldb_k = ldb > (layout == NT ? K8 : N8) ? ldb : (layout == NT ? K8 : N8);
    const int64_t lim = ((int64_t)1 << 31) - 16;
    if (((int64_t)(BM - 1) * lda_k + K8) * 2 >= lim) return DENSE_GEMM_TOO_LARGE;
    if (layout == NT && ((int64_t)(BN - 1) * ldb_k + K8) * 2 >= lim) return DENSE_GEMM_TOO_LARGE;
    if (layout == NN && ((int64_t)(BK - 1) * ldb_k + N8) * 2 >= lim) return DENSE_GEMM_TOO_LARGE;
  }
  if (ldd >= kMaxDim || lda >= kMaxDim || ldb >= kMaxDim) return DENSE_GEMM_TOO_LARGE;
  return DENSE_GEMM_OK;
}

dense_gemm_status dense_gemm_tile_of_task(int64_t task, int64_t tiles_m, int64_t tiles_n,
                                          int64_t group_m, int64_t* tile_m, int64_t* tile_n) {
  if (tiles_m <= 0 || tiles_n <= 0 || group_m <= 0 || task < 0 || task >= tiles_m * tiles_n ||
      tiles_m * tiles_n >= kMaxDim || !tile_m || !tile_n)
    return DENSE_GEMM_BAD_ARG;
  int tm, tn;
  tile_of_task((int)task, (int)tiles_m, (int)tiles_n, (int)group_m, &tm, &tn);
  *tile_m = tm;
  *tile_n = tn;
  return DENSE_GEMM_OK;
}

int64_t dense_gemm_xcd_slot(int64_t b, int64_t grid, int64_t num_xcds) {
  if (grid <= 0 || num_xcds <= 0 || b < 0 || b >= grid || grid >= kMaxDim) return -1;
  return xcd_slot((int)b, (int)grid, (int)num_xcds);
}

dense_gemm_status dense_gemm_plan(int layout, int64_t M, int64_t N, int64_t K, int64_t num_cus,
                                  int64_t* out) {
  if ((layout != NT && layout != NN) || M <= 0 || N <= 0 || K < 0 || num_cus <= 0 || !out)
    return DENSE_GEMM_BAD_ARG;
  if (small_output(layout, M, N, K)) {
    // the small-output kernel: one workgroup per tile, K split among its
    // eight waves (no workspace); A @ B in 16 x 16 tiles
    out[0] = out[1] = SMALL_TILE;
    if (layout == NT) small_tile(M, N, num_cus, &out[0], &out[1]);
    out[2] = BK;
    out[3] = (M + out[0] - 1) / out[0];
    out[4] = (N + out[1] - 1) / out[1];
    out[5] = out[3] * out[4];
    out[6] = 1;
    out[7] = SMALL_THREADS;
    out[8] = 1;
    out[9] = (K + BK - 1) / BK;
    return DENSE_GEMM_OK;
  }
  return tiled_plan(layout, M, N, K, num_cus, out);
}

}  // extern "C"

namespace dg {

// Measured on the MI355X against the tiled kernel's best plan (split-K
// where it pays), per call: 128 x 128 x 64 4.0 against 5.2 us, 128 x 128 x
// 4096 4.4 against 10.9, 128 x 128 x 16384 11.6 against 14.9 (but with K =
// 65536 the tiled kernel's 16-way split is faster), 128 x 1024 x 1024 4.1
// against 13.3.  With one tile row (M <= 16) every B row is streamed once,
// whatever N: 1 x 4096 x 4096 6.6 against 11.4, 16 x 16384 x 4096 22.7
// against 28.6, 16 x 32768 x 4096 43.1 against 47.4.  With more tile rows
// and more tiles (each operand row streamed by many workgroups: 64 x 4096
// x 4096 19.0 against 14.9) the tiled kernel is faster.
//
// A @ B: a 16 x 16 tile reads B in 32-byte row segments, four tiles to a
// 128-byte line (the lines are fetched once: the tiles that share them run
// on one XCD), which takes four times the L2 requests of A @ B.T (measured at
// 1 x 8192 x 8192: 4.3 against 1.1 million): a CU streams its tiles at
// about 40 GB/s, against about 90 for A @ B.T.  So A @ B runs the
// small-output kernel only where K is at most SMALL_NN_K_MAX = 4096 and the
// B elements its tiles stream, tile rows x N x K, are at most SMALL_NN_ELEMS
// = 21 * 2^20.  Measured against the tiled kernel with its workspace passed
// (with the workspace allocated per call, the tiled kernel's split costs
// about 4 us more): 1 x 4096 x 4096 8.6 against 10.9 us, 16 x 4096 x 4096
// 10.5 against 12.0, 32 x 1024 x 4096 5.7 against 10.4, 100 x 1000 x 3000
// 13.6 against 14.4, 128 x 128 x 4096 5.3 against 10.9; beyond the limits
// 1 x 6144 x 4096 18.3 against 14.7 (384 tiles: more than one per CU),
// 1 x 8192 x 4096 17.3 against 16.4, 64 x 2048 x 4096 19.5 against 14.4,
// 1 x 8192 x 8192 31.4 against 25.4, 128 x 1024 x 8192 35.8 against 19.6,
// 1 x 2048 x 16384 30.3 against 17.6.
//
// A @ B.T also takes products of more tiles where tiles of 32 x 32 times K
// are at most SMALL_T32_K = 2^21: its 32-row tiles (small_tile) and
// XCD-grouped tile order cut each tile row's pass over B to about half and
// serve it from L2.  Measured per call on one box against the tiled kernel
// (128-row tiles, split-K, workspace passed): 32 x 8192 x 8192 21.2
// against 25.4 us, 64 x 4096 x 4096 8.9 against 13.6, 128 x 2048 x 8192
// 13.8 against 16.2, 48 x 8192 x 4096 16.5 against 17.6, 128 x 4096 x 4096
// 15.5 against 16.4 (all at 2^20 or 2^21); past the limit 96 x 4096 x 8192
// 25.5 against 19.3 (3 2^20), 64 x 8192 x 8192 28.2 against 26.9 (2^22),
// 128 x 8192 x 8192 49.9 against 29.6 (2^23).
bool small_output(int layout, int64_t M, int64_t N, int64_t K) {
  if ((layout != NT && layout != NN) || M > SMALL_MAX || K > SMALL_K_MAX) return false;
  const int64_t tiles_m = (M + SMALL_TILE - 1) / SMALL_TILE;
  const int64_t tiles = tiles_m * ((N + SMALL_TILE - 1) / SMALL_TILE);
  if (layout == NT) {
    const int64_t t32 = ((M + 31) / 32) * ((N + 31) / 32);
    return M <= SMALL_TILE || tiles <= SMALL_MAX_TILES || t32 * K <= SMALL_T32_K;
  }
  if (tiles > SMALL_MAX_TILES && M > SMALL_TILE) return false;
  return K <= SMALL_NN_K_MAX && tiles_m * N * K <= SMALL_NN_ELEMS;
}

// The largest tile whose grid still covers the CUs: more columns per tile
// read each chunk of A once for more blocks, more rows each chunk of B, but
// fewer tiles leave CUs idle.  Measured on one box, FP8: 64 x 1024 x 4096
// 4.3 us in 16 x 16 tiles (256 of them) against 5.1 in 32 x 16 and 6.0 in
// 32 x 32; 128 x 1024 x 4096 5.2 us in 32 x 16 (256 tiles) against 6.2 in
// the others; FP16 A @ B.T alike (64 x 1024 x 4096 4.9 in 16 x 16 against
// 5.7 and 6.8; 128 x 1024 x 4096 6.4 in 32 x 16 against 7.6 and 6.9).  One
// 16-row tile row keeps 16 x 16 tiles: there a taller tile only computes
// padding (FP8 16 x 8192 x 8192 13.5 us against 16.0 in 32 x 16).
void small_tile(int64_t M, int64_t N, int64_t num_cus, int64_t* rows, int64_t* cols) {
  *rows = *cols = SMALL_TILE;
  if (M <= SMALL_TILE) return;
  const int64_t tm = (M + 31) / 32;
  if (tm * ((N + 31) / 32) >= num_cus) {
    *rows = *cols = 32;
  } else if (tm * ((N + 15) / 16) >= num_cus) {
    *rows = 32;
  }
}

// Split-K for the tiles of the last, partial wave (all tiles when there
// are fewer than CUs), at most one part per idle CU and at least 4 K steps
// per part.
//   * Fewer tiles than CUs: the split (if any) with the least estimated
//     time, from a model fitted to measured times on the MI355X (in units
//     of 0.01 us): step_cost per K step of a tile, fixed_cost for a split
//     call's extra work (the reduce launch, the workspace), and part_cost
//     per partial tile for its FP32 write and read back, scaled by
//     blocks16 / 16, the share of the tile's 16 16-row blocks inside D.
//   * After full waves: split when the last wave would leave at least
//     three quarters of the CUs idle (measured: splitting a half-full last
//     wave gains nothing), into as many parts as fit.
void choose_split(int64_t tasks, int64_t nk, int64_t num_cus, int64_t step_cost,
                  int64_t fixed_cost, int64_t part_cost, int64_t blocks16, int64_t* splits_out,
                  int64_t* steps_out) {
  const int64_t rem = tasks % num_cus;
  int64_t splits = 1, steps = nk;
  if (rem > 0 && nk >= 8) {
    const int64_t by_cus = num_cus / rem, by_k = nk / 4;
    const int64_t most = by_cus < by_k ? by_cus : by_k;
    if (tasks < num_cus) {
      // (in 1/16 of the units above)
      int64_t best = nk * 16 * step_cost;
      for (int64_t sp = 2; sp <= most; ++sp) {
        const int64_t st = (nk + sp - 1) / sp, parts = (nk + st - 1) / st;
        const int64_t t = st * 16 * step_cost + 16 * fixed_cost + part_cost * blocks16 * parts * rem;
        if (t < best) {
          best = t;
          steps = st;
          splits = parts;
        }
      }
    } else if (rem * 4 <= num_cus && most >= 2) {
      steps = (nk + most - 1) / most;
      splits = (nk + steps - 1) / steps;
    }
  }
  *splits_out = splits;
  *steps_out = steps;
}

dense_gemm_status tiled_plan(int layout, int64_t M, int64_t N, int64_t K, int64_t num_cus,
                             int64_t* out) {
  // Tile rows: 256, or 128 when M <= 128 (one tile row either way, half the
  // MFMA work of a 256-row tile that would be half padding).
  const int64_t tr = M <= BM / 2 ? BM / 2 : BM;
  const int64_t tiles_m = (M + tr - 1) / tr;
  // Tile width: 256, or for A @ B.T 128
  //   * when the output is at most 128 wide: the same single tile column,
  //     with half the MFMA work and B traffic of a 256-wide tile that would
  //     be half padding (measured: 128 x 128 x 64 7.5 -> 5.2 us, 128 x 128 x
  //     4096 in 16 parts 13.4 -> 11.3 us);
  //   * when 256-wide tiles would occupy at most half the CUs (one wave) and
  //     the output is wider than 128: twice the tiles, still one wave.
  //     Narrow tiles then read A twice as often, so they are kept for
  //     operands that stay in the 256 MB Infinity Cache (at most 192 MiB);
  //     beyond it (measured: 8192 x 1024 x 16384) 256-wide tiles with split-K
  //     are faster.
  const int64_t t256 = tiles_m * ((N + BN - 1) / BN);
  const bool cached = K == 0 || (M + N) <= ((int64_t)96 << 20) / K;  // (M + N) K 2 B <= 192 MiB
  const bool narrow = N <= BN / 2 || (2 * t256 <= num_cus && cached);
  const int64_t tw = layout == NT && narrow ? BN / 2 : BN;
  const int64_t tiles_n = (N + tw - 1) / tw;
  const int64_t tasks = tiles_m * tiles_n;
  const int64_t grid = tasks < num_cus ? tasks : num_cus;
  out[0] = tr;
  out[1] = tw;
  out[2] = BK;
  out[3] = tiles_m;
  out[4] = tiles_n;
  out[5] = grid;
  out[6] = choose_group_m(tiles_m);
  out[7] = THREADS;
  // Split-K: the model of choose_split with the FP16 kernel's costs (a K
  // step of a 256-wide tile 105, of a 128-wide one 70; a split call 1200; a
  // partial tile 12 or 6); a partial tile writes and the reduction reads
  // only its 16-row blocks inside D, so with one tile row that cost shrinks
  // to their share.
  const int64_t nk = (K + BK - 1) / BK;
  const int64_t blocks16 = tiles_m == 1 ? (M + 15) / 16 : BM / 16;
  int64_t splits = 1, steps = nk;
  choose_split(tasks, nk, num_cus, tw == BN ? 105 : 70, 1200, tw == BN ? 12 : 6, blocks16, &splits,
               &steps);
  out[8] = splits;
  out[9] = steps;
  if (splits > 1 && tasks < num_cus) out[5] = tasks * splits;
  return DENSE_GEMM_OK;
}

bool valid_op(int op) { return op >= DENSE_GEMM_NT_F16 && op <= DENSE_GEMM_NN_F16; }
int op_layout(int op) { return op == DENSE_GEMM_NN_BF16 || op == DENSE_GEMM_NN_F16 ? NN : NT; }

dense_gemm_status plan_call(int layout, int64_t M, int64_t N, int64_t K, const void* A,
                            int64_t lda, const void* B, int64_t ldb, int64_t cus,
                            const dense_gemm_options* opt, CallPlan* cp) {
  int64_t* plan = cp->plan;
  dense_gemm_status st = dense_gemm_plan(layout, M, N, K, cus, plan);
  if (st != DENSE_GEMM_OK) return st;
  // Any option asks for the tiled kernel, with that option applied to its
  // plan; without one, a small output runs the small-output kernel (one
  // workgroup per 16 x 16 tile, no split).
  const bool options = opt != nullptr && (opt->split_k != 0 || opt->tile_n != 0);
  if (options && cp->small()) {
    st = tiled_plan(layout, M, N, K, cus, plan);
    if (st != DENSE_GEMM_OK) return st;
  }
  const int64_t nk = (K + BK - 1) / BK;
  bool forced_split = false;
  if (cp->small()) {
    cp->full_tasks = plan[5];
    cp->split_tiles = 0;
  } else if (opt != nullptr) {
    if (opt->tile_n != 0) {
      const int64_t want = opt->tile_n;
      if (want != BN && !(want == BN / 2 && layout == NT)) return DENSE_GEMM_BAD_ARG;
      if (want != plan[1]) {
        plan[1] = want;
        plan[4] = (N + want - 1) / want;
        plan[5] = plan[3] * plan[4] < cus ? plan[3] * plan[4] : cus;
        plan[6] = choose_group_m(plan[3]);
        plan[8] = 1;  // the split is then forced below, or none
        plan[9] = nk;
      }
    }
    if (opt->split_k < 0) return DENSE_GEMM_BAD_ARG;
    if (opt->split_k > 0 && nk >= 1) {
      // n parts on every tile (at most one per K step): the K steps per part
      // and the number of non-empty parts that gives
      const int64_t want = opt->split_k < nk ? opt->split_k : nk;
      plan[9] = (nk + want - 1) / want;
      plan[8] = (nk + plan[9] - 1) / plan[9];
      forced_split = true;
    }
  }
  const int64_t tasks = plan[3] * plan[4];
  if (cp->small()) {
    // (one workgroup per tile, set above)
  } else if (plan[8] > 1) {
    cp->full_tasks = forced_split ? 0 : tasks - tasks % cus;
    cp->split_tiles = tasks - cp->full_tasks;
    plan[5] = cp->full_tasks + cp->split_tiles * plan[8];
    if (plan[5] > cus) plan[5] = cus;
  } else {
    plan[8] = 1;
    plan[9] = nk;
    cp->full_tasks = tasks;
    cp->split_tiles = 0;
    plan[5] = tasks < cus ? tasks : cus;
  }
  // Operands the 16-byte chunk loader cannot read in place (a pointer not
  // 16-byte aligned, a leading dimension or K -- or N for the A.B layout's
  // B -- not a multiple of 8) are first copied into a dense, zero-padded
  // layout (`repack`) in the workspace.
  const int64_t K8 = (K + 7) & ~(int64_t)7, N8 = (N + 7) & ~(int64_t)7;
  cp->a_direct = K == 0 || (((uintptr_t)A & 15) == 0 && (lda & 7) == 0 && (K & 7) == 0);
  cp->b_direct = K == 0 || (((uintptr_t)B & 15) == 0 && (ldb & 7) == 0 &&
                            (layout == NT ? (K & 7) == 0 : (N & 7) == 0));
  const int64_t b_rows = layout == NT ? N : K, b_dcols = layout == NT ? K8 : N8;
  // sizes in bytes, checked for overflow (a forced split of a huge product
  // could exceed 2^64 bytes): such a plan is TOO_LARGE
  const size_t cap = (size_t)1 << 62;
  auto bytes_of = [&](size_t a, size_t b, size_t c, size_t* out) {
    size_t ab, abc;
    if (__builtin_mul_overflow(a, b, &ab) || __builtin_mul_overflow(ab, c, &abc) || abc > cap)
      return false;
    *out = (abc + 255) & ~(size_t)255;
    return true;
  };
  cp->a_bytes = cp->b_bytes = cp->split_bytes = 0;
  if (!cp->a_direct && !bytes_of((size_t)M, (size_t)K8, 2, &cp->a_bytes)) return DENSE_GEMM_TOO_LARGE;
  if (!cp->b_direct && !bytes_of((size_t)b_rows, (size_t)b_dcols, 2, &cp->b_bytes))
    return DENSE_GEMM_TOO_LARGE;
  if (plan[8] > 1 && !bytes_of((size_t)plan[8] * (size_t)cp->split_tiles, (size_t)plan[0] * plan[1],
                               sizeof(float), &cp->split_bytes))
    return DENSE_GEMM_TOO_LARGE;
  if (cp->a_bytes + cp->b_bytes + cp->split_bytes > cap) return DENSE_GEMM_TOO_LARGE;
  return DENSE_GEMM_OK;
}

// Products the FP8 small-output kernel computes (gemm_mx_small): M <= 128,
// K <= MX_SMALL_K_MAX = 8192 (its scales are staged in LDS), and one 16-row
// tile row, or at most MX_SMALL_T32 = 1024 tiles of 32 x 32 in D, or at most
// MX_SMALL_T32_MAX = 1536 of them with tiles x K at most MX_SMALL_T32_K =
// 2^23.  The tiled FP8 kernel has no 128-row tile and, at these M, splits K
// into FP32 partial tiles; the small kernel's cost is each tile row's pass
// over B, which its 32-row tiles halve and its XCD-grouped tile order
// serves from L2.  Measured per call on one box over the 23 products of M
// = 24 ... 128, N = 2048 ... 16384 and K = 2048 ... 8192 that the former
// rule (at most 2048 tiles of 16 x 16 with tiles x K <= 2^23) left to the
// tiled kernel, the small kernel (its tile as small_tile picks) against
// the tiled one through the plain entry point (which allocates the split's
// workspace per call; with a preallocated workspace, about 3 us less): up
// to 1024 tiles of 32 x 32 1.17-2.31x as fast (e.g. 64 x 8192 x 8192 17.3
// against 32.2 us, 128 x 8192 x 8192 30.9 against 36.0);
// at 1536 tiles (96 x 16384) 1.26x and 1.10x at K = 2048 and 4096, 0.99x at
// 8192 (tiles x K 3 2^20, 3 2^21 and 3 2^22); at 2048 tiles (128 x 16384)
// 0.98x and 0.88x at K = 2048 and 4096.  Products inside the former rule
// run the small kernel as before, its new tiles no slower (one tile row:
// 16 x 16 as before; more rows: measured 1.0-1.9x as fast).
bool mx_small_output(int64_t M, int64_t N, int64_t K) {
  if (M > SMALL_MAX || K > mx::MX_SMALL_K_MAX) return false;
  if (M <= SMALL_TILE) return true;
  const int64_t t32 = ((M + 31) / 32) * ((N + 31) / 32);
  return t32 <= mx::MX_SMALL_T32 || (t32 <= mx::MX_SMALL_T32_MAX && t32 * K <= mx::MX_SMALL_T32_K);
}

dense_gemm_status mx_plan_call(int64_t M, int64_t N, int64_t K, int64_t num_cus, MxPlan* mp) {
  if (M <= 0 || N <= 0 || K < 0 || K % mx::GROUP != 0 || num_cus <= 0 || mp == nullptr ||
      M >= kMaxDim || N >= kMaxDim || K >= kMaxDim)
    return DENSE_GEMM_BAD_ARG;
  int64_t* out = mp->plan;
  const int64_t nks = (K + mx::BKE - 1) / mx::BKE;
  mp->panel_bytes[0] = mp->panel_bytes[1] = mp->split_bytes = 0;
  if (mx_small_output(M, N, K)) {
    // one workgroup per tile, the scales staged in LDS: no workspace
    small_tile(M, N, num_cus, &out[0], &out[1]);
    out[2] = mx::BKE;
    out[3] = (M + out[0] - 1) / out[0];
    out[4] = (N + out[1] - 1) / out[1];
    out[5] = out[3] * out[4];
    out[6] = 1;
    out[7] = SMALL_THREADS;
    out[8] = 1;
    out[9] = nks;
    mp->full_tasks = out[5];
    mp->split_tiles = 0;
    return DENSE_GEMM_OK;
  }
  const int64_t tiles_m = (M + mx::BM - 1) / mx::BM, tiles_n = (N + mx::BN - 1) / mx::BN;
  const int64_t tasks = tiles_m * tiles_n;
  if (tasks >= kMaxDim) return DENSE_GEMM_TOO_LARGE;
  // Split-K: the model of choose_split with the FP8 kernel's costs (a
  // 128-deep K stage of a tile 100, a split call 1000, a partial tile 5),
  // fitted to the workspace-passing call's times on the MI355X over 18
  // products of fewer tiles than CUs (256 x 256 x 16384 to 8192 x 1024 x
  // 16384), each at 6-9 part counts: the model's pick was the fastest
  // measured on 13 of them and within 10% on all (1% on the geometric
  // mean), 1.55 times as fast as the unsplit call on the geometric mean;
  // the FP16 kernel's split and partial-tile costs (1200, 12) picked up to
  // 14% slower.  (The partial tiles of these products, at most 64 MiB, stay
  // in the 256 MB Infinity Cache between their write and the reduction's
  // read.)
  const int64_t blocks16 = tiles_m == 1 ? (M + 15) / 16 : mx::BM / 16;
  int64_t splits = 1, steps = nks;
  choose_split(tasks, nks, num_cus, MX_STEP_COST, MX_SPLIT_COST, MX_PART_COST, blocks16, &splits,
               &steps);
  out[0] = mx::BM;
  out[1] = mx::BN;
  out[2] = mx::BKE;
  out[3] = tiles_m;
  out[4] = tiles_n;
  out[6] = choose_group_m(tiles_m);
  out[7] = THREADS;
  out[8] = splits;
  out[9] = steps;
  mp->full_tasks = splits > 1 ? tasks - tasks % num_cus : tasks;
  mp->split_tiles = tasks - mp->full_tasks;
  const int64_t all = mp->full_tasks + mp->split_tiles * splits;
  out[5] = all < num_cus ? all : num_cus;
  // packed scale panels (at least one stage), then the FP32 partial tiles
  const size_t stages = (size_t)(nks > 0 ? nks : 1);
  mp->panel_bytes[0] = (size_t)tiles_m * stages * mx::SC_BYTES;
  mp->panel_bytes[1] = (size_t)tiles_n * stages * mx::SC_BYTES;
  if (splits > 1) {
    size_t n;
    if (__builtin_mul_overflow((size_t)splits * (size_t)mp->split_tiles,
                               (size_t)mx::BM * mx::BN * sizeof(float), &n) ||
        n > ((size_t)1 << 62))
      return DENSE_GEMM_TOO_LARGE;
    mp->split_bytes = n;
  }
  return DENSE_GEMM_OK;
}

}  // namespace dg

extern "C" dense_gemm_status gemm_nt_e4m3_mx_plan(int64_t M, int64_t N, int64_t K,
                                                  int64_t num_cus, int64_t* out) {
  if (out == nullptr) return DENSE_GEMM_BAD_ARG;
  dg::MxPlan mp;
  const dense_gemm_status st = dg::mx_plan_call(M, N, K, num_cus, &mp);
  if (st == DENSE_GEMM_OK)
    for (int i = 0; i < 10; ++i) out[i] = mp.plan[i];
  return st;
}
