// plan.h -- host-side planning of the GEMM calls (plain C++, no device
// code): the FP16/BF16 argument check, the launch plans with the caller's
// options, and the workspace a call needs.  Implemented in plan.cpp.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "dense_gemm.h"
#include "tile_config.h"

namespace dg {

constexpr int64_t kMaxDim = (int64_t)1 << 31;

// Tile rows per group of the grouped order (see plan.cpp).
int choose_group_m(int64_t tiles_m);

// Everything one call launches, decided on the host before any launch.
struct CallPlan {
  int64_t plan[10];          // as dense_gemm_plan, after the caller's options
  int64_t full_tasks;        // tiles computed whole
  int64_t split_tiles;       // tiles computed in K parts
  bool a_direct, b_direct;   // operands read in place (else repacked)
  size_t a_bytes, b_bytes;   // workspace of the repacked copies
  size_t split_bytes;        // workspace of the FP32 partial tiles
  size_t total() const { return a_bytes + b_bytes + split_bytes; }
  // the small-output kernel (one 512-thread workgroup per tile) instead of
  // the tiled kernel
  bool small() const { return plan[7] == SMALL_THREADS; }
};

// Products the small-output kernel computes when no option asks for the
// tiled kernel: M at most SMALL_MAX, K at most SMALL_K_MAX, and one tile
// row or at most SMALL_MAX_TILES 16 x 16 tiles, or for A @ B.T tiles of
// 32 x 32 x K at most SMALL_T32_K; for A @ B also K at most SMALL_NN_K_MAX
// and tile rows x N x K at most SMALL_NN_ELEMS.
bool small_output(int layout, int64_t M, int64_t N, int64_t K);
// The small-output kernel's tile rows and columns for a product with M
// rows and N columns on a device with num_cus CUs: 16 x 16 where M <= 16,
// else 32 x 32 where those tiles number at least num_cus, else 32 x 16
// where those do, else 16 x 16.  (A @ B takes 16 x 16 tiles.)
void small_tile(int64_t M, int64_t N, int64_t num_cus, int64_t* rows, int64_t* cols);
// The tiled kernel's plan (dense_gemm_plan for the other products).
dense_gemm_status tiled_plan(int layout, int64_t M, int64_t N, int64_t K, int64_t num_cus,
                             int64_t* out);

// Split-K of the last, partial wave of `tasks` tiles over nk K steps on
// num_cus CUs (the cost model in plan.cpp): parts and K steps per part.
void choose_split(int64_t tasks, int64_t nk, int64_t num_cus, int64_t step_cost,
                  int64_t fixed_cost, int64_t part_cost, int64_t blocks16, int64_t* splits,
                  int64_t* steps);

bool valid_op(int op);
int op_layout(int op);

// The plan of one call on a device with `cus` CUs: dense_gemm_plan, the
// caller's options (may be null), and the workspace the call needs.
// Arguments must have passed dense_gemm_validate, with M, N > 0.
dense_gemm_status plan_call(int layout, int64_t M, int64_t N, int64_t K, const void* A,
                            int64_t lda, const void* B, int64_t ldb, int64_t cus,
                            const dense_gemm_options* opt, CallPlan* cp);

// ---- the FP8 block-scaled product ----

// The FP8 costs of the split model (0.01 us): one 128-deep K stage of a
// 256 x 256 tile, a split call's extra work, one partial tile.
constexpr int64_t MX_STEP_COST = 100;
constexpr int64_t MX_SPLIT_COST = 1000;
constexpr int64_t MX_PART_COST = 5;

// Everything an FP8 call launches.  plan: as gemm_nt_e4m3_mx_plan (tiles of
// 16 x 16, 32 x 16 or 32 x 32 for the small-output kernel, else 256 x 256
// tiles with `splits` parts of `steps` stages on the split tiles).  The
// workspace holds A's and B's packed scale panels, then the FP32 partial
// tiles.
struct MxPlan {
  int64_t plan[10];
  int64_t full_tasks, split_tiles;
  size_t panel_bytes[2];  // A's, B's (multiples of 1 KiB)
  size_t split_bytes;
  size_t total() const { return panel_bytes[0] + panel_bytes[1] + split_bytes; }
  bool small() const { return plan[7] == SMALL_THREADS; }
};

// The FP8 small-output kernel's products (M <= 128, K <= MX_SMALL_K_MAX,
// and one 16-row tile row, or at most MX_SMALL_T32 tiles of 32 x 32, or at
// most MX_SMALL_T32_MAX of them with tiles x K at most MX_SMALL_T32_K).
bool mx_small_output(int64_t M, int64_t N, int64_t K);
// (Its tile: small_tile, as for FP16 A @ B.T.)
// The plan of an FP8 call with M, N > 0 and K a multiple of 32 on a device
// with num_cus CUs.
dense_gemm_status mx_plan_call(int64_t M, int64_t N, int64_t K, int64_t num_cus, MxPlan* mp);

}  // namespace dg
