// plan.h -- host-side planning of the FP16/BF16 GEMM calls (plain C++, no
// device code): the argument check, the launch plan with the caller's
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
  // the small-output kernel (one workgroup per 16 x 16 tile) instead of the
  // tiled kernel
  bool small() const { return plan[0] == SMALL_TILE; }
};

// A @ B.T outputs the small-output kernel computes when no option asks for
// the tiled kernel: M and N at most SMALL_MAX, K at most SMALL_K_MAX.
bool small_output(int layout, int64_t M, int64_t N, int64_t K);
// The tiled kernel's plan (dense_gemm_plan for the other products).
dense_gemm_status tiled_plan(int layout, int64_t M, int64_t N, int64_t K, int64_t num_cus,
                             int64_t* out);

bool valid_op(int op);
int op_layout(int op);

// The plan of one call on a device with `cus` CUs: dense_gemm_plan, the
// caller's options (may be null), and the workspace the call needs.
// Arguments must have passed dense_gemm_validate, with M, N > 0.
dense_gemm_status plan_call(int layout, int64_t M, int64_t N, int64_t K, const void* A,
                            int64_t lda, const void* B, int64_t ldb, int64_t cus,
                            const dense_gemm_options* opt, CallPlan* cp);

}  // namespace dg
