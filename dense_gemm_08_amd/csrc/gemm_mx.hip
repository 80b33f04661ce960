// gemm_mx.hip -- host side of the FP8 block-scaled GEMM for the MI355X
// (gfx950): argument checks, the launches and the C ABI.  The operation and
// the kernel design are described in gemm_mx_kernel.h, the plan (kernel,
// split-K, workspace) is made in plan.cpp.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dense_gemm.h"
#include "gemm_mx_kernel.h"
#include "gemm_mx_small_kernel.h"
#include "plan.h"
#include "split_reduce.h"

namespace dg {

// current device's CU and XCD counts, checked to be a gfx950 (dense_gemm.hip)
dense_gemm_status device_topology(int* cus, int* xcds);

namespace mx {

// The argument check of the FP8 entry points (no device call).
static dense_gemm_status validate(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                                  const void* SA, int64_t ldsa, const void* B, int64_t ldb,
                                  const void* SB, int64_t ldsb, const void* D, int64_t ldd) {
  if (M < 0 || N < 0 || K < 0) return DENSE_GEMM_INVALID_DIM;
  if (M == 0 || N == 0) return DENSE_GEMM_OK;
  const int64_t lim = (int64_t)1 << 31;
  if (M >= lim || N >= lim || K >= lim) return DENSE_GEMM_TOO_LARGE;
  // task numbers are 32-bit
  if (((M + BM - 1) / BM) * ((N + BN - 1) / BN) >= lim) return DENSE_GEMM_TOO_LARGE;
  if (K % GROUP != 0) return DENSE_GEMM_BAD_ARG;
  const int64_t nb = K / GROUP;
  if (D == nullptr) return DENSE_GEMM_NULL_PTR;
  if (K > 0 && (!A || !B || !SA || !SB)) return DENSE_GEMM_NULL_PTR;
  if (ldd < N) return DENSE_GEMM_BAD_LD;
  if (K > 0 && (lda < K || ldb < K || ldsa < nb || ldsb < nb)) return DENSE_GEMM_BAD_LD;
  if (((uintptr_t)D & 1) != 0) return DENSE_GEMM_MISALIGNED;
  if (K > 0 && ((((uintptr_t)A | (uintptr_t)B) & 15) != 0 || ((lda | ldb) & 15) != 0))
    return DENSE_GEMM_MISALIGNED;
  if (K > 0 && (lda >= lim || ldb >= lim)) return DENSE_GEMM_TOO_LARGE;  // before the spans
  if (K > 0 && ((BM - 1) * lda + K >= lim - 16 || (BN - 1) * ldb + K >= lim - 16))
    return DENSE_GEMM_TOO_LARGE;
  if (ldd >= lim || lda >= lim || ldb >= lim || ldsa >= lim || ldsb >= lim) return DENSE_GEMM_TOO_LARGE;
  return DENSE_GEMM_OK;
}

// The launches of a validated call with M, N > 0 into a workspace of at
// least mp.total() bytes (256-byte aligned; null when that is 0).
static dense_gemm_status enqueue(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                                 const void* SA, int64_t ldsa, const void* B, int64_t ldb,
                                 const void* SB, int64_t ldsb, void* D, int64_t ldd,
                                 const MxPlan& mp, uint8_t* ws, int cus, int xcds,
                                 hipStream_t stream) {
  const int64_t* plan = mp.plan;
  if (mp.small()) {
    MxSmallParams q;
    q.A = (const uint8_t*)A;
    q.B = (const uint8_t*)B;
    q.SA = (const uint8_t*)SA;
    q.SB = (const uint8_t*)SB;
    q.D = (uint16_t*)D;
    q.M = (int)M;
    q.N = (int)N;
    q.K = (int)K;
    q.lda = (int)lda;
    q.ldb = (int)ldb;
    q.ldsa = (int)ldsa;
    q.ldsb = (int)ldsb;
    q.ldd = (int)ldd;
    q.tiles_m = (int)plan[3];
    q.tiles_n = (int)plan[4];
    q.num_xcds = xcds;
    q.d_vec = (((uintptr_t)D & 7) == 0 && (ldd & 3) == 0) ? 1 : 0;
    const dim3 grid((unsigned)(plan[3] * plan[4])), block(SMALL_THREADS);
    if (plan[0] == 2 * SMALL_TILE && plan[1] == 2 * SMALL_TILE)
      hipLaunchKernelGGL((gemm_mx_small<2, 2>), grid, block, 0, stream, q);
    else if (plan[0] == 2 * SMALL_TILE)
      hipLaunchKernelGGL((gemm_mx_small<2, 1>), grid, block, 0, stream, q);
    else
      hipLaunchKernelGGL((gemm_mx_small<1, 1>), grid, block, 0, stream, q);
    return hipGetLastError() == hipSuccess ? DENSE_GEMM_OK : DENSE_GEMM_LAUNCH_FAILED;
  }
  MxParams p;
  p.A = (const uint8_t*)A;
  p.B = (const uint8_t*)B;
  p.D = (uint16_t*)D;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  p.lda = (int)lda;
  p.ldb = (int)ldb;
  p.ldd = (int)ldd;
  p.tiles_m = (int)plan[3];
  p.tiles_n = (int)plan[4];
  p.group_m = (int)plan[6];
  p.num_xcds = xcds;
  p.d_vec = (((uintptr_t)D & 15) == 0 && (ldd & 7) == 0) ? 1 : 0;
  p.nks = (int)((K + BKE - 1) / BKE);
  p.koff = (int)((BKE - K % BKE) % BKE);
  p.PSA = ws;
  p.PSB = ws + mp.panel_bytes[0];
  p.full_tasks = (int)mp.full_tasks;
  p.tiles = (int)mp.split_tiles;
  p.splits = (int)plan[8];
  p.split_steps = (int)plan[9];
  p.num_tasks = (int)(mp.full_tasks + mp.split_tiles * plan[8]);
  p.ws = plan[8] > 1 ? (float*)(ws + mp.panel_bytes[0] + mp.panel_bytes[1]) : nullptr;
  if (p.nks > 0) {
    PackArgs pk{{(const uint8_t*)SA, (const uint8_t*)SB}, {p.M, p.N}, {(int)ldsa, (int)ldsb},
                {p.tiles_m, p.tiles_n}};
    hipLaunchKernelGGL(scale_pack,
                       dim3((unsigned)(p.tiles_m + p.tiles_n),
                            (unsigned)((p.nks + PACK_STAGES - 1) / PACK_STAGES)),
                       dim3(256), 0, stream, pk, (int)(K / GROUP), p.nks, p.koff, ws);
  }
  const unsigned grid = (unsigned)(p.num_tasks < cus ? p.num_tasks : cus);
  if (p.splits > 1) {
    // whole tiles, then the parts of the split tiles writing FP32 partials,
    // summed in part order and rounded to BF16 by the reduction
    hipLaunchKernelGGL(gemm_mx_kernel<true>, dim3(grid), dim3(THREADS), 0, stream, p);
    const ReduceParams r = {p.D, p.ws, p.M, p.N, p.ldd, p.tiles_m, p.tiles_n, p.group_m,
                            p.full_tasks, p.splits, p.tiles, p.d_vec};
    enqueue_split_reduce<__bf16, BN, BM>(r, cus, stream);
  } else {
    hipLaunchKernelGGL(gemm_mx_kernel<false>, dim3(grid), dim3(THREADS), 0, stream, p);
  }
  return hipGetLastError() == hipSuccess ? DENSE_GEMM_OK : DENSE_GEMM_LAUNCH_FAILED;
}

}  // namespace mx
}  // namespace dg

using namespace dg;

extern "C" {

dense_gemm_status gemm_nt_e4m3_mx_workspace_size(int64_t M, int64_t N, int64_t K,
                                                  int64_t num_cus, size_t* bytes) {
  if (bytes == nullptr || num_cus < 0) return DENSE_GEMM_BAD_ARG;
  if (M < 0 || N < 0 || K < 0) return DENSE_GEMM_INVALID_DIM;
  if (K % mx::GROUP != 0) return DENSE_GEMM_BAD_ARG;
  const int64_t lim = (int64_t)1 << 31;
  if (M >= lim || N >= lim || K >= lim) return DENSE_GEMM_TOO_LARGE;
  *bytes = 0;
  if (M == 0 || N == 0) return DENSE_GEMM_OK;
  if (num_cus == 0) {
    int cus = 0, xcds = 1;
    const dense_gemm_status st = device_topology(&cus, &xcds);
    if (st != DENSE_GEMM_OK) return st;
    num_cus = cus;
  }
  MxPlan mp;
  const dense_gemm_status st = mx_plan_call(M, N, K, num_cus, &mp);
  if (st == DENSE_GEMM_OK) *bytes = mp.total();
  return st;
}

dense_gemm_status gemm_nt_e4m3_mx_ex(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                                     const void* SA, int64_t ldsa, const void* B, int64_t ldb,
                                     const void* SB, int64_t ldsb, void* D, int64_t ldd,
                                     void* workspace, size_t workspace_bytes,
                                     hipStream_t stream) {
  dense_gemm_status st = mx::validate(M, N, K, A, lda, SA, ldsa, B, ldb, SB, ldsb, D, ldd);
  if (st != DENSE_GEMM_OK || M == 0 || N == 0) return st;
  int cus = 0, xcds = 1;
  st = device_topology(&cus, &xcds);
  if (st != DENSE_GEMM_OK) return st;
  MxPlan mp;
  st = mx_plan_call(M, N, K, cus, &mp);
  if (st != DENSE_GEMM_OK) return st;
  const size_t need = mp.total();
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need) return DENSE_GEMM_WORKSPACE_TOO_SMALL;
    if (((uintptr_t)workspace & 255) != 0) return DENSE_GEMM_MISALIGNED;
  }
  return mx::enqueue(M, N, K, A, lda, SA, ldsa, B, ldb, SB, ldsb, D, ldd, mp, (uint8_t*)workspace,
                     cus, xcds, stream);
}

dense_gemm_status gemm_nt_e4m3_mx(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                                  const void* SA, int64_t ldsa, const void* B, int64_t ldb,
                                  const void* SB, int64_t ldsb, void* D, int64_t ldd,
                                  hipStream_t stream) {
  dense_gemm_status st = mx::validate(M, N, K, A, lda, SA, ldsa, B, ldb, SB, ldsb, D, ldd);
  if (st != DENSE_GEMM_OK || M == 0 || N == 0) return st;
  int cus = 0, xcds = 1;
  st = device_topology(&cus, &xcds);
  if (st != DENSE_GEMM_OK) return st;
  MxPlan mp;
  st = mx_plan_call(M, N, K, cus, &mp);
  if (st != DENSE_GEMM_OK) return st;
  // packed scale panels and split-K partials, stream-ordered workspace (none
  // for small outputs)
  const size_t need = mp.total();
  uint8_t* ws = nullptr;
  if (need > 0 && (hipMallocAsync((void**)&ws, need, stream) != hipSuccess || ws == nullptr)) {
    (void)hipGetLastError();
    return DENSE_GEMM_NO_MEMORY;
  }
  st = mx::enqueue(M, N, K, A, lda, SA, ldsa, B, ldb, SB, ldsb, D, ldd, mp, ws, cus, xcds, stream);
  if (ws != nullptr) (void)hipFreeAsync(ws, stream);
  return st;
}

}  // extern "C"
