// gemm_mx.hip -- host side of the FP8 block-scaled GEMM for the MI355X
// (gfx950): argument checks, workspace and the C ABI.  The operation and
// the kernel design are described in gemm_mx_kernel.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dense_gemm.h"
#include "gemm_mx_kernel.h"

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

// Workspace of a call: the packed scale panels, 1 KiB per 256-row tile of A
// and of B per 128-deep K stage (at least one stage).
static size_t workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0) return 0;
  const int64_t tiles = (M + BM - 1) / BM + (N + BN - 1) / BN;
  const int64_t nks = (K + BKE - 1) / BKE;
  return (size_t)tiles * (size_t)(nks > 0 ? nks : 1) * SC_BYTES;
}

// The launches of a validated call with M, N > 0 into a workspace of at
// least workspace_bytes(M, N, K).
static dense_gemm_status enqueue(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                                 const void* SA, int64_t ldsa, const void* B, int64_t ldb,
                                 const void* SB, int64_t ldsb, void* D, int64_t ldd, uint8_t* ws,
                                 int cus, int xcds, hipStream_t stream) {
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
  p.tiles_m = (int)((M + BM - 1) / BM);
  p.tiles_n = (int)((N + BN - 1) / BN);
  p.group_m = p.tiles_m < 8 ? p.tiles_m : 8;
  p.num_tasks = p.tiles_m * p.tiles_n;
  p.num_xcds = xcds;
  p.d_vec = (((uintptr_t)D & 15) == 0 && (ldd & 7) == 0) ? 1 : 0;
  p.nks = (int)((K + BKE - 1) / BKE);
  p.koff = (int)((BKE - K % BKE) % BKE);
  const size_t pa = (size_t)p.tiles_m * (p.nks > 0 ? p.nks : 1) * SC_BYTES;
  p.PSA = ws;
  p.PSB = ws + pa;
  if (p.nks > 0) {
    PackArgs pk{{(const uint8_t*)SA, (const uint8_t*)SB}, {p.M, p.N}, {(int)ldsa, (int)ldsb},
                {p.tiles_m, p.tiles_n}};
    hipLaunchKernelGGL(scale_pack,
                       dim3((unsigned)(p.tiles_m + p.tiles_n),
                            (unsigned)((p.nks + PACK_STAGES - 1) / PACK_STAGES)),
                       dim3(256), 0, stream, pk, (int)(K / GROUP), p.nks, p.koff, ws);
  }
  hipLaunchKernelGGL(gemm_mx_kernel, dim3((unsigned)(p.num_tasks < cus ? p.num_tasks : cus)),
                     dim3(THREADS), 0, stream, p);
  return hipGetLastError() == hipSuccess ? DENSE_GEMM_OK : DENSE_GEMM_LAUNCH_FAILED;
}

}  // namespace mx
}  // namespace dg

using namespace dg;

extern "C" {

dense_gemm_status gemm_nt_e4m3_mx_workspace_size(int64_t M, int64_t N, int64_t K, size_t* bytes) {
  if (bytes == nullptr) return DENSE_GEMM_BAD_ARG;
  if (M < 0 || N < 0 || K < 0) return DENSE_GEMM_INVALID_DIM;
  if (K % mx::GROUP != 0) return DENSE_GEMM_BAD_ARG;
  const int64_t lim = (int64_t)1 << 31;
  if (M >= lim || N >= lim || K >= lim) return DENSE_GEMM_TOO_LARGE;
  *bytes = mx::workspace_bytes(M, N, K);
  return DENSE_GEMM_OK;
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
  if (workspace == nullptr || workspace_bytes < mx::workspace_bytes(M, N, K))
    return DENSE_GEMM_WORKSPACE_TOO_SMALL;
  if (((uintptr_t)workspace & 255) != 0) return DENSE_GEMM_MISALIGNED;
  return mx::enqueue(M, N, K, A, lda, SA, ldsa, B, ldb, SB, ldsb, D, ldd, (uint8_t*)workspace,
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
  // packed scale panels, stream-ordered workspace
  uint8_t* ws = nullptr;
  if (hipMallocAsync((void**)&ws, mx::workspace_bytes(M, N, K), stream) != hipSuccess ||
      ws == nullptr) {
    (void)hipGetLastError();
    return DENSE_GEMM_NO_MEMORY;
  }
  st = mx::enqueue(M, N, K, A, lda, SA, ldsa, B, ldb, SB, ldsb, D, ldd, ws, cus, xcds, stream);
  (void)hipFreeAsync(ws, stream);
  return st;
}

}  // extern "C"
