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

// Products the small-output kernel computes (gemm_mx_small): M <= 128, K
// <= MX_SMALL_K_MAX, at most SMALL_MAX_TILES tiles of 16 x 16 or one tile
// row.  Measured per call against the tiled kernel (its scale packing and
// workspace included), one box: 128 x 128 x 4096 6.2 against 45.3 us,
// 1 x 4096 x 4096 6.2 against 44.5, 16 x 16384 x 4096 21.3 against 48.3,
// 128 x 1024 x 8192 12.3 against 75.6, 128 x 128 x 64 4.5 against 23.1.
static bool small_output(int64_t M, int64_t N, int64_t K) {
  if (M > SMALL_MAX || K > MX_SMALL_K_MAX) return false;
  const int64_t tiles = ((M + SMALL_TILE - 1) / SMALL_TILE) * ((N + SMALL_TILE - 1) / SMALL_TILE);
  return tiles <= SMALL_MAX_TILES || M <= SMALL_TILE;
}

// Workspace of a call: the packed scale panels, 1 KiB per 256-row tile of A
// and of B per 128-deep K stage (at least one stage); none for the
// small-output kernel, which stages the scales in LDS itself.
static size_t workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || small_output(M, N, K)) return 0;
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
  if (small_output(M, N, K)) {
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
    q.tiles_n = (int)((N + SMALL_TILE - 1) / SMALL_TILE);
    q.d_vec = (((uintptr_t)D & 7) == 0 && (ldd & 3) == 0) ? 1 : 0;
    const int64_t tiles = ((M + SMALL_TILE - 1) / SMALL_TILE) * q.tiles_n;
    hipLaunchKernelGGL(gemm_mx_small, dim3((unsigned)tiles), dim3(SMALL_THREADS), 0, stream, q);
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
  const size_t need = mx::workspace_bytes(M, N, K);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need) return DENSE_GEMM_WORKSPACE_TOO_SMALL;
    if (((uintptr_t)workspace & 255) != 0) return DENSE_GEMM_MISALIGNED;
  }
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
  // packed scale panels, stream-ordered workspace (none for small outputs)
  const size_t need = mx::workspace_bytes(M, N, K);
  uint8_t* ws = nullptr;
  if (need > 0 && (hipMallocAsync((void**)&ws, need, stream) != hipSuccess || ws == nullptr)) {
    (void)hipGetLastError();
    return DENSE_GEMM_NO_MEMORY;
  }
  st = mx::enqueue(M, N, K, A, lda, SA, ldsa, B, ldb, SB, ldsb, D, ldd, ws, cus, xcds, stream);
  if (ws != nullptr) (void)hipFreeAsync(ws, stream);
  return st;
}

}  // extern "C"
