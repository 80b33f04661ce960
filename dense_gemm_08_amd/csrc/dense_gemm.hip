// dense_gemm.hip -- host side of the FP16/BF16 tiled GEMM for the MI355X
// (gfx950): argument checks, the launch plan, workspaces and the C ABI.
//
// The operation (D = A @ B.T in FP16, D = A @ B in BF16, FP32 accumulation,
// one rounding to the output type) is defined in include/dense_gemm.h with
// its citations; the kernels are in gemm_kernel.h.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "dense_gemm.h"
#include "gemm_kernel.h"

namespace dg {

// ---- host side ----------------------------------------------------------

// Workgroups of a repack launch (capped; the kernel strides over the rest).
static unsigned repack_blocks(int64_t chunks) {
  const int64_t b = (chunks + 255) / 256;
  return (unsigned)(b < REPACK_MAX_BLOCKS ? b : REPACK_MAX_BLOCKS);
}

struct DeviceInfo {
  int cus = 0;
  int xcds = 1;
  bool gfx950 = false;
};

static std::mutex g_mu;
static DeviceInfo g_dev[64];
static bool g_dev_ok[64];

// Properties of the current device, queried once per device.  The XCD count
// (8 on an unpartitioned MI355X, fewer when the chip is partitioned into
// several devices) sets the workgroup-to-L2 remap of the tile scheduler.
static dense_gemm_status device_info(DeviceInfo* out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return DENSE_GEMM_NO_DEVICE;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_dev_ok[dev]) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return DENSE_GEMM_NO_DEVICE;
    int xcds = 1;
    if (hipDeviceGetAttribute(&xcds, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || xcds < 1) {
      (void)hipGetLastError();
      xcds = 1;
    }
    g_dev[dev].cus = prop.multiProcessorCount;
    g_dev[dev].xcds = xcds;
    g_dev[dev].gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    g_dev_ok[dev] = true;
  }
  *out = g_dev[dev];
  return out->gfx950 && out->cus > 0 ? DENSE_GEMM_OK : DENSE_GEMM_NO_DEVICE;
}

dense_gemm_status device_topology(int* cus, int* xcds) {
  DeviceInfo info;
  const dense_gemm_status st = device_info(&info);
  if (st == DENSE_GEMM_OK) {
    *cus = info.cus;
    *xcds = info.xcds;
  }
  return st;
}

static constexpr int64_t kMaxDim = (int64_t)1 << 31;

// Tile rows per group of the grouped order.  The workgroups resident on one
// XCD take consecutive tasks, i.e. a block of group_m tile rows by a few
// tile columns that shares its A and B panels in that XCD's L2; 8 rows made
// that block closest to square for the grids measured (32 workgroups per
// XCD at 4096^3: an 8 x 4 block of 12 panels).
static int choose_group_m(int64_t tiles_m) { return (int)(tiles_m < 8 ? tiles_m : 8); }

// Everything one call launches, decided on the host before any launch.
struct CallPlan {
  int64_t plan[10];          // as dense_gemm_plan, after the caller's options
  int64_t full_tasks;        // tiles computed whole
  int64_t split_tiles;       // tiles computed in K parts
  bool a_direct, b_direct;   // operands read in place (else repacked)
  size_t a_bytes, b_bytes;   // workspace of the repacked copies
  size_t split_bytes;        // workspace of the FP32 partial tiles
  size_t total() const { return a_bytes + b_bytes + split_bytes; }
};

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
  const int64_t tiles_m = (M + BM - 1) / BM;
  // Tile width: 256, or for A @ B.T 128 when 256-wide tiles would occupy at
  // most half the CUs (one wave) and the output is wider than 128: twice the
  // tiles, still one wave.  Narrow tiles read A twice as often, so they are
  // kept for operands that stay in the 256 MB Infinity Cache (at most
  // 192 MiB); beyond it (measured: 8192 x 1024 x 16384) 256-wide tiles with
  // split-K are faster.
  const int64_t t256 = tiles_m * ((N + BN - 1) / BN);
  const bool cached = K == 0 || (M + N) <= ((int64_t)96 << 20) / K;  // (M + N) K 2 B <= 192 MiB
  const int64_t tw = layout == NT && N > BN / 2 && 2 * t256 <= num_cus && cached ? BN / 2 : BN;
  const int64_t tiles_n = (N + tw - 1) / tw;
  const int64_t tasks = tiles_m * tiles_n;
  const int64_t grid = tasks < num_cus ? tasks : num_cus;
  out[0] = BM;
  out[1] = tw;
  out[2] = BK;
  out[3] = tiles_m;
  out[4] = tiles_n;
  out[5] = grid;
  out[6] = choose_group_m(tiles_m);
  out[7] = THREADS;
  // Split-K for the tiles of the last, partial wave (all tiles when there
  // are fewer than CUs), at most one part per idle CU and at least 4 K steps
  // per part.
  //   * Fewer tiles than CUs: the split (if any) with the least estimated
  //     time, from a model fitted to measured times on the MI355X (in units
  //     of 0.01 us): a K step of a 256-wide tile 105 (128-wide: 70), a split
  //     call's fixed cost (the reduce launch, the workspace) 1200 plus 12 per
  //     256-wide partial tile (6 per 128-wide one) for its FP32 write and
  //     read back.
  //   * After full waves: split when the last wave would leave at least
  //     three quarters of the CUs idle (measured: splitting a half-full last
  //     wave gains nothing), into as many parts as fit.
  const int64_t nk = (K + BK - 1) / BK;
  const int64_t rem = tasks % num_cus;
  int64_t splits = 1, steps = nk;
  if (rem > 0 && nk >= 8) {
    const int64_t by_cus = num_cus / rem, by_k = nk / 4;
    const int64_t most = by_cus < by_k ? by_cus : by_k;
    if (tasks < num_cus) {
      const int64_t step_cost = tw == BN ? 105 : 70, part_cost = tw == BN ? 12 : 6;
      int64_t best = nk * step_cost;
      for (int64_t sp = 2; sp <= most; ++sp) {
        const int64_t st = (nk + sp - 1) / sp, parts = (nk + st - 1) / st;
        const int64_t t = st * step_cost + 1200 + part_cost * parts * rem;
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
  out[8] = splits;
  out[9] = steps;
  if (splits > 1 && tasks < num_cus) out[5] = tasks * splits;
  return DENSE_GEMM_OK;
}

}  // extern "C"

namespace dg {

static bool valid_op(int op) { return op >= DENSE_GEMM_NT_F16 && op <= DENSE_GEMM_NN_F16; }
static int op_layout(int op) { return op == DENSE_GEMM_NN_BF16 || op == DENSE_GEMM_NN_F16 ? NN : NT; }

// The plan of one call on a device with `cus` CUs: dense_gemm_plan, the
// caller's options, and the workspace the call needs.  Arguments must have
// passed dense_gemm_validate, with M, N > 0.
static dense_gemm_status plan_call(int layout, int64_t M, int64_t N, int64_t K, const void* A,
                                   int64_t lda, const void* B, int64_t ldb, int64_t cus,
                                   const dense_gemm_options* opt, CallPlan* cp) {
  int64_t* plan = cp->plan;
  dense_gemm_status st = dense_gemm_plan(layout, M, N, K, cus, plan);
  if (st != DENSE_GEMM_OK) return st;
  const int64_t nk = (K + BK - 1) / BK;
  bool forced_split = false;
  if (opt != nullptr) {
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
  if (plan[8] > 1) {
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
  auto round256 = [](size_t x) { return (x + 255) & ~(size_t)255; };
  cp->a_bytes = cp->a_direct ? 0 : round256((size_t)M * K8 * 2);
  cp->b_bytes = cp->b_direct ? 0 : round256((size_t)b_rows * b_dcols * 2);
  cp->split_bytes = plan[8] > 1 ? (size_t)plan[8] * cp->split_tiles * BM * plan[1] * sizeof(float) : 0;
  return DENSE_GEMM_OK;
}

// The launches of one call with tile width TN, given its plan and a
// workspace of at least cp.total() bytes (256-byte aligned; null when the
// plan needs none).
template <typename T, int LAYOUT, int TN>
static dense_gemm_status enqueue(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                                 const void* B, int64_t ldb, void* D, int64_t ldd,
                                 const CallPlan& cp, const DeviceInfo& info, char* ws,
                                 hipStream_t stream) {
  const int64_t* plan = cp.plan;
  Params p;
  p.A = (const uint16_t*)A;
  p.B = (const uint16_t*)B;
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
  p.num_xcds = info.xcds;
  p.d_vec = (((uintptr_t)D & 15) == 0 && (ldd & 7) == 0) ? 1 : 0;
  p.full_tasks = (int)cp.full_tasks;
  p.tiles = (int)cp.split_tiles;
  p.splits = (int)plan[8];
  p.split_steps = (int)plan[9];
  p.num_tasks = (int)(cp.full_tasks + cp.split_tiles * plan[8]);
  p.ws = plan[8] > 1 ? (float*)(ws + cp.a_bytes + cp.b_bytes) : nullptr;

  const int64_t K8 = (K + 7) & ~(int64_t)7, N8 = (N + 7) & ~(int64_t)7;
  if (!cp.a_direct) {
    uint16_t* a2 = (uint16_t*)ws;
    hipLaunchKernelGGL(repack, dim3(repack_blocks(M * (K8 / 8))), dim3(256), 0, stream,
                       (const uint16_t*)A, M, K, lda, a2, K8);
    p.A = a2;
    p.lda = (int)K8;
  }
  if (!cp.b_direct) {
    const int64_t b_rows = LAYOUT == NT ? N : K, b_cols = LAYOUT == NT ? K : N;
    const int64_t b_dcols = LAYOUT == NT ? K8 : N8;
    uint16_t* b2 = (uint16_t*)(ws + cp.a_bytes);
    hipLaunchKernelGGL(repack, dim3(repack_blocks(b_rows * (b_dcols / 8))), dim3(256), 0, stream,
                       (const uint16_t*)B, b_rows, b_cols, ldb, b2, b_dcols);
    p.B = b2;
    p.ldb = (int)b_dcols;
  }
  const unsigned grid = (unsigned)(p.num_tasks < info.cus ? p.num_tasks : info.cus);
  if (p.splits > 1) {
    // whole tiles, then the parts of the split tiles writing FP32 partials,
    // summed by a second kernel
    hipLaunchKernelGGL((gemm_kernel<T, LAYOUT, true, TN>), dim3(grid), dim3(THREADS), 0, stream, p);
    hipLaunchKernelGGL((split_reduce<T, TN>), dim3((unsigned)(p.tiles * (TN / 8))), dim3(256), 0,
                       stream, p);
  } else {
    hipLaunchKernelGGL((gemm_kernel<T, LAYOUT, false, TN>), dim3(grid), dim3(THREADS), 0, stream,
                       p);
  }
  return hipGetLastError() == hipSuccess ? DENSE_GEMM_OK : DENSE_GEMM_LAUNCH_FAILED;
}

template <typename T, int LAYOUT>
static dense_gemm_status enqueue_width(int64_t M, int64_t N, int64_t K, const void* A,
                                       int64_t lda, const void* B, int64_t ldb, void* D,
                                       int64_t ldd, const CallPlan& cp, const DeviceInfo& info,
                                       char* ws, hipStream_t stream) {
  if constexpr (LAYOUT == NT) {
    if (cp.plan[1] == BN / 2)
      return enqueue<T, LAYOUT, BN / 2>(M, N, K, A, lda, B, ldb, D, ldd, cp, info, ws, stream);
  }
  return enqueue<T, LAYOUT, BN>(M, N, K, A, lda, B, ldb, D, ldd, cp, info, ws, stream);
}

// A call with the caller's workspace (ws, ws_bytes): nothing is allocated.
template <typename T, int LAYOUT>
static dense_gemm_status run_with(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                                  const void* B, int64_t ldb, void* D, int64_t ldd,
                                  const dense_gemm_options* opt, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  dense_gemm_status st = dense_gemm_validate(LAYOUT, M, N, K, A, lda, B, ldb, D, ldd);
  if (st != DENSE_GEMM_OK || M == 0 || N == 0) return st;
  DeviceInfo info;
  st = device_info(&info);
  if (st != DENSE_GEMM_OK) return st;
  CallPlan cp;
  st = plan_call(LAYOUT, M, N, K, A, lda, B, ldb, info.cus, opt, &cp);
  if (st != DENSE_GEMM_OK) return st;
  if (cp.total() > 0) {
    if (ws == nullptr || ws_bytes < cp.total()) return DENSE_GEMM_WORKSPACE_TOO_SMALL;
    if (((uintptr_t)ws & 255) != 0) return DENSE_GEMM_MISALIGNED;
  }
  return enqueue_width<T, LAYOUT>(M, N, K, A, lda, B, ldb, D, ldd, cp, info, (char*)ws, stream);
}

// ---- the entry point that allocates nothing --------------------------------
// gemm_nt_f16_noalloc takes its scratch memory (split-K partial tiles and
// repacked operands) from this fixed array instead of the caller or the
// allocator.  Each device the library runs on holds its own copy, from the
// code object's load until the process ends.  64 MiB holds every split-K
// plan on a 256-CU device (at most one partial tile of 256 KiB per CU) and
// repacked operands up to that size.  In host code `scratch` only stands in
// for the symbol: its device address, looked up once per device with that
// device current, is what the launches take.
constexpr size_t SCRATCH_BYTES = (size_t)64 << 20;
static __device__ __align__(256) char scratch[SCRATCH_BYTES];

static void* g_scratch[64];
static bool g_scratch_ok[64];

static dense_gemm_status scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return DENSE_GEMM_NO_DEVICE;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch_ok[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return DENSE_GEMM_NO_MEMORY;
    }
    g_scratch[dev] = ptr;
    g_scratch_ok[dev] = true;
  }
  *out = g_scratch[dev];
  return DENSE_GEMM_OK;
}

// A call with the device's fixed scratch array: the library's own plan,
// rejected (before any launch) if it needs more than the array holds.
template <typename T, int LAYOUT>
static dense_gemm_status run_noalloc(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                                     const void* B, int64_t ldb, void* D, int64_t ldd,
                                     hipStream_t stream) {
  dense_gemm_status st = dense_gemm_validate(LAYOUT, M, N, K, A, lda, B, ldb, D, ldd);
  if (st != DENSE_GEMM_OK || M == 0 || N == 0) return st;
  DeviceInfo info;
  st = device_info(&info);
  if (st != DENSE_GEMM_OK) return st;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != DENSE_GEMM_OK) return st;
  CallPlan cp;
  st = plan_call(LAYOUT, M, N, K, A, lda, B, ldb, info.cus, nullptr, &cp);
  if (st != DENSE_GEMM_OK) return st;
  if (cp.total() > SCRATCH_BYTES) return DENSE_GEMM_SCRATCH_TOO_SMALL;
  return enqueue_width<T, LAYOUT>(M, N, K, A, lda, B, ldb, D, ldd, cp, info, (char*)ws, stream);
}

// A call of the plain entry points: the workspace (if the plan needs one)
// is taken with hipMallocAsync on `stream` and returned with hipFreeAsync
// after the launches.  A split call that cannot get its workspace runs
// unsplit; a repack that cannot get it returns DENSE_GEMM_NO_MEMORY.
template <typename T, int LAYOUT>
static dense_gemm_status run(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                             const void* B, int64_t ldb, void* D, int64_t ldd,
                             hipStream_t stream) {
  dense_gemm_status st = dense_gemm_validate(LAYOUT, M, N, K, A, lda, B, ldb, D, ldd);
  if (st != DENSE_GEMM_OK || M == 0 || N == 0) return st;
  DeviceInfo info;
  st = device_info(&info);
  if (st != DENSE_GEMM_OK) return st;
  CallPlan cp;
  st = plan_call(LAYOUT, M, N, K, A, lda, B, ldb, info.cus, nullptr, &cp);
  if (st != DENSE_GEMM_OK) return st;
  char* ws = nullptr;
  if (cp.total() > 0 && hipMallocAsync((void**)&ws, cp.total(), stream) != hipSuccess) {
    (void)hipGetLastError();
    ws = nullptr;
    if (cp.split_bytes > 0) {
      // retry without the partials: run unsplit, same tile width
      const dense_gemm_options unsplit = {1, (int32_t)cp.plan[1]};
      st = plan_call(LAYOUT, M, N, K, A, lda, B, ldb, info.cus, &unsplit, &cp);
      if (st != DENSE_GEMM_OK) return st;
    }
    if (cp.total() > 0 && hipMallocAsync((void**)&ws, cp.total(), stream) != hipSuccess) {
      (void)hipGetLastError();
      return DENSE_GEMM_NO_MEMORY;
    }
  }
  st = enqueue_width<T, LAYOUT>(M, N, K, A, lda, B, ldb, D, ldd, cp, info, ws, stream);
  if (ws != nullptr) (void)hipFreeAsync(ws, stream);
  return st;
}

template <typename T, int LAYOUT>
static dense_gemm_status run_op_ex(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                                   const void* B, int64_t ldb, void* D, int64_t ldd,
                                   const dense_gemm_options* opt, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
  return run_with<T, LAYOUT>(M, N, K, A, lda, B, ldb, D, ldd, opt, ws, ws_bytes, stream);
}

}  // namespace dg

extern "C" {

dense_gemm_status gemm_nt_f16(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                              const void* B, int64_t ldb, void* D, int64_t ldd,
                              hipStream_t stream) {
  return run<_Float16, NT>(M, N, K, A, lda, B, ldb, D, ldd, stream);
}

dense_gemm_status gemm_nn_bf16(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                               const void* B, int64_t ldb, void* D, int64_t ldd,
                               hipStream_t stream) {
  return run<__bf16, NN>(M, N, K, A, lda, B, ldb, D, ldd, stream);
}

dense_gemm_status gemm_nt_bf16(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                               const void* B, int64_t ldb, void* D, int64_t ldd,
                               hipStream_t stream) {
  return run<__bf16, NT>(M, N, K, A, lda, B, ldb, D, ldd, stream);
}

dense_gemm_status gemm_nn_f16(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda,
                              const void* B, int64_t ldb, void* D, int64_t ldd,
                              hipStream_t stream) {
  return run<_Float16, NN>(M, N, K, A, lda, B, ldb, D, ldd, stream);
}

dense_gemm_status gemm_nt_f16_noalloc(int64_t M, int64_t N, int64_t K, const void* A,
                                      int64_t lda, const void* B, int64_t ldb, void* D,
                                      int64_t ldd, hipStream_t stream) {
  return run_noalloc<_Float16, NT>(M, N, K, A, lda, B, ldb, D, ldd, stream);
}

dense_gemm_status dense_gemm_workspace_size(int op, int64_t M, int64_t N, int64_t K,
                                            const void* A, int64_t lda, const void* B,
                                            int64_t ldb, int64_t num_cus,
                                            const dense_gemm_options* opt, size_t* bytes) {
  if (!valid_op(op) || bytes == nullptr || num_cus < 0) return DENSE_GEMM_BAD_ARG;
  const int layout = op_layout(op);
  // D is not looked at beyond its null check: any non-null stand-in will do
  dense_gemm_status st =
      dense_gemm_validate(layout, M, N, K, A, lda, B, ldb, (const void*)(uintptr_t)16, N);
  if (st != DENSE_GEMM_OK) return st;
  *bytes = 0;
  if (M == 0 || N == 0) return DENSE_GEMM_OK;
  if (num_cus == 0) {
    DeviceInfo info;
    st = device_info(&info);
    if (st != DENSE_GEMM_OK) return st;
    num_cus = info.cus;
  }
  CallPlan cp;
  st = plan_call(layout, M, N, K, A, lda, B, ldb, num_cus, opt, &cp);
  if (st == DENSE_GEMM_OK) *bytes = cp.total();
  return st;
}

dense_gemm_status dense_gemm_ex(int op, int64_t M, int64_t N, int64_t K, const void* A,
                                int64_t lda, const void* B, int64_t ldb, void* D, int64_t ldd,
                                const dense_gemm_options* opt, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  switch (op) {
    case DENSE_GEMM_NT_F16:
      return run_op_ex<_Float16, NT>(M, N, K, A, lda, B, ldb, D, ldd, opt, workspace,
                                     workspace_bytes, stream);
    case DENSE_GEMM_NN_BF16:
      return run_op_ex<__bf16, NN>(M, N, K, A, lda, B, ldb, D, ldd, opt, workspace,
                                   workspace_bytes, stream);
    case DENSE_GEMM_NT_BF16:
      return run_op_ex<__bf16, NT>(M, N, K, A, lda, B, ldb, D, ldd, opt, workspace,
                                   workspace_bytes, stream);
    case DENSE_GEMM_NN_F16:
      return run_op_ex<_Float16, NN>(M, N, K, A, lda, B, ldb, D, ldd, opt, workspace,
                                     workspace_bytes, stream);
    default:
      return DENSE_GEMM_BAD_ARG;
  }
}

}  // extern "C"
