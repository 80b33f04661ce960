// host_fuzz.cpp -- exercises the host-side planning code of the library
// (dense_gemm_08_amd/csrc/plan.cpp: the argument check, the tile scheduler
// helpers, the FP16/BF16 launch plan with options, the FP8 plan, the
// workspace sizes) over edge and random arguments, and checks the plans'
// invariants.  tests/test_sanitizers.py
// builds it with -fsanitize=address,undefined, so an out-of-bounds access,
// a signed overflow or any other undefined behaviour also ends the run.
// Prints "ok" and exits 0 on success.
#include <stdint.h>
#include <stdio.h>

#include <random>
#include <vector>

#include "dense_gemm.h"
#include "plan.h"

using namespace dg;

static long fails = 0;
#define CHECK(c)                                                              \
  do {                                                                        \
    if (!(c)) {                                                               \
      if (fails < 20) fprintf(stderr, "line %d: check failed: %s\n", __LINE__, #c); \
      ++fails;                                                                \
    }                                                                         \
  } while (0)

static int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
// a + b - c, saturated to [INT64_MIN, INT64_MAX] (the driver's own arithmetic
// on extreme arguments must not overflow)
static int64_t sat(int64_t a, int64_t b, int64_t c = 0) {
  __int128 v = (__int128)a + b - c;
  if (v > INT64_MAX) return INT64_MAX;
  if (v < INT64_MIN) return INT64_MIN;
  return (int64_t)v;
}

static void check_repack(int layout, int64_t M, int64_t N, int64_t K, const CallPlan& cp) {
  const int64_t K8 = (K + 7) & ~(int64_t)7, N8 = (N + 7) & ~(int64_t)7;
  if (!cp.a_direct) CHECK(cp.a_bytes >= (size_t)(M * K8 * 2) && cp.a_bytes % 256 == 0);
  if (!cp.b_direct) CHECK(cp.b_bytes >= (size_t)((layout == NT ? N * K8 : K * N8) * 2));
  if (cp.a_direct) CHECK(cp.a_bytes == 0);
  if (cp.b_direct) CHECK(cp.b_bytes == 0);
}

static void check_plan(int layout, int64_t M, int64_t N, int64_t K, int64_t cus,
                       const dense_gemm_options* opt, const CallPlan& cp) {
  const int64_t* p = cp.plan;
  const bool options = opt && (opt->split_k != 0 || opt->tile_n != 0);
  // the small-output kernel exactly where its rule holds and no option asks
  // for the tiled kernel
  CHECK(cp.small() == (small_output(layout, M, N, K) && !options));
  if (cp.small()) {
    CHECK(M <= SMALL_MAX && K <= SMALL_K_MAX);
    CHECK(layout == NT || (K <= SMALL_NN_K_MAX && ceil_div(M, SMALL_TILE) * N * K <= SMALL_NN_ELEMS));
    // A @ B.T: the tile small_tile gives (16 x 16 for one 16-row tile row,
    // else the largest whose grid covers the CUs); A @ B: 16 x 16
    const int64_t tr = p[0], tc = p[1];
    int64_t er = SMALL_TILE, ec = SMALL_TILE;
    if (layout == NT) small_tile(M, N, cus, &er, &ec);
    CHECK(tr == er && tc == ec);
    CHECK((tr == 16 && tc == 16) || (tr == 32 && (tc == 16 || tc == 32)));
    if (tc == 32) CHECK(ceil_div(M, 32) * ceil_div(N, 32) >= cus);
    if (tr == 32 && tc == 16) CHECK(ceil_div(M, 32) * ceil_div(N, 16) >= cus);
    CHECK(p[2] == BK && p[7] == SMALL_THREADS);
    CHECK(p[3] == ceil_div(M, tr) && p[4] == ceil_div(N, tc));
    CHECK(p[5] == p[3] * p[4] && cp.full_tasks == p[5]);
    const int64_t t16 = ceil_div(M, 16) * ceil_div(N, 16), t32 = ceil_div(M, 32) * ceil_div(N, 32);
    CHECK(M <= SMALL_TILE || t16 <= SMALL_MAX_TILES || (layout == NT && t32 * K <= SMALL_T32_K));
    CHECK(p[8] == 1 && cp.split_tiles == 0 && cp.split_bytes == 0);
    check_repack(layout, M, N, K, cp);
    return;
  }
  // 128 tile rows exactly when M <= 128
  CHECK(p[0] == (M <= BM / 2 ? BM / 2 : BM) && p[2] == BK && p[7] == THREADS);
  CHECK(p[1] == BN || (p[1] == BN / 2 && layout == NT));
  if (opt && opt->tile_n) CHECK(p[1] == opt->tile_n);
  CHECK(p[3] == ceil_div(M, p[0]) && p[4] == ceil_div(N, p[1]));
  CHECK(p[6] >= 1 && p[6] <= 8 && p[6] <= p[3]);
  const int64_t tasks = p[3] * p[4], nk = ceil_div(K, BK);
  CHECK(cp.full_tasks + cp.split_tiles == tasks);
  CHECK(p[5] >= 1 && p[5] <= cus);
  CHECK(p[8] >= 1);
  if (p[8] > 1) {
    // every K step in exactly one part, no empty part
    CHECK(p[8] * p[9] >= nk && (p[8] - 1) * p[9] < nk);
    CHECK(cp.split_tiles > 0);
    CHECK(cp.split_bytes == (size_t)p[8] * (size_t)cp.split_tiles * (size_t)p[0] * (size_t)p[1] * 4);
    if (!(opt && opt->split_k > 1)) {
      // the library's own split: the last partial wave, at most one part per CU
      CHECK(cp.split_tiles == (tasks < cus ? tasks : tasks % cus));
      CHECK(cp.split_tiles * p[8] <= cus);
      CHECK(p[9] >= 4);
    }
  } else {
    CHECK(cp.split_tiles == 0 && cp.split_bytes == 0);
  }
  if (opt && opt->split_k == 1) CHECK(p[8] == 1);
  check_repack(layout, M, N, K, cp);
}

// The FP8 plan's invariants (mx_plan_call succeeded for M, N > 0).
static void check_mx_plan(int64_t M, int64_t N, int64_t K, int64_t cus, const MxPlan& mp) {
  const int64_t* p = mp.plan;
  const int64_t nks = ceil_div(K, mx::BKE);
  CHECK(mp.small() == mx_small_output(M, N, K));
  CHECK(p[2] == mx::BKE && p[9] >= 0);
  if (mp.small()) {
    CHECK(M <= SMALL_MAX && K <= mx::MX_SMALL_K_MAX);
    const int64_t t32 = ceil_div(M, 32) * ceil_div(N, 32);
    CHECK(M <= SMALL_TILE || t32 <= mx::MX_SMALL_T32 ||
          (t32 <= mx::MX_SMALL_T32_MAX && t32 * K <= mx::MX_SMALL_T32_K));
    // tiles of 16 x 16, 32 x 16 or 32 x 32: the largest whose grid covers
    // the CUs, 16 x 16 for one 16-row tile row
    const int64_t tr = p[0], tc = p[1];
    int64_t er, ec;
    small_tile(M, N, cus, &er, &ec);
    CHECK(tr == er && tc == ec);
    CHECK((tr == 16 && tc == 16) || (tr == 32 && (tc == 16 || tc == 32)));
    CHECK(p[3] == ceil_div(M, tr) && p[4] == ceil_div(N, tc) && p[5] == p[3] * p[4]);
    if (M <= SMALL_TILE) {
      CHECK(tr == 16);
    } else if (tc == 32) {
      CHECK(p[5] >= cus);
    } else if (tr == 32) {
      CHECK(p[5] >= cus && t32 < cus);
    } else {
      CHECK(ceil_div(M, 32) * ceil_div(N, 16) < cus);
    }
    CHECK(p[6] == 1 && p[7] == SMALL_THREADS && p[8] == 1 && p[9] == nks && mp.total() == 0);
    return;
  }
  CHECK(p[0] == mx::BM && p[1] == mx::BN && p[7] == THREADS);
  CHECK(p[3] == ceil_div(M, mx::BM) && p[4] == ceil_div(N, mx::BN));
  CHECK(p[6] >= 1 && p[6] <= 8 && p[6] <= p[3]);
  const int64_t tasks = p[3] * p[4];
  CHECK(mp.full_tasks + mp.split_tiles == tasks);
  CHECK(p[5] >= 1 && p[5] <= cus);
  const size_t stages = (size_t)(nks > 0 ? nks : 1);
  CHECK(mp.panel_bytes[0] == (size_t)p[3] * stages * mx::SC_BYTES);
  CHECK(mp.panel_bytes[1] == (size_t)p[4] * stages * mx::SC_BYTES);
  if (p[8] > 1) {
    CHECK(p[8] * p[9] >= nks && (p[8] - 1) * p[9] < nks && p[9] >= 4);
    CHECK(mp.split_tiles == (tasks < cus ? tasks : tasks % cus) && mp.split_tiles > 0);
    CHECK(mp.split_tiles * p[8] <= cus);
    CHECK(mp.split_bytes == (size_t)p[8] * (size_t)mp.split_tiles * mx::BM * mx::BN * 4);
  } else {
    CHECK(p[9] == nks && mp.split_tiles == 0 && mp.split_bytes == 0);
  }
}

int main() {
  std::mt19937_64 rng(20261202);
  auto pick = [&](const std::vector<int64_t>& v) { return v[rng() % v.size()]; };
  const std::vector<int64_t> dims = {-1, 0, 1, 7, 8, 9, 63, 64, 65, 127, 128, 129, 255, 256, 257,
                                     1000, 3000, 4096, 4097, 5120, 17408, 1 << 20, 16777208,
                                     16777216, (1LL << 31) - 1, 1LL << 31, INT64_MAX};
  const std::vector<int64_t> extra = {0, 0, 0, 1, 5, 8, 13, 1 << 20, 1LL << 31, INT64_MAX / 4};
  const std::vector<int64_t> ptrs = {0, 1, 2, 16, 18, 256, 4096 + 6};
  const std::vector<int64_t> cus_list = {1, 8, 80, 255, 256, 304};
  const std::vector<int64_t> splits = {0, 0, 1, 2, 3, 7, 16, 64, 1 << 20, -1};
  const std::vector<int64_t> tns = {0, 0, 128, 256, 64};
  long planned = 0;
  for (long it = 0; it < 300000; ++it) {
    const int layout = (int)(rng() % 3) - (it % 97 == 0 ? 1 : 0);  // mostly 0/1, some invalid
    int64_t M = pick(dims), N = pick(dims), K = pick(dims);
    if (rng() % 2) M = (int64_t)(rng() % 9000);
    if (rng() % 2) N = (int64_t)(rng() % 20000);
    if (rng() % 2) K = (int64_t)(rng() % 20000);
    const int64_t lda = sat(K, pick(extra), rng() % 16 == 0 ? 1 : 0);
    const int64_t ldb = sat(layout == NN ? N : K, pick(extra));
    const int64_t ldd = sat(N, pick(extra), rng() % 16 == 0 ? 1 : 0);
    const void* A = (const void*)(uintptr_t)pick(ptrs);
    const void* B = (const void*)(uintptr_t)pick(ptrs);
    const void* D = (const void*)(uintptr_t)pick(ptrs);
    const dense_gemm_status st = dense_gemm_validate(layout, M, N, K, A, lda, B, ldb, D, ldd);
    CHECK(st >= DENSE_GEMM_OK && st <= DENSE_GEMM_BAD_ARG);
    if (st != DENSE_GEMM_OK || M <= 0 || N <= 0) continue;
    CHECK(layout == NT || layout == NN);
    CHECK(M < kMaxDim && N < kMaxDim && K < kMaxDim && ldd >= N);
    const int64_t cus = pick(cus_list);
    dense_gemm_options o = {(int32_t)pick(splits), (int32_t)pick(tns)};
    const dense_gemm_options* opt = rng() % 3 ? &o : nullptr;
    CallPlan cp;
    const dense_gemm_status ps = plan_call(layout, M, N, K, A, lda, B, ldb, cus, opt, &cp);
    const bool bad_opt = opt && (o.split_k < 0 ||
                                 (o.tile_n != 0 && o.tile_n != BN && !(o.tile_n == BN / 2 && layout == NT)));
    // TOO_LARGE only for a workspace beyond 2^62 bytes (a forced split of a
    // huge product)
    CHECK(ps == (bad_opt ? DENSE_GEMM_BAD_ARG : DENSE_GEMM_OK) ||
          (!bad_opt && ps == DENSE_GEMM_TOO_LARGE && opt && o.split_k > 1));
    if (ps != DENSE_GEMM_OK) continue;
    CHECK(cp.total() <= ((size_t)1 << 62));
    check_plan(layout, M, N, K, cus, opt, cp);
    ++planned;
    // the public planner agrees with the call plan when no option is given
    int64_t out[10];
    CHECK(dense_gemm_plan(layout, M, N, K, cus, out) == DENSE_GEMM_OK);
    if (!opt) {
      for (int i = 0; i < 5; ++i) CHECK(out[i] == cp.plan[i]);
      CHECK(out[8] == cp.plan[8]);
    }
  }
  // the FP8 plan
  long mx_planned = 0;
  for (long it = 0; it < 200000; ++it) {
    int64_t M = pick(dims), N = pick(dims), K = pick(dims);
    if (rng() % 2) M = (int64_t)(rng() % 9000);
    if (rng() % 2) N = (int64_t)(rng() % 20000);
    if (rng() % 2) K = 32 * (int64_t)(rng() % 700);
    const int64_t cus = rng() % 8 == 0 ? (int64_t)(rng() % 4) - 1 : pick(cus_list);
    MxPlan mp;
    const dense_gemm_status st = mx_plan_call(M, N, K, cus, &mp);
    const bool args_ok = M > 0 && N > 0 && K >= 0 && K % 32 == 0 && cus > 0 && M < kMaxDim &&
                         N < kMaxDim && K < kMaxDim;
    if (!args_ok) {
      CHECK(st == DENSE_GEMM_BAD_ARG);
      continue;
    }
    const bool many_tiles = ceil_div(M, mx::BM) * ceil_div(N, mx::BN) >= kMaxDim;
    CHECK(st == (many_tiles && !mx_small_output(M, N, K) ? DENSE_GEMM_TOO_LARGE : DENSE_GEMM_OK));
    if (st != DENSE_GEMM_OK) continue;
    check_mx_plan(M, N, K, cus, mp);
    ++mx_planned;
  }
  CHECK(mx_planned > 1000);
  // the public planner's own argument check
  int64_t out[10];
  CHECK(dense_gemm_plan(2, 8, 8, 8, 256, out) == DENSE_GEMM_BAD_ARG);
  CHECK(dense_gemm_plan(0, 0, 8, 8, 256, out) == DENSE_GEMM_BAD_ARG);
  CHECK(dense_gemm_plan(0, 8, 8, -1, 256, out) == DENSE_GEMM_BAD_ARG);
  CHECK(dense_gemm_plan(0, 8, 8, 8, 0, out) == DENSE_GEMM_BAD_ARG);
  CHECK(dense_gemm_plan(0, 8, 8, 8, 256, nullptr) == DENSE_GEMM_BAD_ARG);
  // the scheduler: a bijection of tasks onto tiles, and of workgroups onto slots
  for (int it = 0; it < 3000; ++it) {
    const int64_t tm = 1 + rng() % 40, tn = 1 + rng() % 40, g = 1 + rng() % 17;
    std::vector<char> seen(tm * tn, 0);
    for (int64_t t = 0; t < tm * tn; ++t) {
      int64_t a = -1, b = -1;
      CHECK(dense_gemm_tile_of_task(t, tm, tn, g, &a, &b) == DENSE_GEMM_OK);
      CHECK(a >= 0 && a < tm && b >= 0 && b < tn);
      if (a >= 0 && a < tm && b >= 0 && b < tn) {
        CHECK(!seen[a * tn + b]);
        seen[a * tn + b] = 1;
      }
    }
    int64_t a, b;
    CHECK(dense_gemm_tile_of_task(tm * tn, tm, tn, g, &a, &b) == DENSE_GEMM_BAD_ARG);
    CHECK(dense_gemm_tile_of_task(-1, tm, tn, g, &a, &b) == DENSE_GEMM_BAD_ARG);
    CHECK(dense_gemm_tile_of_task(0, tm, tn, 0, &a, &b) == DENSE_GEMM_BAD_ARG);
    CHECK(dense_gemm_tile_of_task(0, tm, tn, g, nullptr, &b) == DENSE_GEMM_BAD_ARG);
  }
  int64_t a, b;
  CHECK(dense_gemm_tile_of_task(0, 1LL << 31, 2, 8, &a, &b) == DENSE_GEMM_BAD_ARG);
  for (int64_t grid = 1; grid <= 600; ++grid) {
    for (int64_t x = 1; x <= 8; ++x) {
      std::vector<char> seen(grid, 0);
      for (int64_t w = 0; w < grid; ++w) {
        const int64_t s = dense_gemm_xcd_slot(w, grid, x);
        CHECK(s >= 0 && s < grid);
        if (s >= 0 && s < grid) {
          CHECK(!seen[s]);
          seen[s] = 1;
        }
      }
      CHECK(dense_gemm_xcd_slot(grid, grid, x) == -1);
    }
  }
  CHECK(dense_gemm_xcd_slot(0, 0, 8) == -1 && dense_gemm_xcd_slot(0, 8, 0) == -1);
  for (int s = -2; s < 14; ++s) CHECK(dense_gemm_status_string(s) != nullptr);
  if (fails) {
    fprintf(stderr, "%ld checks failed\n", fails);
    return 1;
  }
  printf("ok: %ld plans checked\n", planned);
  return 0;
}
