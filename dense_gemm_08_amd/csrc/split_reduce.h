// split_reduce.h -- the second kernel of a split-K product on the MI355X
// (gfx950), shared by the FP16/BF16 GEMM (gemm_kernel.h) and the FP8
// block-scaled GEMM (gemm_mx_kernel.h): the sum of the FP32 partial tiles of
// every split tile, in part order, rounded once to the 16-bit output type.
// The sum is the one the unsplit kernel forms (TileFoundry's schedule
// tutorial, section 1: FP32 accumulation of the K blocks' products), with
// its K range cut into parts whose sums are added in a fixed order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cdna_ops.h"
#include "tile_sched.h"

namespace dg {

// What the reduction reads and writes.  Split tile st (0 .. tiles-1) is
// task full_tasks + st of the grouped order over tiles_m x tiles_n tiles of
// TM x TN; part k of it is the row-major TM x TN FP32 tile at ws + (k *
// tiles + st) * TM * TN, of which only the 16 x 16 blocks inside D were
// written.
struct ReduceParams {
  uint16_t* D;
  const float* ws;
  int M, N, ldd;
  int tiles_m, tiles_n, group_m;
  int full_tasks, splits, tiles;
  int d_vec;  // D rows are 16-byte aligned (16-byte stores allowed)
};

// One thread per 8 consecutive columns of a row, RT threads per workgroup:
// a workgroup covers RT / (TN / 8) rows, a split tile TM * TN / (8 RT)
// workgroups.  The launch takes RT = 64 (one wave) when 256-thread
// workgroups would be fewer than the CUs, so that the partials' reads spread
// over more CUs (measured with 16 parts of one 128 x 128 output: 3.1 against
// 3.6 us), and RT = 256 otherwise (one-wave workgroups measured up to 1%
// slower on the split products of the M = 8192 sweep).
template <int TN, int RT, int TM>
constexpr int reduce_blocks_per_tile() { return TM * TN / (8 * RT); }
template <typename T, int TN, int RT, int TM>
__global__ __launch_bounds__(RT) void split_reduce(ReduceParams p) {
  constexpr int TPR = TN / 8;      // threads per row
  constexpr int RPW = RT / TPR;    // rows per workgroup
  constexpr int WPT = TM / RPW;    // workgroups per split tile
  static_assert(RT % TPR == 0 && WPT == reduce_blocks_per_tile<TN, RT, TM>(), "whole rows per workgroup");
  const int st = blockIdx.x / WPT;      // split tile (0 .. tiles-1)
  int tm, tn;
  tile_of_task(p.full_tasks + st, p.tiles_m, p.tiles_n, p.group_m, &tm, &tn);
  const int r = (blockIdx.x % WPT) * RPW + (int)threadIdx.x / TPR;
  const int c = ((int)threadIdx.x % TPR) * 8;
  const int row = tm * TM + r;
  const int col = tn * TN + c;
  if (row >= p.M || col >= p.N) return;
  const float* w = p.ws + (size_t)st * (TM * TN) + (size_t)r * TN + c;
  const size_t stride = (size_t)p.tiles * (TM * TN);  // between the partials of two splits
  float s[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = 0.0f;
  // U splits' loads in flight at once, then added in split order: 16 for the
  // few one-wave workgroups, 8 (half the registers, so more waves per SIMD)
  // for the wide launches
  constexpr int U = RT == 64 ? 16 : 8;
  for (int k0 = 0; k0 < p.splits; k0 += U) {
    float4 a[U], b[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (k0 + u < p.splits) {
        a[u] = *(const float4*)(w + (k0 + u) * stride);
        b[u] = *(const float4*)(w + (k0 + u) * stride + 4);
      } else {
        a[u] = b[u] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (k0 + u < p.splits) {
        s[0] += a[u].x; s[1] += a[u].y; s[2] += a[u].z; s[3] += a[u].w;
        s[4] += b[u].x; s[5] += b[u].y; s[6] += b[u].z; s[7] += b[u].w;
      }
    }
  }
  u32x4 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = pack2<T>(s[2 * e], s[2 * e + 1]);
  uint16_t* dst = p.D + (int64_t)row * p.ldd + col;
  if (p.d_vec && col + 8 <= p.N) {
    __builtin_nontemporal_store(v, (u32x4*)dst);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (col + e < p.N) dst[e] = (uint16_t)(v[e >> 1] >> ((e & 1) * 16));
  }
}

// The reduction's launch on `stream`, after the partial tiles' kernel on
// the same stream (one-wave workgroups where 256-thread ones would not
// cover the CUs).
template <typename T, int TN, int TM>
static inline void enqueue_split_reduce(const ReduceParams& r, int cus, hipStream_t stream) {
  const int64_t wide = r.tiles * (int64_t)reduce_blocks_per_tile<TN, 256, TM>();
  if (wide < cus)
    hipLaunchKernelGGL((split_reduce<T, TN, 64, TM>),
                       dim3((unsigned)(r.tiles * reduce_blocks_per_tile<TN, 64, TM>())), dim3(64), 0,
                       stream, r);
  else
    hipLaunchKernelGGL((split_reduce<T, TN, 256, TM>), dim3((unsigned)wide), dim3(256), 0, stream, r);
}

}  // namespace dg
