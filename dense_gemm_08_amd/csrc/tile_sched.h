// tile_sched.h -- the persistent workgroup tile scheduler (host and device).
//
// Tile order.  TileFoundry's schedule tutorial, section 3 ("Group 16 M
// tiles"), splits the M tile index into a group and an index inside the
// group, with the N index between them, so that consecutive work shares B
// tiles in L2; section 5 decodes a flat task index the same way (group,
// then N tile, then M tile inside the group).  Here the last group may be
// shorter than group_m when the tile rows do not divide evenly; that case is
// not on the page (every page shape divides), and the plainest reading is to
// walk the leftover rows the same way.
//
// XCD remap.  The MI355X has 8 XCDs, each with its own L2, and consecutive
// workgroups of a launch are dealt to XCDs round-robin.  xcd_slot() gives the
// workgroups of one XCD a contiguous run of task slots, so tiles that are
// adjacent in the grouped order (and share A or B tiles) also share an L2.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define DG_HD __host__ __device__
#else
#define DG_HD
#endif

namespace dg {

// Task index -> (tile row, tile column) in the grouped order.
DG_HD inline void tile_of_task(int task, int tiles_m, int tiles_n, int group_m, int* tm, int* tn) {
  const int per_group = group_m * tiles_n;
  const int g = task / per_group;
  const int first_m = g * group_m;
  const int rows_left = tiles_m - first_m;
  const int gsize = rows_left < group_m ? rows_left : group_m;
  const int local = task - g * per_group;
  *tm = first_m + local % gsize;
  *tn = local / gsize;
}

// Workgroup b of a grid of `grid` -> its slot in the task order, such that the
// workgroups on one XCD (b mod num_xcds equal) hold consecutive slots.
DG_HD inline int xcd_slot(int b, int grid, int num_xcds) {
  const int xcd = b % num_xcds;
  const int local = b / num_xcds;
  const int full = grid / num_xcds;
  const int rem = grid % num_xcds;
  return xcd < rem ? xcd * (full + 1) + local : rem * (full + 1) + (xcd - rem) * full + local;
}

}  // namespace dg
