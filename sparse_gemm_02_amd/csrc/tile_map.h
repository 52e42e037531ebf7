// Block -> output tile mapping shared by the tiled GEMM kernels.
#pragma once
#include "common.h"

namespace slope {

// MI355X dispatches consecutive workgroups round-robin over its 8 XCDs, each
// with a private L2.  Renumber so that the workgroups resident on one XCD at
// the same time get consecutive logical ids, then walk the logical ids in
// groups of `group` row tiles so that those workgroups share operand tiles.
__device__ __forceinline__ void tile_of_block(int bid, int nblocks, int tiles_r, int tiles_c, int group,
                                              int& tr, int& tc) {
  constexpr int kXcds = 8;
  int logical = bid;
  if (nblocks % kXcds == 0) logical = (bid % kXcds) * (nblocks / kXcds) + bid / kXcds;
  const int per_group = group * tiles_c;
  const int g = logical / per_group;
  const int first = g * group;
  const int gsize = (tiles_r - first) < group ? (tiles_r - first) : group;
  const int in_group = logical - g * per_group;
  tr = first + in_group % gsize;
  tc = in_group / gsize;
}

}  // namespace slope
