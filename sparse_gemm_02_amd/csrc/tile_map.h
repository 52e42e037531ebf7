// Block -> output tile mapping shared by the tiled GEMM kernels.
#pragma once
#include "common.h"

namespace slope {

// Logical tile id -> (row tile, column tile): groups of `group` row tiles, all
// column tiles of a group before the next, row tiles fastest within a group,
// so that consecutive logical ids share operand tiles.
__device__ __forceinline__ void logical_tile(int logical, int tiles_r, int tiles_c, int group, int& tr, int& tc) {
  const int per_group = group * tiles_c;
  const int g = logical / per_group;
  const int first = g * group;
  const int gsize = (tiles_r - first) < group ? (tiles_r - first) : group;
  const int in_group = logical - g * per_group;
  tr = first + in_group % gsize;
  tc = in_group / gsize;
}

// MI355X dispatches consecutive workgroups round-robin over its 8 XCDs, each
// with a private L2.  Renumber so that the workgroups resident on one XCD at
// the same time get consecutive logical ids, then map those to tiles.
__device__ __forceinline__ void tile_of_block(int bid, int nblocks, int tiles_r, int tiles_c, int group,
                                              int& tr, int& tc) {
  constexpr int kXcds = 8;
  int logical = bid;
  if (nblocks % kXcds == 0) logical = (bid % kXcds) * (nblocks / kXcds) + bid / kXcds;
  logical_tile(logical, tiles_r, tiles_c, group, tr, tc);
}

// Host side: how many row tiles of a product to run in full tiles when the
// remaining rows take half tiles (cols_half blocks per row, each costing
// about 0.65 of a full tile, measured on the OPT-66B shapes), so that a
// launch whose full-tile grid would end in a partly filled round of blocks
// finishes sooner.  Minimises the estimated time in rounds of `cus` blocks
// over all-half and the last 4 * cus rows (more half rows than that only pay
// when every row does, as for a single column tile); ties keep more full rows.
inline int64_t full_width_rows(int64_t tiles_r, int64_t cols_full, int64_t cols_half, int64_t cus) {
  auto rounds = [cus](int64_t blocks) { return (blocks + cus - 1) / cus; };
  auto cost = [&](int64_t rows) { return 100 * rounds(rows * cols_full) + 65 * rounds((tiles_r - rows) * cols_half); };
  int64_t best_rows = tiles_r, best_cost = cost(tiles_r);
  const int64_t lowest = tiles_r > 4 * cus ? tiles_r - 4 * cus : 0;
  for (int64_t rows = tiles_r - 1; rows >= lowest; --rows) {
    if (cost(rows) < best_cost) {
      best_cost = cost(rows);
      best_rows = rows;
    }
  }
  if (cost(0) < best_cost) best_rows = 0;
  return best_rows;
}

}  // namespace slope
