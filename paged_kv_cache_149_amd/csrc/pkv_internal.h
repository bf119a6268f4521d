// Internal declarations shared by the planner and the kernel launchers.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "pkv.h"

namespace pkv {

constexpr int kBlock = 16;       // tokens per paged block
constexpr int kHeadDim = 128;    // supported head dimension
constexpr int kTileCols = 16;    // MFMA columns of a narrow tile
constexpr int kWideCols = 256;   // columns (positions x heads) of a wide tile
constexpr int kWideWaves = 8;    // wavefronts of a wide-tile workgroup (32 columns each)
constexpr int kChunkKeys = 32;   // keys per inner-loop step (two blocks)
constexpr size_t kAlign = 256;

// One attention work item (PKV_ITEM_INTS int32 in the workspace).
struct Item {
  int32_t seq;   // sequence index (block-table row)
  int32_t kvh;   // kv head
  int32_t t0;    // first packed row of the tile
  int32_t np;    // query positions in the tile
  int32_t pos0;  // position of row t0
  int32_t k0;    // first key (multiple of kChunkKeys)
  int32_t k1;    // one past the last key
  int32_t part;  // partial-result column base, or -1 for a direct write
};
static_assert(sizeof(Item) == PKV_ITEM_INTS * 4, "item size");

// One merge entry: an output (row, head) whose keys were split.
struct Merge {
  int32_t out_row;  // t * Hq + h
  int32_t first;    // partial column of split 0
  int32_t nsplit;   // number of splits
  int32_t stride;   // column distance between consecutive splits
};
static_assert(sizeof(Merge) == PKV_MERGE_INTS * 4, "merge size");

inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Role of row rho (eight consecutive workgroups, one per XCD) of a launch
// with wide tiles: narrow_rows of the rows, spread evenly over all of them,
// first walk narrow wavefront shares (ord = their narrow row); ord of a wide
// row counts the wide rows.  Shared by the planner and the kernel.
struct RowRole {
  bool narrow;
  int ord;
};
constexpr RowRole mixed_row(int rows, int narrow_rows, int rho) {
  const int lo = rho * narrow_rows / rows, hi = (rho + 1) * narrow_rows / rows;
  return RowRole{hi > lo, hi > lo ? lo : rho - lo};
}

inline int log2_exact(int x) {
  int l = 0;
  while ((1 << l) < x) ++l;
  return (1 << l) == x ? l : -1;
}

}  // namespace pkv
