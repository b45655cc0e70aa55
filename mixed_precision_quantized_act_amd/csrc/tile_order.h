// Order of a GEMM's output tiles and the K split of its last round, shared
// by the GEMM kernels (device), their launch code (host) and a host-side
// test that enumerates every workgroup of a launch.
#pragma once

#include <stdint.h>

#if defined(__HIP__)
#define QACT_HD __host__ __device__
#else
#define QACT_HD
#endif

namespace qact {

// `total` tiles run in rounds of `cus` workgroups (one per CU).  A last
// round at most half full is split along K: its `tail` tiles into `splits`
// slices of `split_units` units (at most max_splits, at least 2 units each,
// no empty slice), when that takes at least min_saved units off the round.
struct SplitPlan {
  int main_tiles, tail, splits, split_units;
};
QACT_HD inline SplitPlan plan_split(int total, int units, int cus, int max_splits, int min_saved) {
  SplitPlan p = {total, 0, 1, units};
  const int tail = total % cus;
  if (tail == 0 || 2 * tail > cus) return p;
  int s = cus / tail;
  if (s > max_splits) s = max_splits;
  if (s > units / 2) s = units / 2;
  if (s < 2 || units * (s - 1) / s < min_saved) return p;
  p.main_tiles = total - tail;
  p.tail = tail;
  p.split_units = (units + s - 1) / s;
  p.splits = (units + p.split_units - 1) / p.split_units;
  return p;
}

// Launch modes: whole tiles (grid 8 ceil(main_tiles / 8)), the K slices of
// the tail tiles (grid tail * splits) and their fixup (workgroup bid: tail
// tile bid; the fp16 kernel launches four workgroups per tail tile and
// passes bid / 4).
enum { kWhole = 0, kSlice = 1, kFixup = 2 };

// Workgroup bid of a launch in `mode`: its logical tile and the units it
// computes; false for a whole-tile workgroup past the last tile.  Whole
// tiles give each of the 8 XCDs (workgroups are dealt to XCDs round-robin)
// a contiguous range of logical tiles.
struct TileWork {
  int logical, slice, u_begin, u_count;
};
QACT_HD inline bool tile_work(int mode, int bid, int main_tiles, int splits, int split_units,
                              int units, TileWork& w) {
  w.slice = 0;
  w.u_begin = 0;
  w.u_count = units;
  if (mode == kWhole) {
    const int per_xcd = (main_tiles + 7) / 8;
    w.logical = (bid & 7) * per_xcd + (bid >> 3);
    return w.logical < main_tiles;
  }
  if (mode == kSlice) {
    w.logical = main_tiles + bid / splits;
    w.slice = bid % splits;
    w.u_begin = w.slice * split_units;
    w.u_count = units - w.u_begin < split_units ? units - w.u_begin : split_units;
    return true;
  }
  w.logical = main_tiles + bid;
  return true;
}

// Logical tile -> (tile row tm, tile column tn): groups of `group_m` tile
// rows, each walked column by column, so that consecutive tiles share
// their weight columns and a group's activation rows stay in L2.
QACT_HD inline void tile_coords(int logical, int mt, int nt, int group_m, int& tm, int& tn) {
  const int group = logical / (group_m * nt);
  const int first_m = group * group_m;
  const int gsz = mt - first_m < group_m ? mt - first_m : group_m;
  const int in_group = logical - group * group_m * nt;
  tm = first_m + in_group % gsz;
  tn = in_group / gsz;
}

}  // namespace qact
