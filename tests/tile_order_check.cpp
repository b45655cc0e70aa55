// Host build of the GEMM kernels' tile order (csrc/tile_order.h): every
// workgroup of every launch mode is enumerated for many shapes, and the
// tiles, unit ranges and tile coordinates it reaches are checked to be in
// bounds and to cover each output tile (and each K unit of a split tile)
// exactly once.  Exit status 0 when every check holds.
#include <cstdio>
#include <vector>

#include "tile_order.h"

using namespace qact;

static int fails = 0;
#define CHECK(c, ...)                    \
  do {                                   \
    if (!(c)) {                          \
      if (fails < 20) {                  \
        std::printf("FAIL " __VA_ARGS__); \
        std::printf("\n");               \
      }                                  \
      ++fails;                           \
    }                                    \
  } while (0)

static void check(int mt, int nt, int units, int cus, int max_splits, int min_saved, int group_m) {
  const int total = mt * nt;
  const SplitPlan p = plan_split(total, units, cus, max_splits, min_saved);
  CHECK(p.main_tiles + p.tail == total, "plan tiles %d %d", mt, nt);
  CHECK(p.splits >= 1 && p.split_units >= 1, "plan slices");
  CHECK((long)p.splits * p.split_units >= units && (long)(p.splits - 1) * p.split_units < units,
        "slices cover units without an empty one: mt %d nt %d units %d", mt, nt, units);
  if (p.tail) {
    CHECK(p.splits >= 2 && p.split_units >= 2 && p.tail * p.splits <= cus, "split shape");
  } else {
    CHECK(p.splits == 1 && p.split_units == units, "unsplit plan");
  }
  std::vector<int> seen(total, 0);
  // whole tiles
  const int grid_main = 8 * ((p.main_tiles + 7) / 8);
  for (int b = 0; b < grid_main; ++b) {
    TileWork w;
    if (!tile_work(kWhole, b, p.main_tiles, p.splits, p.split_units, units, w)) continue;
    CHECK(w.logical >= 0 && w.logical < p.main_tiles, "whole tile %d of %d", w.logical, p.main_tiles);
    CHECK(w.u_begin == 0 && w.u_count == units, "whole units");
    if (w.logical >= 0 && w.logical < total) ++seen[w.logical];
  }
  // K slices of the tail tiles
  std::vector<int> unit_seen((size_t)p.tail * units, 0);
  if (p.tail) {
    for (int b = 0; b < p.tail * p.splits; ++b) {
      TileWork w;
      CHECK(tile_work(kSlice, b, p.main_tiles, p.splits, p.split_units, units, w), "slice live");
      const int t = w.logical - p.main_tiles;
      CHECK(t >= 0 && t < p.tail, "slice tile %d", t);
      CHECK(w.u_count >= 1 && w.u_begin >= 0 && w.u_begin + w.u_count <= units, "slice units %d+%d of %d",
            w.u_begin, w.u_count, units);
      if (t >= 0 && t < p.tail)
        for (int u = w.u_begin; u < w.u_begin + w.u_count && u < units; ++u)
          ++unit_seen[(size_t)t * units + u];
    }
    for (size_t i = 0; i < unit_seen.size(); ++i) CHECK(unit_seen[i] == 1, "unit covered once");
    for (int b = 0; b < p.tail; ++b) {
      TileWork w;
      tile_work(kFixup, b, p.main_tiles, p.splits, p.split_units, units, w);
      CHECK(w.logical >= p.main_tiles && w.logical < total, "fixup tile");
      if (w.logical >= 0 && w.logical < total) ++seen[w.logical];
    }
  }
  for (int i = 0; i < total; ++i) CHECK(seen[i] == 1, "logical tile %d computed %d times", i, seen[i]);
  // coordinates
  std::vector<int> cell(total, 0);
  for (int l = 0; l < total; ++l) {
    int tm, tn;
    tile_coords(l, mt, nt, group_m, tm, tn);
    CHECK(tm >= 0 && tm < mt && tn >= 0 && tn < nt, "coords %d,%d of %d,%d", tm, tn, mt, nt);
    if (tm >= 0 && tm < mt && tn >= 0 && tn < nt) ++cell[tm * nt + tn];
  }
  for (int i = 0; i < total; ++i) CHECK(cell[i] == 1, "output tile %d reached %d times", i, cell[i]);
}

int main() {
  long cases = 0;
  const int units_list[] = {1, 2, 3, 30, 48, 120, 192};
  for (int group_m : {4, 8, 16})
    for (int min_saved : {24, 40})
      for (int units : units_list)
        for (int mt = 1; mt <= 72; ++mt)
          for (int nt = 1; nt <= 48; ++nt) {
            check(mt, nt, units, 256, 4, min_saved, group_m);
            ++cases;
          }
  // the CogVideoX linears at 17776 tokens: 70 tile rows; 128- and
  // 256-column tiles; K = 1920, 3072, 7680, 12288 in units of 64
  const int nts[] = {45, 15, 60, 23, 8, 30, 72, 24, 96, 36, 12, 48};
  for (int nt : nts)
    for (int units : {30, 48, 120, 192})
      for (int min_saved : {24, 40}) {
        check(70, nt, units, 256, 4, min_saved, 8);
        ++cases;
      }
  std::printf("%ld shapes, %d failures\n", cases, fails);
  return fails ? 1 : 0;
}
