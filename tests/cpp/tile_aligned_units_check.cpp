// Host-side check of ubx::tile_aligned_units (the device-side chunk loop's tile cut):
// every row of [lo, hi) in exactly one tile, tiles aligned to the cut, tiles listed in
// the units' order by the unit holding their last row, and the tile count of row_tiles.
#include <cstdio>
#include <cstdlib>
#include <vector>
#include <algorithm>
#include "ub_internal.h"
using namespace ubx;
int main() {
  srand(1);
  long checks = 0;
  for (int it = 0; it < 200000; ++it) {
    int n = 1 + rand() % 12;
    GemmUnits u; u.n = n;
    int lo = rand() % 50, r = lo;
    std::vector<int> sizes(n);
    for (int i = 0; i < n; ++i) sizes[i] = 1 + rand() % 700;
    std::vector<int> perm(n); for (int i = 0; i < n; ++i) perm[i] = i;
    std::random_shuffle(perm.begin(), perm.end());
    std::vector<int> r0(n);
    for (int i = 0; i < n; ++i) { r0[i] = r; r += sizes[i]; }
    int hi = r;
    for (int i = 0; i < n; ++i) { u.row0[i] = r0[perm[i]]; u.rows[i] = sizes[perm[i]]; }
    int bm = (int[]){128, 256, 320}[rand() % 3];
    GemmUnits s = tile_aligned_units(u, bm);
    std::vector<int> cover(hi, 0);
    int prev_unit_pos = -1;
    for (int k = 0; k < s.n; ++k) {
      int a = s.row0[k], b = s.row0[k] + s.rows[k];
      if (a < lo || b > hi || s.rows[k] <= 0) { printf("FAIL range\n"); return 1; }
      if ((a - lo) % bm != 0) { printf("FAIL align\n"); return 1; }
      for (int t = a; t < b; t += bm) {
        int last = std::min(b, t + bm) - 1;
        // unit holding the last row: must be this segment's unit, in plan order
        int pos = -1;
        for (int i = 0; i < n; ++i) if (last >= u.row0[i] && last < u.row0[i] + u.rows[i]) pos = i;
        if (pos < prev_unit_pos) { printf("FAIL order\n"); return 1; }
        prev_unit_pos = pos;
        if (std::min(b, t + bm) != std::min(hi, t + bm)) { printf("FAIL tile end\n"); return 1; }
      }
      for (int x = a; x < b; ++x) cover[x]++;
    }
    for (int x = lo; x < hi; ++x) if (cover[x] != 1) { printf("FAIL cover %d\n", x); return 1; }
    if (row_tiles(u, bm) != (hi - lo + bm - 1) / bm) { printf("FAIL count\n"); return 1; }
    ++checks;
  }
  // non-contiguous units are returned unchanged
  GemmUnits g; g.n = 2; g.row0[0] = 0; g.rows[0] = 100; g.row0[1] = 200; g.rows[1] = 50;
  GemmUnits s = tile_aligned_units(g, 128);
  if (s.n != 2 || s.row0[1] != 200 || s.rows[1] != 50) { printf("FAIL gap\n"); return 1; }
  printf("ok: %ld layouts\n", checks);
  return 0;
}
