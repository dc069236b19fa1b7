// Host-side check of ubx::tile_of (workgroup -> tile of the device-side chunk loop) for
// several group sizes: over a grid of one workgroup per tile every tile (row tile of every
// unit x tile column) is taken by exactly one workgroup, and the rows a tile reports are
// inside its unit.
#include <cstdio>
#include <cstdlib>
#include <algorithm>
#include <vector>

#include "gemm_common.h"
#include "ub_internal.h"

using namespace ubx;

struct P {
  int32_t tiles_n, group, n_units;
  int32_t unit_row0[kMaxGemmUnits], unit_rows[kMaxGemmUnits], unit_tile0[kMaxGemmUnits + 1];
};

int main() {
  srand(3);
  long checks = 0;
  for (int it = 0; it < 20000; ++it) {
    P p{};
    const int bm = (int[]){128, 256, 320}[rand() % 3];
    p.group = (int[]){1, 2, 4, 8}[rand() % 4];
    p.tiles_n = 1 + rand() % 40;
    p.n_units = 1 + rand() % 64;
    int row = rand() % 1000, tiles = 0;
    std::vector<int> rt0;  // first row tile of each unit
    for (int u = 0; u < p.n_units; ++u) {
      p.unit_row0[u] = row;
      p.unit_rows[u] = 1 + rand() % (rand() % 4 == 0 ? 5000 : 600);
      row += p.unit_rows[u] + rand() % 3;  // units need not be adjacent here
      p.unit_tile0[u] = tiles;
      rt0.push_back(tiles / p.tiles_n);
      tiles += ((p.unit_rows[u] + bm - 1) / bm) * p.tiles_n;
    }
    p.unit_tile0[p.n_units] = tiles;
    const int R = tiles / p.tiles_n;
    const int64_t grid = tiles;
    std::vector<int> seen((size_t)tiles, 0);
    for (int wg = 0; wg < grid; ++wg) {
      int m0, m_end, tn;
      if (!tile_of(p, wg, bm, m0, m_end, tn)) continue;
      int u = -1;
      for (int k = 0; k < p.n_units; ++k)
        if (m0 >= p.unit_row0[k] && m0 < p.unit_row0[k] + p.unit_rows[k]) u = k;
      if (u < 0 || m_end != p.unit_row0[u] + p.unit_rows[u] || (m0 - p.unit_row0[u]) % bm) {
        printf("FAIL rows wg=%d\n", wg);
        return 1;
      }
      if (tn < 0 || tn >= p.tiles_n) { printf("FAIL column\n"); return 1; }
      const int row_tile = rt0[u] + (m0 - p.unit_row0[u]) / bm;
      seen[(size_t)row_tile * p.tiles_n + tn]++;
    }
    for (int t = 0; t < tiles; ++t)
      if (seen[t] != 1) { printf("FAIL tile %d seen %d times\n", t, seen[t]); return 1; }
    ++checks;
  }
  printf("ok: %ld layouts\n", checks);
  return 0;
}
