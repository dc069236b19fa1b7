// Host-side check of ubx::choose_segmentation (K segmentation of the all-gather GEMM) over
// the workloads' shapes and random ones: the answer is deterministic; no segmentation for
// batched launches or short K; a segmentation has a segment count from the priced set, at
// most one segment per 32-deep k-step, a first segmented row inside [0, T) on a 64-row
// boundary, a tile the library builds, and partials within the 64 MiB the scratch sizing
// promises.
#include <cstdio>
#include <cstdlib>

#include "ub_internal.h"

using namespace ubx;

static int fails = 0;
#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      std::printf("FAIL %s:%d %s\n", __FILE__, __LINE__, #c);       \
      if (++fails > 20) return 1;                                  \
    }                                                              \
  } while (0)

int main() {
  srand(11);
  long checks = 0, segmented = 0;
  const long shapes[][2] = {{1280, 8192}, {1536, 4096}, {3584, 4096}, {4096, 1792}};
  for (int it = 0; it < 6000; ++it) {
    long n, k, T;
    if (it < 4 * 300) {
      n = shapes[it % 4][0];
      k = shapes[it % 4][1];
      T = 8 * (1 + (it / 4) * 14);
    } else {
      n = 8 * (1 + rand() % 1024);
      k = 8 * (1 + rand() % 2048);
      T = 1 + rand() % 40000;
    }
    const SegPlan a = choose_segmentation(T, n, k, 1);
    const SegPlan b = choose_segmentation(T, n, k, 1);
    CHECK(a.seg_row == b.seg_row && a.nseg == b.nseg && a.tile_m == b.tile_m && a.tile_n == b.tile_n);
    const SegPlan batched = choose_segmentation(T, n, k, 8);
    CHECK(batched.nseg <= 1);
    const long nk = (k + 31) / 32;
    if (a.nseg > 1) {
      ++segmented;
      CHECK(a.nseg == 2 || a.nseg == 3 || a.nseg == 4 || a.nseg == 6 || a.nseg == 8 ||
            a.nseg == 12 || a.nseg == 16);
      CHECK(a.nseg <= nk && nk >= 4);
      CHECK(a.seg_row >= 0 && a.seg_row < T && a.seg_row % 64 == 0);
      CHECK(gemm_bf16_tile_supported(a.tile_m, a.tile_n));
      CHECK(a.reduce == 2);
      const long tiles = ((T - a.seg_row + a.tile_m - 1) / a.tile_m) * ((n + a.tile_n - 1) / a.tile_n);
      CHECK(tiles * a.nseg * a.tile_m * a.tile_n * 4 <= (64L << 20));
    } else {
      CHECK(a.nseg == 1 && a.seg_row == -1);
    }
    ++checks;
  }
  std::printf("ok %ld %ld\n", checks, segmented);
  return fails ? 1 : 0;
}
