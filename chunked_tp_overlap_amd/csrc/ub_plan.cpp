// Chunk plan of one overlapped GEMM call.
//
// From "How to setup TP Overlap configs" (Transformer Engine issue 1344), option list:
//   - ring exchange ignores num_splits and cuts the GEMM into tp_size chunks; pipeline
//     and bulk cut it into num_splits chunks;
//   - the chunks run on min(num_splits, num_max_streams) compute streams;
//   - aggregate merges two chunks per launch when the all-gather is overlapped.
// From "[Feature Request] Support dynamic token counts in TP communication/GEMM overlap"
// (Transformer Engine issue 3564), "Implementation approach in the prototype": chunk
// views and offsets come from the active first dimension T, never from the capacity.
//
// Choices the pages leave open: chunk c covers rows [floor(cT/n), floor((c+1)T/n));
// aggregate pairs chunks {2u, 2u+1} (a trailing odd chunk stays alone); ring all-gather
// step i runs unit (rank/agg - i) mod U, i.e. a rank starts on its own chunk and then
// takes the chunks arriving from its left neighbour; ring reduce-scatter step i runs
// chunk (rank + 1 + i) mod U, so a rank's own shard is completed last; pipeline and bulk
// run units in natural order; execution position j uses compute stream j mod S.
#include <algorithm>

#include "ub_internal.h"

namespace ubx {

ub_status_t build_plan(int64_t T, int32_t tp, const ub_overlap_cfg_t& cfg, ub_op_t op,
                       Plan* out, std::string* err) {
  if (cfg.method != UB_RING_EXCHANGE && cfg.method != UB_PIPELINE && cfg.method != UB_BULK) {
    *err = "unknown overlap method " + std::to_string(cfg.method);
    return UB_ERR_INVALID_ARG;
  }
  if (op != UB_OP_AG && op != UB_OP_RS) {
    *err = "unknown op " + std::to_string(static_cast<int>(op));
    return UB_ERR_INVALID_ARG;
  }
  if (cfg.num_splits < 1) {
    *err = "num_splits must be >= 1, got " + std::to_string(cfg.num_splits);
    return UB_ERR_INVALID_ARG;
  }
  if (cfg.num_max_streams < 1) {
    *err = "num_max_streams must be >= 1, got " + std::to_string(cfg.num_max_streams);
    return UB_ERR_INVALID_ARG;
  }
  if (cfg.rank < 0 || cfg.rank >= tp) {
    *err = "rank must be in [0, tp_size), got " + std::to_string(cfg.rank);
    return UB_ERR_INVALID_ARG;
  }
  const int32_t n = (cfg.method == UB_RING_EXCHANGE) ? tp : cfg.num_splits;
  const int32_t agg = (cfg.aggregate && op == UB_OP_AG) ? 2 : 1;
  const int32_t U = (n + agg - 1) / agg;
  const int32_t S = std::min(std::min(n, cfg.num_max_streams), static_cast<int32_t>(UB_MAX_STREAMS));

  auto chunk_start = [&](int64_t c) { return (c * T) / n; };  // floor(c T / n), from active T

  out->units.clear();
  out->units.reserve(static_cast<size_t>(U));
  out->n_chunks = n;
  out->n_streams = S;
  for (int32_t j = 0; j < U; ++j) {
    int32_t u;
    if (cfg.method == UB_RING_EXCHANGE && op == UB_OP_AG) {
      const int32_t home = cfg.rank / agg;
      u = ((home - j) % U + U) % U;
    } else if (cfg.method == UB_RING_EXCHANGE) {
      u = (cfg.rank + 1 + j) % U;
    } else {
      u = j;
    }
    const int64_t first = static_cast<int64_t>(u) * agg;
    const int64_t last = std::min<int64_t>(first + agg, n);  // one past the unit's last chunk
    ub_plan_unit_t pu{};
    pu.pos = j;
    pu.unit = u;
    pu.row0 = chunk_start(first);
    pu.row1 = chunk_start(last);
    pu.stream = j % S;
    out->units.push_back(pu);
  }
  return UB_OK;
}

}  // namespace ubx

namespace ubx {

namespace {

// Whether the units tile one contiguous row range [*lo, *hi) without gaps or overlaps.
bool contiguous(const GemmUnits& u, int64_t* lo, int64_t* hi) {
  if (u.n <= 0) return false;
  int32_t order[kMaxGemmUnits];
  for (int i = 0; i < u.n; ++i) order[i] = i;
  std::sort(order, order + u.n, [&](int32_t a, int32_t b) { return u.row0[a] < u.row0[b]; });
  int64_t end = u.row0[order[0]];
  *lo = end;
  for (int i = 0; i < u.n; ++i) {
    const int k = order[i];
    if (u.rows[k] <= 0 || u.row0[k] != end) return false;
    end += u.rows[k];
  }
  *hi = end;
  return true;
}

}  // namespace

bool contiguous_rows(const GemmUnits& u, int64_t* lo, int64_t* hi) { return contiguous(u, lo, hi); }

GemmUnits tile_aligned_units(const GemmUnits& u, int bm) {
  int64_t lo = 0, hi = 0;
  if (u.n <= 1 || bm <= 0 || !contiguous(u, &lo, &hi)) return u;
  const int64_t nt = (hi - lo + bm - 1) / bm;
  GemmUnits out;
  out.n = 0;
  for (int i = 0; i < u.n; ++i) {
    // tiles t whose last row min(hi, lo + (t+1) bm) - 1 lies in [row0, row0 + rows)
    const int64_t r0 = u.row0[i], r1 = u.row0[i] + u.rows[i];
    int64_t t0 = (r0 - lo + 1 + bm - 1) / bm - 1;  // smallest t with lo + (t+1) bm - 1 >= r0
    if (t0 < 0) t0 = 0;
    int64_t t1 = (r1 - lo) / bm - 1;                // largest t with lo + (t+1) bm - 1 < r1
    if (r1 == hi) t1 = nt - 1;                      // the last tile ends at hi
    if (t1 < t0) continue;
    out.row0[out.n] = static_cast<int32_t>(lo + t0 * bm);
    out.rows[out.n] = static_cast<int32_t>(std::min(hi, lo + (t1 + 1) * bm) - (lo + t0 * bm));
    ++out.n;
  }
  return out;
}

int64_t row_tiles(const GemmUnits& u, int bm) {
  const GemmUnits a = tile_aligned_units(u, bm);
  int64_t n = 0;
  for (int i = 0; i < a.n; ++i) n += (a.rows[i] + bm - 1) / bm;
  return n;
}

int64_t fuse_counter_stream_words(int64_t capacity, int64_t n) {
  // One launch over up to `capacity` rows: re-cutting a unit at tile boundaries adds at
  // most one row tile, and no tile is smaller than 128 x 128.
  return ((capacity + 127) / 128 + 1) * ((n + 127) / 128);
}

int64_t fuse_counter_words(int64_t capacity, int64_t n) {
  const int64_t streams = UB_MAX_STREAMS * fuse_counter_stream_words(capacity, n);
  const int64_t device_loop = ((capacity + 127) / 128 + kMaxGemmUnits) * ((n + 127) / 128);
  return std::max(streams, device_loop);
}

}  // namespace ubx
