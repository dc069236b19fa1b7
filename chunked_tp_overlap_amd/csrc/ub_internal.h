// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>
#include <vector>

#include "ub.h"

namespace ubx {

// Kernel timing hook.  While a timed call runs (timed_launch in ub_api.cpp) this is the
// call's stop event, and every kernel the library launches in it records the event at its
// own end: hipExtLaunchKernel's stop event uses the dispatch's completion timestamp, where a
// separate hipEventRecord adds a marker packet of its own (~3 us of GPU time per record,
// measured on a back-to-back sweep).  Launches in order on the call's stream, so the event
// ends with the call's last kernel.  nullptr: no call is timed on this thread.
inline thread_local hipEvent_t g_launch_stop = nullptr;
inline thread_local bool g_launch_stop_used = false;

template <class T>
struct same_type { using type = T; };

// Every kernel launch of the library.
template <class... KA>
hipError_t launch_k(void (*kernel)(KA...), dim3 grid, dim3 block, size_t shmem, hipStream_t s,
                    typename same_type<KA>::type... args) {
  void* argv[sizeof...(KA) > 0 ? sizeof...(KA) : 1] = {(void*)&args...};
  const hipError_t e = hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block,
                                          argv, shmem, s, nullptr, g_launch_stop, 0);
  if (g_launch_stop && e == hipSuccess) g_launch_stop_used = true;
  return e;
}


// ---- chunk plan (host only; ub_plan.cpp) ------------------------------------------------
struct Plan {
  std::vector<ub_plan_unit_t> units;  // in execution order
  int32_t n_chunks = 0;               // chunks before aggregation
  int32_t n_streams = 0;              // compute streams used (stream 0 = caller's)
};

// Validates cfg (method, num_splits, num_max_streams, rank) and builds the plan for an
// active T.  Returns UB_OK or UB_ERR_INVALID_ARG with a message in *err.
ub_status_t build_plan(int64_t T, int32_t tp, const ub_overlap_cfg_t& cfg, ub_op_t op,
                       Plan* out, std::string* err);

// ---- kernels (gemm_bf16.hip, reduce_partials.hip) ----------------------------------------
// Batched row-major bf16 GEMM, C[b] = bf16(A[b] * B[b]) with fp32 accumulation.
// All strides in elements.  Requirements checked by the caller: k % 8 == 0,
// n % 8 == 0, lda/ldb/ldc % 8 == 0, pointers 16-byte aligned.
constexpr int kMaxGemmUnits = 64;

// Arrival flags of the device-side chunk loop: kReadySlots slots of kReadyWords words, one
// slot per handle that gates on arrivals (words 0..63: the chunks' flags; word 64: a count
// of waits that timed out).  ready_flags_base() is the device address of slot 0 on the
// current device (nullptr and *err set on failure).
constexpr int kReadySlots = 64;
constexpr int kReadyWords = 72;
constexpr int kReadyTimeoutWord = 64;
uint32_t* ready_flags_base(hipError_t* err);

// Per-handle debug and tuning settings (ub_debug_set).  All zero: the library's own
// choices.  Nothing else (no environment variable) changes what a launch does.
struct DebugOpts {
  int32_t tile_m = 0, tile_n = 0;  // force one tile shape (one launch, unless cut_row)
  int64_t cut_row = 0;             // > 0: cut a launch group's rows there (see ub_debug_set)
  int32_t tail_m = 0, tail_n = 0;  // tile of the second launch of a forced cut
  int32_t tile_group = 0;          // force the row-tile group size of the workgroup map
  int64_t seg_row = -1;            // >= 0: force K segmentation from this row (with nseg)
  int32_t nseg = 0;                // forced segment count (>= 2 with seg_row >= 0)
  int32_t seg_m = 0, seg_n = 0;    // tile of forced split pieces (0: the library's choice)
  int32_t seg_reduce = 0;          // forced split sum: 1 in the kernel, 2 a separate launch
  int32_t rs_pieces = 0;           // device-side reduce-scatter row pieces (0: the library's)
  int64_t arrival_wait_us = 0;     // bound of a gated tile's wait (0: ~0.5 s)
  int32_t arrival_drop_flags = 0;  // write no flag after delivered chunks
};

// The tile plan the last GEMM launch group took (ub_debug_last_plan).
struct TilePlanRecord {
  int32_t tile_m = 0, tile_n = 0;
  int64_t cut = -1;
  int32_t tail_m = 0, tail_n = 0;
  int64_t seg_row = -1;  // first K-segmented row of the launch group, or -1
  int32_t nseg = 0;
  int32_t split = 0;     // the segments ran as separate workgroups (split-K), summed in the
                         // kernel (1) or by a separate launch (2); 0: one workgroup per tile
  int32_t seg_m = 0, seg_n = 0;  // tile of the segmented rows' launch
  int32_t dispatches = 0;        // GEMM kernels the call launched (all its launch groups)
  int32_t rs_pieces = 0;         // row pieces of a pipelined device-side reduce-scatter
};

// K segmentation of an all-gather-side GEMM call: rows [seg_row, T) of the call are summed
// in nseg K segments (see gemm_bf16.hip), the rows before seg_row in one.  A function of the
// call's shape alone, so that every schedule computes the same bits.  nseg <= 1: none.
struct SegPlan {
  int64_t seg_row = -1;
  int32_t nseg = 1;
  int32_t tile_m = 0, tile_n = 0;  // tile of the split pieces (0: the library's choice)
  int32_t reduce = 0;              // 1: sum in the split kernel; 2: a separate launch (0: 2)
};
SegPlan choose_segmentation(int64_t T, int64_t n, int64_t k, int32_t batch);

struct GemmArgs {
  const uint16_t* a;
  int64_t lda;
  int64_t a_batch_stride;
  const uint16_t* b;
  int64_t ldb;
  int64_t b_batch_stride;
  uint16_t* c;
  int64_t ldc;
  int64_t c_batch_stride;
  int32_t m, n, k, batch;
  int32_t concurrency;  // launches expected to share the GPU with this one (>= 1)
  // Arrival gating (device-side chunk loop): before loading A, a tile waits until
  // ready[c] == epoch for every chunk c its rows touch (chunk c = rows [chunk_row0[c],
  // chunk_row0[c + 1])), then acquires; a wait over ~0.5 s gives up and counts one in
  // *timeouts.  ready == nullptr: no gating.
  const uint32_t* ready = nullptr;
  uint32_t epoch = 0;
  uint32_t* timeouts = nullptr;
  uint64_t wait_ticks = 0;  // bound of a tile's wait in 100 MHz ticks (0: ~0.5 s)
  int32_t n_chunks = 0;
  int32_t chunk_row0[kMaxGemmUnits + 1] = {};
  // Fused reduction (reduce-scatter side): fuse_nslots > 0 (== batch) makes the last of the
  // batch entries' tiles of each output tile to finish sum the entries' bf16 C tiles (the
  // slice partials) into fuse_out (row stride fuse_ldo), exactly as launch_reduce_partials
  // sums them: ascending slot order, or ring order (fuse_ring) with local row i in shard
  // (fuse_row0 + i) / fuse_shard_rows.  counters holds one word per tile of the launch,
  // zero at launch and left zero; a launch of more than counters_n tiles fails with
  // hipErrorInvalidValue.
  uint16_t* fuse_out = nullptr;
  int64_t fuse_ldo = 0;
  int32_t fuse_nslots = 0;
  int32_t fuse_ring = 0;
  int64_t fuse_row0 = 0;
  int64_t fuse_shard_rows = 1;
  uint32_t* counters = nullptr;
  int64_t counters_n = 0;
  // debug settings of the handle (nullptr: none) and where to record the plan taken
  const DebugOpts* dbg = nullptr;
  TilePlanRecord* plan_out = nullptr;
  // K segmentation (batch 1 only): rows of this launch at or after seg_row (in the
  // launch's own row coordinates) are summed in nseg K segments; nseg <= 1: none.  With a
  // split scratch (fp32 partial tiles and one zero word per tile, left zero) the segments
  // run as separate workgroups; without one, or when the launch needs more than it holds,
  // one workgroup per tile sums them in the same order.
  int64_t seg_row = 0;
  int32_t nseg = 1;
  int32_t seg_m = 0, seg_n = 0;  // tile of the split pieces (0: the library's choice)
  int32_t seg_reduce = 0;        // 1: sum in the split kernel; 2 (or 0): a separate launch
  float* split_parts = nullptr;
  int64_t split_parts_n = 0;   // floats
  uint32_t* split_counters = nullptr;
  int64_t split_counters_n = 0;
};
// Counter words the fused reduction of a handle can need: one range per compute stream,
// each large enough for one launch over up to `capacity` rows, and one for a device-side
// chunk loop over up to kMaxGemmUnits units (tiles of every shape counted at the smallest
// tile).  The words live in the registered workspace, after the partial slots.
int64_t fuse_counter_words(int64_t capacity, int64_t n);
// The range of one compute stream within those words.
int64_t fuse_counter_stream_words(int64_t capacity, int64_t n);
hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t stream);
// Whether the bf16 GEMM builds a tile of tile_m x tile_n.
bool gemm_bf16_tile_supported(int tile_m, int tile_n);
constexpr int kGemmKStep = 8;  // k must be a multiple of this (16-byte rows)

// Row units of a device-side chunk loop: one launch whose workgroups cover every unit's
// tiles, units in the given order, no tile spanning two units.  Unit u covers rows
// [row0[u], row0[u] + rows[u]) of A and C (g.m is ignored).
struct GemmUnits {
  int32_t n;
  int32_t row0[kMaxGemmUnits];
  int32_t rows[kMaxGemmUnits];
};
hipError_t launch_gemm_bf16_units(const GemmArgs& g, const GemmUnits& u, hipStream_t stream);

// Units of a device-side chunk loop re-cut for tiles of `bm` rows.  When the units tile a
// contiguous row range (they do for every plan), the range is cut into bm-row tiles from
// its first row, and each tile goes to the unit that holds its last row; the result lists,
// in the units' order, each unit's run of tiles as one unit (units left without a tile are
// dropped).  A tile then spans a unit boundary only where a unit is not a multiple of bm,
// and no row is computed twice.  Such a tile also reads rows of the unit before its own in
// row order; the device-side wait for arriving chunks therefore covers every chunk that
// the tile's rows touch, not the unit's alone.  Units that do not
// tile a contiguous range are returned unchanged.
GemmUnits tile_aligned_units(const GemmUnits& u, int bm);
// Row tiles of bm rows that a launch over `u` runs (after tile_aligned_units).
int64_t row_tiles(const GemmUnits& u, int bm);
// Whether the units tile one contiguous row range [*lo, *hi) without gaps or overlaps.
bool contiguous_rows(const GemmUnits& u, int64_t* lo, int64_t* hi);

// FP8 (E4M3) GEMM: C [*, n] bf16 = bf16(scale * A B^T) with A [*, k] and B [n, k] E4M3
// codes (row strides in bytes), units of rows as for launch_gemm_bf16_units.  batch > 1
// runs batch entries (blockIdx.z) whose A and B start a/b_batch_stride bytes further and
// whose C starts c_batch_stride elements further (the reduce-scatter side's K slices).
constexpr int kGemmF8KStep = 64;
struct GemmF8Args {
  const uint8_t* a;
  int64_t lda;
  const uint8_t* b;
  int64_t ldb;
  uint16_t* c;
  int64_t ldc;
  int32_t n, k;
  float scale;
  int concurrency;
  int64_t a_batch_stride = 0, b_batch_stride = 0, c_batch_stride = 0;
  int32_t batch = 1;
  const DebugOpts* dbg = nullptr;
  TilePlanRecord* plan_out = nullptr;
};
// Whether the FP8 GEMM builds a tile of tile_m x tile_n.
bool gemm_fp8_tile_supported(int tile_m, int tile_n);
bool gemm_fp8_shape_supported(const GemmF8Args& g);
hipError_t launch_gemm_fp8_units(const GemmF8Args& g, const GemmUnits& u, hipStream_t stream);

// bf16 rows -> E4M3 rows: dst[r, c] = sat(RNE_e4m3(fp32(src[r, c] * scale))).
hipError_t launch_quantize_e4m3(const uint16_t* src, int64_t lds, uint8_t* dst, int64_t ldd,
                                int64_t rows, int64_t cols, float scale, hipStream_t stream);

// Partial-sum reduction of `rows` x `cols` elements: slot s at parts + s * slot_stride
// (row stride ldp), result at out (row stride ldo).  ring == 0:
// out[r, c] = bf16(sum_{s < nslots} float(parts[s*slot_stride + r*ldp + c])), ascending s.
// ring != 0: ring order with a bf16 rounding per hop, where local row i is global row
// row0 + i of shard (row0 + i) / shard_rows.  cols % 8 == 0, ldp/ldo % 8 == 0, pointers
// 16-byte aligned.
struct ReduceArgs {
  const uint16_t* parts;
  int64_t slot_stride;
  int64_t ldp;
  int32_t nslots;
  uint16_t* out;
  int64_t ldo;
  int64_t rows;
  int64_t cols;
  int32_t ring;
  int64_t row0;
  int64_t shard_rows;
};
hipError_t launch_reduce_partials(const ReduceArgs& r, hipStream_t stream);

// The fixed device scratch of ub_gemm_rs_chunked_noalloc (static_scratch.hip): its size, its
// address on the current device (nullptr and *err set on failure), and a fill of n 32-bit
// words with zeros on `stream` (a kernel, so that the call can be captured into a graph).
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
unsigned char* static_scratch_base(hipError_t* err);
hipError_t launch_clear_words(uint32_t* p, int64_t n, hipStream_t stream);

}  // namespace ubx
