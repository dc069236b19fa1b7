// C ABI of the capacity/active-shape UserBuffer and its chunked overlap GEMMs.
//
// Buffer manager: "[Feature Request] Support dynamic token counts in TP communication/GEMM
// overlap" (Transformer Engine issue 3564), sections "Proposed API" and "Implementation
// approach in the prototype": a buffer registered once at [max_tokens, hidden]; a separate
// active shape per microbatch whose data is the buffer's contiguous prefix; views, offsets
// and copy-size checks recomputed from the active T; no allocation, free or
// re-registration on a shape change; the constraint list on the active shape.
//
// Scheduler: "How to setup TP Overlap configs" (Transformer Engine issue 1344), option
// list: GEMM chunks on min(num_splits, num_max_streams) compute streams.  Here stream 0 of
// a plan is the caller's stream and streams 1..S-1 are the handle's own non-blocking HIP
// streams (default priority).  A call forks them from the caller's stream with one event
// and joins them back with one event each, so the call as a whole is ordered on the
// caller's stream and never synchronises the host.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <mutex>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include <rocprofiler-sdk-roctx/roctx.h>

#include "ub_internal.h"

constexpr int kMaxArrivalChunks = 64;
constexpr int kMaxRsPieces = 8;

struct ub_ctx {
  // registration
  int64_t capacity = 0;
  int64_t hidden = 0;
  int32_t tp = 1;
  ub_dtype_t dtype = UB_DTYPE_BF16;
  int64_t elem_bytes = 2;        // 2 (bf16) or 1 (fp8)
  uint16_t* ub = nullptr;        // the buffer as bf16 elements
  uint8_t* ub8 = nullptr;        // the same buffer as bytes (fp8 codes)
  size_t ub_bytes = 0;
  uint16_t* ws = nullptr;
  size_t ws_bytes = 0;
  // active shape
  int64_t T = 0;
  // device resources, created on the first GEMM call
  int device = -1;
  hipStream_t streams[UB_MAX_STREAMS] = {};  // [0] unused: the caller's stream
  int n_streams_created = 1;
  hipEvent_t ev_fork = nullptr;
  hipEvent_t ev_join[UB_MAX_STREAMS] = {};
  // kernel timing: 0 off, 1 an event pair per launch, 2 chained (a launch starts at the
  // end event of the previous timed launch on its stream)
  int32_t timing = 0;
  struct TimedLaunch {
    hipEvent_t start, stop;
    int kind;  // 0 gemm, 1 reduce
    double flops, bytes;
  };
  std::vector<hipEvent_t> free_events;
  std::vector<TimedLaunch> pending;
  std::vector<std::pair<hipStream_t, hipEvent_t>> chain;  // last end event per stream (mode 2)
  ub_kernel_stats_t stats[2] = {};
  // arrival stand-in: copy stream, one arrival event per chunk, its join event
  hipStream_t copy_stream = nullptr;
  hipEvent_t ev_arrive[kMaxArrivalChunks] = {};
  hipEvent_t ev_piece[kMaxRsPieces] = {};  // pipelined device-side reduce-scatter
  hipEvent_t ev_copy_join = nullptr;
  // device-side arrival gating: this handle's slot of arrival flags (-1: none yet)
  int ready_slot = -1;
  uint32_t* ready = nullptr;  // device address of the slot's words
  // fused reduction: per-tile arrival counters in the workspace, after the partial slots
  // (zero at registration, left zero by every launch)
  uint32_t* fuse_counters = nullptr;
  int64_t fuse_counters_n = 0;
  // debug settings (ub_debug_set) and the tile plan of the last GEMM launch group
  ubx::DebugOpts dbg;
  ubx::TilePlanRecord last_plan;
  // split-K scratch (ub_register_scratch): counter words (zero at registration, left zero)
  // and fp32 partial tiles; one range of each per compute stream
  uint32_t* split_counters = nullptr;
  int64_t split_counters_n = 0;
  float* split_parts = nullptr;
  int64_t split_parts_n = 0;
  // scratch for plans
  ubx::Plan plan;
  std::string last_error;
};

namespace {

// A roctx range around each work-issuing entry point, so that a marker trace
// (rocprofv3 --marker-trace) shows which library call issued which launches and copies.
// Without a profiler attached the push and pop do nothing.
struct TraceRange {
  explicit TraceRange(const char* name) { roctxRangePushA(name); }
  ~TraceRange() { roctxRangePop(); }
  TraceRange(const TraceRange&) = delete;
  TraceRange& operator=(const TraceRange&) = delete;
};

constexpr int64_t kMaxRowsPerUnit = int64_t(1) << 30;

ub_status_t fail(ub_ctx* h, ub_status_t st, const char* fmt, ...) {
  if (h) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    h->last_error = buf;
  }
  return st;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t elem_bytes_of(ub_dtype_t dtype) { return dtype == UB_DTYPE_FP8_E4M3 ? 1 : 2; }

ub_status_t check_registration(int64_t capacity, int64_t hidden, int32_t tp, ub_dtype_t dtype,
                               std::string* err) {
  if (dtype != UB_DTYPE_BF16 && dtype != UB_DTYPE_FP8_E4M3) {
    *err = "UserBuffers are bf16 or fp8 E4M3";
    return UB_ERR_DTYPE;
  }
  if (dtype == UB_DTYPE_FP8_E4M3 && hidden % 16 != 0) {
    *err = "an fp8 UserBuffer needs hidden to be a multiple of 16 (16-byte rows)";
    return UB_ERR_INVALID_ARG;
  }
  if (capacity <= 0 || hidden <= 0) {
    *err = "capacity and hidden must be > 0";
    return UB_ERR_INVALID_ARG;
  }
  if (tp < 1 || tp > UB_MAX_TP) {
    *err = "tp_size must be in [1, " + std::to_string(UB_MAX_TP) + "]";
    return UB_ERR_INVALID_ARG;
  }
  if (hidden % 8 != 0) {
    *err = "hidden must be a multiple of 8 (16-byte rows)";
    return UB_ERR_INVALID_ARG;
  }
  if (capacity % tp != 0) {
    *err = "capacity must be divisible by tp_size (the initial active shape is the capacity)";
    return UB_ERR_TP_DIVISIBILITY;
  }
  if (capacity > (int64_t(1) << 40) / hidden) {
    *err = "capacity * hidden too large";
    return UB_ERR_INVALID_ARG;
  }
  return UB_OK;
}

// Reduce-scatter workspace: tp_size partial slots of [capacity, hidden] bf16, then, from
// the next 256-byte boundary, the fused reduction's counter words (ubx::fuse_counter_words).
struct WsLayout {
  size_t partial_bytes, counter_offset, counter_words, total;
};

WsLayout ws_layout(int64_t capacity, int64_t hidden, int32_t tp) {
  WsLayout l;
  l.partial_bytes = static_cast<size_t>(capacity) * static_cast<size_t>(hidden) * 2 *
                    static_cast<size_t>(tp);
  l.counter_offset = (l.partial_bytes + 255) / 256 * 256;
  l.counter_words = static_cast<size_t>(ubx::fuse_counter_words(capacity, hidden));
  l.total = l.counter_offset + l.counter_words * sizeof(uint32_t);
  return l;
}

ub_status_t hip_fail(ub_ctx* h, hipError_t e, const char* what) {
  return fail(h, UB_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Bind the handle to the current device and create the streams/events it needs.
ub_status_t ensure_device(ub_ctx* h, int need_streams) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(h, e, "hipGetDevice");
  if (h->device < 0) {
    h->device = dev;
    e = hipEventCreateWithFlags(&h->ev_fork, hipEventDisableTiming);
    if (e != hipSuccess) return hip_fail(h, e, "hipEventCreate");
    for (hipEvent_t& ev : h->ev_piece) {
      e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
      if (e != hipSuccess) return hip_fail(h, e, "hipEventCreate");
    }
  } else if (h->device != dev) {
    return fail(h, UB_ERR_INVALID_ARG, "handle is bound to device %d but device %d is current",
                h->device, dev);
  }
  while (h->n_streams_created < need_streams) {
    const int i = h->n_streams_created;
    e = hipStreamCreateWithFlags(&h->streams[i], hipStreamNonBlocking);
    if (e != hipSuccess) return hip_fail(h, e, "hipStreamCreate");
    e = hipEventCreateWithFlags(&h->ev_join[i], hipEventDisableTiming);
    if (e != hipSuccess) return hip_fail(h, e, "hipEventCreate");
    h->n_streams_created = i + 1;
  }
  return UB_OK;
}

// The copy stream and arrival events of the arrival stand-in.
ub_status_t ensure_arrival(ub_ctx* h, int n_chunks) {
  hipError_t e;
  if (!h->copy_stream) {
    e = hipStreamCreateWithFlags(&h->copy_stream, hipStreamNonBlocking);
    if (e != hipSuccess) return hip_fail(h, e, "hipStreamCreate(copy)");
    e = hipEventCreateWithFlags(&h->ev_copy_join, hipEventDisableTiming);
    if (e != hipSuccess) return hip_fail(h, e, "hipEventCreate");
  }
  for (int c = 0; c < n_chunks; ++c) {
    if (h->ev_arrive[c]) continue;
    e = hipEventCreateWithFlags(&h->ev_arrive[c], hipEventDisableTiming);
    if (e != hipSuccess) return hip_fail(h, e, "hipEventCreate");
  }
  return UB_OK;
}

// ---- arrival flags of the device-side chunk loop -----------------------------------------
// Slots of the flag array are handed to handles on their first gated call and returned by
// ub_destroy.  Epochs come from one process-wide counter, so a flag left by an earlier call
// (of any handle that held the slot) never equals the epoch of a later call; 0 is skipped,
// the value the flags start from.
std::mutex g_slot_mu;
uint64_t g_slot_used = 0;
std::atomic<uint32_t> g_epoch{0};

uint32_t next_epoch() {
  uint32_t e = ++g_epoch;
  if (e == 0) e = ++g_epoch;
  return e;
}

ub_status_t ensure_ready_slot(ub_ctx* h) {
  if (h->ready) return UB_OK;
  hipError_t e = hipSuccess;
  uint32_t* base = ubx::ready_flags_base(&e);
  if (!base) return hip_fail(h, e, "hipGetSymbolAddress(arrival flags)");
  std::lock_guard<std::mutex> lock(g_slot_mu);
  for (int s = 0; s < ubx::kReadySlots; ++s) {
    if (g_slot_used >> s & 1) continue;
    g_slot_used |= uint64_t(1) << s;
    h->ready_slot = s;
    h->ready = base + (size_t)s * ubx::kReadyWords;
    return UB_OK;
  }
  return fail(h, UB_ERR_UNSUPPORTED,
              "more than %d handles gate the device-side chunk loop on arrivals at once",
              ubx::kReadySlots);
}

void release_ready_slot(ub_ctx* h) {
  if (h->ready_slot < 0) return;
  std::lock_guard<std::mutex> lock(g_slot_mu);
  g_slot_used &= ~(uint64_t(1) << h->ready_slot);
  h->ready_slot = -1;
  h->ready = nullptr;
}

// ---- per-launch timing ----------------------------------------------------------------
bool in_chain(const ub_ctx* h, hipEvent_t ev) {
  for (const auto& c : h->chain)
    if (c.second == ev) return true;
  return false;
}

// Waits for every pending timed launch and adds it to the stats.  Its events go back to
// the pool, except the chain's current end events, which later launches start from (a
// chained launch's start event is the previous launch's stop event: each is freed once).
ub_status_t harvest(ub_ctx* h) {
  for (auto& t : h->pending) {
    hipError_t e = hipEventSynchronize(t.stop);
    if (e != hipSuccess) return hip_fail(h, e, "hipEventSynchronize");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, t.start, t.stop);
    if (e != hipSuccess) return hip_fail(h, e, "hipEventElapsedTime");
    ub_kernel_stats_t& s = h->stats[t.kind];
    s.launches += 1;
    s.total_ms += ms;
    s.flops += t.flops;
    s.bytes += t.bytes;
  }
  std::vector<hipEvent_t> done;
  for (auto& t : h->pending) {
    done.push_back(t.start);
    done.push_back(t.stop);
  }
  std::sort(done.begin(), done.end());
  done.erase(std::unique(done.begin(), done.end()), done.end());
  for (hipEvent_t ev : done)
    if (!in_chain(h, ev)) h->free_events.push_back(ev);
  h->pending.clear();
  return UB_OK;
}

// Ends every chain: the next timed launch on each stream records a start event of its own.
// A chain head that no pending launch holds goes back to the pool now; the others go back
// when harvest takes their launch.
void clear_chain(ub_ctx* h) {
  std::vector<std::pair<hipStream_t, hipEvent_t>> heads;
  heads.swap(h->chain);
  for (const auto& c : heads) {
    bool held = false;
    for (const auto& t : h->pending) held = held || t.start == c.second || t.stop == c.second;
    if (!held) h->free_events.push_back(c.second);
  }
}

hipEvent_t take_event(ub_ctx* h) {
  if (!h->free_events.empty()) {
    hipEvent_t ev = h->free_events.back();
    h->free_events.pop_back();
    return ev;
  }
  hipEvent_t ev = nullptr;
  if (hipEventCreate(&ev) != hipSuccess) return nullptr;
  return ev;
}

constexpr size_t kMaxPendingTimings = 4096;

template <class Launch>
ub_status_t timed_launch(ub_ctx* h, hipStream_t s, int kind, double flops, double bytes,
                         Launch&& launch, const char* what) {
  if (!h->timing) {
    hipError_t e = launch();
    return e == hipSuccess ? UB_OK : hip_fail(h, e, what);
  }
  if (h->pending.size() >= kMaxPendingTimings) {
    ub_status_t st = harvest(h);  // oldest launches finished long ago: no real stall
    if (st != UB_OK) return st;
  }
  hipEvent_t a = nullptr;
  size_t link = h->chain.size();
  if (h->timing == 2)
    for (size_t i = 0; i < h->chain.size(); ++i)
      if (h->chain[i].first == s) link = i;
  if (link < h->chain.size()) a = h->chain[link].second;
  const bool own_a = a == nullptr;
  if (own_a) a = take_event(h);
  hipEvent_t b = take_event(h);
  if (!a || !b) return fail(h, UB_ERR_HIP, "hipEventCreate failed for kernel timing");
  hipError_t e = own_a ? hipEventRecord(a, s) : hipSuccess;
  if (e == hipSuccess) {
    // the call's kernels record b at their end (launch_k); a call that launched none
    // records it here
    ubx::g_launch_stop = b;
    ubx::g_launch_stop_used = false;
    e = launch();
    ubx::g_launch_stop = nullptr;
    if (e == hipSuccess && !ubx::g_launch_stop_used) e = hipEventRecord(b, s);
  }
  if (e != hipSuccess) return hip_fail(h, e, what);
  h->pending.push_back({a, b, kind, flops, bytes});
  if (h->timing == 2) {
    if (link < h->chain.size()) h->chain[link].second = b;
    else h->chain.push_back({s, b});
  }
  return UB_OK;
}

// ---- fork / join ----------------------------------------------------------------------
ub_status_t fork_streams(ub_ctx* h, hipStream_t caller, int S) {
  if (S <= 1) return UB_OK;
  hipError_t e = hipEventRecord(h->ev_fork, caller);
  if (e != hipSuccess) return hip_fail(h, e, "hipEventRecord(fork)");
  for (int i = 1; i < S; ++i) {
    e = hipStreamWaitEvent(h->streams[i], h->ev_fork, 0);
    if (e != hipSuccess) return hip_fail(h, e, "hipStreamWaitEvent(fork)");
  }
  return UB_OK;
}

ub_status_t join_streams(ub_ctx* h, hipStream_t caller, int S) {
  for (int i = 1; i < S; ++i) {
    hipError_t e = hipEventRecord(h->ev_join[i], h->streams[i]);
    if (e != hipSuccess) return hip_fail(h, e, "hipEventRecord(join)");
    e = hipStreamWaitEvent(caller, h->ev_join[i], 0);
    if (e != hipSuccess) return hip_fail(h, e, "hipStreamWaitEvent(join)");
  }
  return UB_OK;
}

ub_status_t need_dtype(ub_ctx* h, ub_dtype_t want, const char* what) {
  if (h->dtype == want) return UB_OK;
  return fail(h, UB_ERR_DTYPE, "%s needs a %s UserBuffer", what,
              want == UB_DTYPE_BF16 ? "bf16" : "fp8 E4M3");
}

ub_status_t check_cfg_common(ub_ctx* h, const ub_overlap_cfg_t* cfg) {
  if (!cfg) return fail(h, UB_ERR_INVALID_ARG, "cfg is NULL");
  if (cfg->reduce_order != UB_REDUCE_ASCENDING && cfg->reduce_order != UB_REDUCE_RING)
    return fail(h, UB_ERR_INVALID_ARG, "reduce_order=%d is not a ub_reduce_order_t",
                cfg->reduce_order);
  if (cfg->fuse_reduce != 0 && cfg->fuse_reduce != 1)
    return fail(h, UB_ERR_INVALID_ARG, "fuse_reduce=%d must be 0 or 1", cfg->fuse_reduce);
  return UB_OK;
}

// K segmentation of an all-gather-side call at the active T (a function of the call's shape
// alone, or forced by the handle's debug settings), and the split scratch range of compute
// stream `si` (of S streams; the device-side loop has the whole scratch).
// Without a registered scratch nothing is segmented unless the debug settings force it.
ubx::SegPlan ag_segmentation(const ub_ctx* h, int64_t n_cols) {
  if (h->dbg.nseg == 1) return ubx::SegPlan{};
  if (h->dbg.nseg >= 2)
    return ubx::SegPlan{std::max<int64_t>(h->dbg.seg_row, 0), h->dbg.nseg, h->dbg.seg_m,
                        h->dbg.seg_n, h->dbg.seg_reduce};
  if (!h->split_parts) return ubx::SegPlan{};
  return ubx::choose_segmentation(h->T, n_cols, h->hidden, 1);
}

void set_segmentation(const ub_ctx* h, ubx::GemmArgs& g, const ubx::SegPlan& sp, int64_t row0,
                      int si, int S) {
  if (sp.nseg <= 1) return;
  g.seg_row = sp.seg_row - row0;
  g.nseg = sp.nseg;
  g.seg_m = sp.tile_m;
  g.seg_n = sp.tile_n;
  g.seg_reduce = sp.reduce;
  if (!h->split_parts) return;
  const int64_t cw = h->split_counters_n / S, pw = h->split_parts_n / S / 64 * 64;  // 256 B aligned
  g.split_counters = h->split_counters + si * cw;
  g.split_counters_n = cw;
  g.split_parts = h->split_parts + si * pw;
  g.split_parts_n = pw;
}

// Units of the plan, in execution order, for a device-side chunk loop.
ub_status_t plan_units(ub_ctx* h, ubx::GemmUnits* u) {
  u->n = 0;
  for (const ub_plan_unit_t& pu : h->plan.units) {
    const int64_t rows = pu.row1 - pu.row0;
    if (rows <= 0) continue;
    if (u->n == ubx::kMaxGemmUnits)
      return fail(h, UB_ERR_UNSUPPORTED, "atomic_gemm supports at most %d non-empty units",
                  ubx::kMaxGemmUnits);
    u->row0[u->n] = static_cast<int32_t>(pu.row0);
    u->rows[u->n] = static_cast<int32_t>(rows);
    ++u->n;
  }
  return UB_OK;
}

// A tile shape forced by ub_debug_set must be one the call's kernel builds.
ub_status_t check_forced_tile(ub_ctx* h, bool fp8) {
  const ubx::DebugOpts& d = h->dbg;
  auto ok = [&](int m, int n) {
    return fp8 ? ubx::gemm_fp8_tile_supported(m, n) : ubx::gemm_bf16_tile_supported(m, n);
  };
  if ((d.tile_m || d.tile_n) && !ok(d.tile_m, d.tile_n))
    return fail(h, UB_ERR_INVALID_ARG, "the %s GEMM has no %dx%d tile (debug tile_m/tile_n)",
                fp8 ? "fp8" : "bf16", d.tile_m, d.tile_n);
  if (d.cut_row > 0 && fp8)
    return fail(h, UB_ERR_INVALID_ARG, "the fp8 GEMM takes no forced cut (debug cut_row)");
  if (d.cut_row > 0 && (d.tail_m || d.tail_n) && !ok(d.tail_m, d.tail_n))
    return fail(h, UB_ERR_INVALID_ARG, "the bf16 GEMM has no %dx%d tile (debug tail_tile_m/n)",
                d.tail_m, d.tail_n);
  if (!fp8 && d.nseg >= 2 && (d.seg_m || d.seg_n) && !ok(d.seg_m, d.seg_n))
    return fail(h, UB_ERR_INVALID_ARG, "the bf16 GEMM has no %dx%d tile (debug seg_tile_m/n)",
                d.seg_m, d.seg_n);
  return UB_OK;
}

ub_status_t check_ld(ub_ctx* h, const char* name, int64_t ld, int64_t cols) {
  if (ld < cols || ld % 8 != 0)
    return fail(h, UB_ERR_INVALID_ARG, "%s=%lld must be >= %lld and a multiple of 8", name,
                (long long)ld, (long long)cols);
  return UB_OK;
}

// The reduction of active rows [row0, row0 + rows): the tp partial slots of the packed
// workspace prefix (slot s at element s*T*H) into out (row stride ldo), ascending or in ring
// order (each row's shard T/tp decides its hop order).
ubx::ReduceArgs reduce_args(const ub_ctx* h, int64_t row0, int64_t rows, void* out, int64_t ldo,
                            bool ring, const uint16_t* ws = nullptr) {
  const int64_t H = h->hidden;
  ubx::ReduceArgs r{};
  r.parts = (ws ? ws : h->ws) + row0 * H;
  r.slot_stride = h->T * H;
  r.ldp = H;
  r.nslots = h->tp;
  r.out = static_cast<uint16_t*>(out) + row0 * ldo;
  r.ldo = ldo;
  r.rows = rows;
  r.cols = H;
  r.ring = ring;
  r.row0 = row0;
  r.shard_rows = h->T / h->tp;
  return r;
}

}  // namespace

extern "C" {

UB_API void ub_overlap_cfg_default(ub_overlap_cfg_t* cfg) {
  if (!cfg) return;
  std::memset(cfg, 0, sizeof(*cfg));
  cfg->method = UB_RING_EXCHANGE;
  cfg->num_splits = 1;
  cfg->num_max_streams = 3;
  cfg->aggregate = 0;
  cfg->atomic_gemm = 0;
  cfg->rank = 0;
  cfg->use_ce = 1;
  cfg->num_sm = 0;
  cfg->set_sm_margin = 0;
  cfg->reduce_order = UB_REDUCE_ASCENDING;
  cfg->fuse_reduce = 0;
}

UB_API const char* ub_status_string(ub_status_t s) {
  switch (s) {
    case UB_OK: return "UB_OK";
    case UB_ERR_INVALID_ARG: return "UB_ERR_INVALID_ARG";
    case UB_ERR_NDIM: return "UB_ERR_NDIM";
    case UB_ERR_ZERO_DIM: return "UB_ERR_ZERO_DIM";
    case UB_ERR_CAPACITY: return "UB_ERR_CAPACITY";
    case UB_ERR_HIDDEN_MISMATCH: return "UB_ERR_HIDDEN_MISMATCH";
    case UB_ERR_TP_DIVISIBILITY: return "UB_ERR_TP_DIVISIBILITY";
    case UB_ERR_DTYPE: return "UB_ERR_DTYPE";
    case UB_ERR_UNSUPPORTED: return "UB_ERR_UNSUPPORTED";
    case UB_ERR_BUFFER_TOO_SMALL: return "UB_ERR_BUFFER_TOO_SMALL";
    case UB_ERR_NOT_INITIALIZED: return "UB_ERR_NOT_INITIALIZED";
    case UB_ERR_HIP: return "UB_ERR_HIP";
  }
  return "UB_ERR_UNKNOWN";
}

UB_API const char* ub_last_error(ub_handle_t h) { return h ? h->last_error.c_str() : ""; }

UB_API ub_status_t ub_required_bytes(int64_t capacity, int64_t hidden, int32_t tp_size,
                                     ub_dtype_t dtype, size_t* ub_bytes,
                                     size_t* rs_workspace_bytes) {
  std::string err;
  ub_status_t st = check_registration(capacity, hidden, tp_size, dtype, &err);
  if (st != UB_OK) return st;
  const size_t elems = static_cast<size_t>(capacity) * static_cast<size_t>(hidden);
  if (ub_bytes) *ub_bytes = elems * static_cast<size_t>(elem_bytes_of(dtype));
  // the reduce-scatter side (bf16 partials) exists for bf16 buffers only
  if (rs_workspace_bytes)
    *rs_workspace_bytes = dtype == UB_DTYPE_BF16 ? ws_layout(capacity, hidden, tp_size).total : 0;
  return UB_OK;
}

UB_API ub_status_t ub_init(ub_handle_t* out, int64_t capacity, int64_t hidden, int32_t tp_size,
                           ub_dtype_t dtype, void* ub_buf, size_t ub_bytes, void* rs_ws,
                           size_t rs_ws_bytes) {
  if (!out) return UB_ERR_INVALID_ARG;
  *out = nullptr;
  std::string err;
  ub_status_t st = check_registration(capacity, hidden, tp_size, dtype, &err);
  if (st != UB_OK) return st;
  const size_t elems = static_cast<size_t>(capacity) * static_cast<size_t>(hidden);
  const size_t need = elems * static_cast<size_t>(elem_bytes_of(dtype));
  if (!ub_buf || !aligned16(ub_buf)) return UB_ERR_INVALID_ARG;
  if (ub_bytes < need) return UB_ERR_BUFFER_TOO_SMALL;
  if (dtype != UB_DTYPE_BF16 && (rs_ws || rs_ws_bytes)) return UB_ERR_INVALID_ARG;
  const WsLayout wl = ws_layout(capacity, hidden, tp_size);
  if (rs_ws) {
    if (!aligned16(rs_ws)) return UB_ERR_INVALID_ARG;
    if (rs_ws_bytes < wl.total) return UB_ERR_BUFFER_TOO_SMALL;
  } else if (rs_ws_bytes != 0) {
    return UB_ERR_INVALID_ARG;
  }
  ub_ctx* h = new (std::nothrow) ub_ctx();
  if (!h) return UB_ERR_INVALID_ARG;
  h->capacity = capacity;
  h->hidden = hidden;
  h->tp = tp_size;
  h->dtype = dtype;
  h->elem_bytes = elem_bytes_of(dtype);
  h->ub = static_cast<uint16_t*>(ub_buf);
  h->ub8 = static_cast<uint8_t*>(ub_buf);
  h->ub_bytes = ub_bytes;
  h->ws = static_cast<uint16_t*>(rs_ws);
  h->ws_bytes = rs_ws_bytes;
  if (rs_ws) {
    h->fuse_counters =
        reinterpret_cast<uint32_t*>(static_cast<unsigned char*>(rs_ws) + wl.counter_offset);
    h->fuse_counters_n = static_cast<int64_t>(wl.counter_words);
  }
  h->T = capacity;  // the initial active shape is the capacity shape
  *out = h;
  return UB_OK;
}

UB_API ub_status_t ub_set_active_shape(ub_handle_t h, const int64_t* shape, int32_t ndim) {
  if (!h) return UB_ERR_NOT_INITIALIZED;
  if (ndim != 2) return fail(h, UB_ERR_NDIM, "active shape must be 2-D, got %d dims", ndim);
  if (!shape) return fail(h, UB_ERR_INVALID_ARG, "shape is NULL");
  const int64_t T = shape[0], H = shape[1];
  if (T <= 0 || H <= 0)
    return fail(h, UB_ERR_ZERO_DIM, "active shape [%lld, %lld] has a dimension <= 0",
                (long long)T, (long long)H);
  if (T > h->capacity)
    return fail(h, UB_ERR_CAPACITY, "active T=%lld exceeds capacity %lld", (long long)T,
                (long long)h->capacity);
  if (H != h->hidden)
    return fail(h, UB_ERR_HIDDEN_MISMATCH, "active hidden %lld != registered %lld",
                (long long)H, (long long)h->hidden);
  if (T % h->tp != 0)
    return fail(h, UB_ERR_TP_DIVISIBILITY, "active T=%lld not divisible by tp_size %d",
                (long long)T, h->tp);
  h->T = T;  // views and offsets are derived from T at each call; nothing else changes
  h->last_error.clear();
  return UB_OK;
}

UB_API ub_status_t ub_get_active_shape(ub_handle_t h, int64_t shape_out[2]) {
  if (!h) return UB_ERR_NOT_INITIALIZED;
  if (!shape_out) return fail(h, UB_ERR_INVALID_ARG, "shape_out is NULL");
  shape_out[0] = h->T;
  shape_out[1] = h->hidden;
  return UB_OK;
}

UB_API ub_status_t ub_get_capacity_shape(ub_handle_t h, int64_t shape_out[2]) {
  if (!h) return UB_ERR_NOT_INITIALIZED;
  if (!shape_out) return fail(h, UB_ERR_INVALID_ARG, "shape_out is NULL");
  shape_out[0] = h->capacity;
  shape_out[1] = h->hidden;
  return UB_OK;
}

UB_API ub_status_t ub_get_plan(ub_handle_t h, const ub_overlap_cfg_t* cfg, ub_op_t op,
                               ub_plan_unit_t* out, int32_t max_units, int32_t* n_units,
                               int32_t* n_streams) {
  if (!h) return UB_ERR_NOT_INITIALIZED;
  if (!cfg) return fail(h, UB_ERR_INVALID_ARG, "cfg is NULL");
  if (max_units < 0 || (max_units > 0 && !out))
    return fail(h, UB_ERR_INVALID_ARG, "bad output array");
  ub_status_t st = ubx::build_plan(h->T, h->tp, *cfg, op, &h->plan, &h->last_error);
  if (st != UB_OK) return st;
  const int32_t U = static_cast<int32_t>(h->plan.units.size());
  for (int32_t i = 0; i < std::min(U, max_units); ++i) out[i] = h->plan.units[i];
  if (n_units) *n_units = U;
  if (n_streams) *n_streams = h->plan.n_streams;
  return UB_OK;
}

UB_API ub_status_t ub_copy_in(ub_handle_t h, const void* src, int64_t rows, int64_t row_offset,
                              ub_stream_t stream) {
  const TraceRange range("ub_copy_in");
  if (!h) return UB_ERR_NOT_INITIALIZED;
  if (!src) return fail(h, UB_ERR_INVALID_ARG, "src is NULL");
  if (rows < 0 || row_offset < 0 || row_offset + rows > h->T)
    return fail(h, UB_ERR_INVALID_ARG,
                "copy of %lld rows at row %lld does not fit the active T=%lld", (long long)rows,
                (long long)row_offset, (long long)h->T);
  if (rows == 0) return UB_OK;
  ub_status_t st = ensure_device(h, 1);
  if (st != UB_OK) return st;
  const int64_t row_bytes = h->hidden * h->elem_bytes;
  hipError_t e = hipMemcpyAsync(h->ub8 + row_offset * row_bytes, src,
                                static_cast<size_t>(rows * row_bytes), hipMemcpyDeviceToDevice,
                                static_cast<hipStream_t>(stream));
  return e == hipSuccess ? UB_OK : hip_fail(h, e, "hipMemcpyAsync");
}

namespace {

// Arguments of an all-gather-side GEMM call, checked before any HIP call; builds the plan.
ub_status_t check_ag_call(ub_ctx* h, const void* w, int64_t n_cols, int64_t ldw, const void* c,
                          int64_t ldc, const ub_overlap_cfg_t* cfg) {
  ub_status_t st = check_cfg_common(h, cfg);
  if (st != UB_OK) return st;
  if (!w || !c) return fail(h, UB_ERR_INVALID_ARG, "w and c must be non-NULL");
  if (!aligned16(w) || !aligned16(c))
    return fail(h, UB_ERR_INVALID_ARG, "w and c must be 16-byte aligned");
  if (n_cols <= 0 || n_cols % 8 != 0 || n_cols > INT32_MAX)
    return fail(h, UB_ERR_INVALID_ARG, "n_cols=%lld must be > 0 and a multiple of 8",
                (long long)n_cols);
  if ((st = check_ld(h, "ldw", ldw, n_cols)) != UB_OK) return st;
  if ((st = check_ld(h, "ldc", ldc, n_cols)) != UB_OK) return st;
  if (h->hidden % ubx::kGemmKStep != 0)
    return fail(h, UB_ERR_UNSUPPORTED, "hidden=%lld must be a multiple of %d",
                (long long)h->hidden, ubx::kGemmKStep);
  if ((st = check_forced_tile(h, false)) != UB_OK) return st;
  return ubx::build_plan(h->T, h->tp, *cfg, UB_OP_AG, &h->plan, &h->last_error);
}

// Chunk c of n covers rows [c*T/n, (c+1)*T/n); a unit of index u covers chunks
// [u*agg, min((u+1)*agg, n)).
struct ChunkMap {
  int n = 0, agg = 1, local = -1;  // local: the chunk already in the UB (ring), or -1
  int64_t row0(int64_t T, int c) const { return (int64_t)c * T / n; }
  int first(int u) const { return u * agg; }
  int last(int u) const { return std::min((u + 1) * agg, n); }
};

ChunkMap chunk_map(const ub_ctx* h, const ub_overlap_cfg_t* cfg) {
  ChunkMap m;
  m.n = cfg->method == UB_RING_EXCHANGE ? h->tp : cfg->num_splits;
  m.agg = cfg->aggregate ? 2 : 1;
  m.local = cfg->method == UB_RING_EXCHANGE ? cfg->rank : -1;
  return m;
}

// The arrival stand-in's copy stream starts when the caller's stream reaches the call.
ub_status_t start_deliveries(ub_ctx* h, int n_chunks, hipStream_t caller) {
  ub_status_t st = ensure_arrival(h, n_chunks);
  if (st != UB_OK) return st;
  hipError_t e = hipEventRecord(h->ev_fork, caller);
  if (e == hipSuccess) e = hipStreamWaitEvent(h->copy_stream, h->ev_fork, 0);
  return e == hipSuccess ? UB_OK : hip_fail(h, e, "copy stream fork");
}

// The copies of one unit's non-local chunks (ascending) on the copy stream; chunk c's
// event is recorded after its copy.
ub_status_t deliver_unit(ub_ctx* h, const uint16_t* src, int src_on_host,
                         const ub_overlap_cfg_t* cfg, const ChunkMap& m,
                         const ub_plan_unit_t& u) {
  // Host source: pinned memory over PCIe, always on the SDMA engines.  Device source: the
  // SDMA engines (use_ce) or the runtime's copy kernel.
  const hipMemcpyKind kind = src_on_host  ? hipMemcpyHostToDevice
                             : cfg->use_ce ? hipMemcpyDeviceToDeviceNoCU
                                           : hipMemcpyDeviceToDevice;
  const int64_t H = h->hidden, T = h->T;
  for (int c = m.first(u.unit); c < m.last(u.unit); ++c) {
    if (c == m.local) continue;
    const int64_t r0 = m.row0(T, c), rows = m.row0(T, c + 1) - r0;
    hipError_t e = hipSuccess;
    if (rows > 0)
      e = hipMemcpyAsync(h->ub + r0 * H, src + r0 * H, static_cast<size_t>(rows * H) * 2, kind,
                         h->copy_stream);
    if (e == hipSuccess) e = hipEventRecord(h->ev_arrive[c], h->copy_stream);
    if (e != hipSuccess) return hip_fail(h, e, "arrival copy");
  }
  return UB_OK;
}

ub_status_t join_deliveries(ub_ctx* h, hipStream_t caller) {
  hipError_t e = hipEventRecord(h->ev_copy_join, h->copy_stream);
  if (e == hipSuccess) e = hipStreamWaitEvent(caller, h->ev_copy_join, 0);
  return e == hipSuccess ? UB_OK : hip_fail(h, e, "copy stream join");
}

// Device-side chunk loop with arrivals: every chunk's copy is followed, on the copy stream,
// by a write of the call's epoch to the chunk's flag (the local chunk's flag first: it is
// already in the UB); the tiles of the one GEMM launch wait for the flags of the chunks
// they read.  Everything on the copy stream is issued before the GEMM, so where the two
// streams share a hardware queue the copies run first and nothing waits on work queued
// behind it.
// Bound of a gated tile's wait in 100 MHz ticks (0: the kernel's default of ~0.5 s).
uint64_t arrival_wait_ticks(const ub_ctx* h) {
  return h->dbg.arrival_wait_us > 0 ? static_cast<uint64_t>(h->dbg.arrival_wait_us) * 100 : 0;
}

ub_status_t deliver_flagged(ub_ctx* h, const uint16_t* src, int src_on_host,
                            const ub_overlap_cfg_t* cfg, const ChunkMap& m, uint32_t epoch) {
  const hipMemcpyKind kind = src_on_host ? hipMemcpyHostToDevice : hipMemcpyDeviceToDeviceNoCU;
  const bool drop = h->dbg.arrival_drop_flags != 0;
  const int64_t H = h->hidden, T = h->T;
  auto flag = [&](int c) {
    hipError_t e = hipStreamWriteValue32(h->copy_stream, h->ready + c, epoch, 0);
    return e == hipSuccess ? UB_OK : hip_fail(h, e, "hipStreamWriteValue32(arrival flag)");
  };
  ub_status_t st;
  if (m.local >= 0 && (st = flag(m.local)) != UB_OK) return st;
  for (const ub_plan_unit_t& u : h->plan.units) {
    for (int c = m.first(u.unit); c < m.last(u.unit); ++c) {
      if (c == m.local) continue;
      const int64_t r0 = m.row0(T, c), rows = m.row0(T, c + 1) - r0;
      if (rows > 0) {
        hipError_t e = hipMemcpyAsync(h->ub + r0 * H, src + r0 * H,
                                      static_cast<size_t>(rows * H) * 2, kind, h->copy_stream);
        if (e != hipSuccess) return hip_fail(h, e, "arrival copy");
      }
      if (!drop && (st = flag(c)) != UB_OK) return st;
    }
  }
  return UB_OK;
}

ub_status_t check_arrival(ub_ctx* h, const void* src, int src_on_host,
                          const ub_overlap_cfg_t* cfg) {
  if (!src || !aligned16(src)) return fail(h, UB_ERR_INVALID_ARG, "src must be 16-byte aligned");
  if (cfg->atomic_gemm && !src_on_host && !cfg->use_ce)
    return fail(h, UB_ERR_UNSUPPORTED,
                "the device-side chunk loop gates on SDMA deliveries only (use_ce=1 or a host "
                "source): the runtime's copy kernel would need CUs that waiting tiles hold");
  const ChunkMap m = chunk_map(h, cfg);
  if (m.n > kMaxArrivalChunks)
    return fail(h, UB_ERR_UNSUPPORTED, "at most %d chunks can be delivered", kMaxArrivalChunks);
  return UB_OK;
}

// Body of both all-gather-side entry points.  src == nullptr: the UB prefix is already
// complete.  Otherwise the non-local chunks are delivered from src while the units run,
// each unit waiting for the arrival of its own chunks.
ub_status_t ag_call(ub_ctx* h, const void* src, int src_on_host, const void* w, int64_t n_cols,
                    int64_t ldw, void* c, int64_t ldc, const ub_overlap_cfg_t* cfg,
                    ub_stream_t stream) {
  if (!h) return UB_ERR_NOT_INITIALIZED;
  ub_status_t st = need_dtype(h, UB_DTYPE_BF16, "this all-gather GEMM");
  if (st != UB_OK) return st;
  st = check_ag_call(h, w, n_cols, ldw, c, ldc, cfg);
  if (st != UB_OK) return st;
  if (src && (st = check_arrival(h, src, src_on_host, cfg)) != UB_OK) return st;
  const int64_t H = h->hidden;
  hipStream_t caller = static_cast<hipStream_t>(stream);
  h->last_plan = ubx::TilePlanRecord{};

  if (cfg->atomic_gemm) {
    // One launch walks every unit in plan order on the caller's stream.
    ubx::GemmUnits units;
    if ((st = plan_units(h, &units)) != UB_OK) return st;
    if ((st = ensure_device(h, 1)) != UB_OK) return st;
    ubx::GemmArgs g{};
    g.dbg = &h->dbg;
    g.plan_out = &h->last_plan;
    g.a = h->ub;
    g.lda = H;
    g.b = static_cast<const uint16_t*>(w);
    g.ldb = ldw;
    g.c = static_cast<uint16_t*>(c);
    g.ldc = ldc;
    g.n = static_cast<int32_t>(n_cols);
    g.k = static_cast<int32_t>(H);
    g.batch = 1;
    g.concurrency = 1;
    set_segmentation(h, g, ag_segmentation(h, n_cols), 0, 0, 1);
    if (src) {
      const ChunkMap m = chunk_map(h, cfg);
      if ((st = ensure_ready_slot(h)) != UB_OK) return st;
      const uint32_t epoch = next_epoch();
      if ((st = start_deliveries(h, m.n, caller)) != UB_OK) return st;
      if ((st = deliver_flagged(h, static_cast<const uint16_t*>(src), src_on_host, cfg, m,
                                epoch)) != UB_OK)
        return st;
      g.ready = h->ready;
      g.epoch = epoch;
      g.timeouts = h->ready + ubx::kReadyTimeoutWord;
      g.wait_ticks = arrival_wait_ticks(h);
      g.n_chunks = m.n;
      for (int c = 0; c <= m.n; ++c) g.chunk_row0[c] = static_cast<int32_t>(m.row0(h->T, c));
    }
    const double flops = 2.0 * h->T * H * n_cols;
    const double bytes = 2.0 * (h->T * H + H * n_cols + h->T * n_cols);
    st = timed_launch(h, caller, 0, flops, bytes,
                      [&] { return ubx::launch_gemm_bf16_units(g, units, caller); },
                      "GEMM launch");
    if (st != UB_OK) return st;
    return src ? join_deliveries(h, caller) : UB_OK;
  }

  const int S = h->plan.n_streams;
  if ((st = ensure_device(h, S)) != UB_OK) return st;
  const ChunkMap m = chunk_map(h, cfg);
  const ubx::SegPlan sp = ag_segmentation(h, n_cols);
  if (src && (st = start_deliveries(h, m.n, caller)) != UB_OK) return st;
  if ((st = fork_streams(h, caller, S)) != UB_OK) return st;
  // With deliveries, each unit's copies are issued just before its GEMM, in plan order, so
  // that no GEMM is enqueued behind copies it does not need (streams may share hardware
  // queues).
  for (const ub_plan_unit_t& u : h->plan.units) {
    if (src && (st = deliver_unit(h, static_cast<const uint16_t*>(src), src_on_host, cfg, m, u)) !=
                   UB_OK)
      return st;
    const int64_t rows = u.row1 - u.row0;
    if (rows <= 0) continue;
    if (rows > kMaxRowsPerUnit) return fail(h, UB_ERR_UNSUPPORTED, "unit too large");
    hipStream_t s = u.stream == 0 ? caller : h->streams[u.stream];
    if (src) {
      for (int ch = m.first(u.unit); ch < m.last(u.unit); ++ch) {
        if (ch == m.local) continue;
        hipError_t e = hipStreamWaitEvent(s, h->ev_arrive[ch], 0);
        if (e != hipSuccess) return hip_fail(h, e, "hipStreamWaitEvent(arrival)");
      }
    }
    ubx::GemmArgs g{};
    g.dbg = &h->dbg;
    g.plan_out = &h->last_plan;
    g.a = h->ub + u.row0 * H;  // byte offset row0 * hidden * 2 into the capacity buffer
    g.lda = H;
    g.b = static_cast<const uint16_t*>(w);
    g.ldb = ldw;
    g.c = static_cast<uint16_t*>(c) + u.row0 * ldc;
    g.ldc = ldc;
    g.m = static_cast<int32_t>(rows);
    g.n = static_cast<int32_t>(n_cols);
    g.k = static_cast<int32_t>(H);
    g.batch = 1;
    g.concurrency = S;
    set_segmentation(h, g, sp, u.row0, u.stream, S);
    const double flops = 2.0 * rows * H * n_cols;
    const double bytes = 2.0 * (rows * H + H * n_cols + rows * n_cols);
    st = timed_launch(h, s, 0, flops, bytes, [&] { return ubx::launch_gemm_bf16(g, s); },
                      "GEMM launch");
    if (st != UB_OK) return st;
  }
  // every chunk was consumed by a unit; join the copy stream all the same
  if (src && (st = join_deliveries(h, caller)) != UB_OK) return st;
  return join_streams(h, caller, S);
}

}  // namespace

UB_API ub_status_t ub_gemm_ag_chunked(ub_handle_t h, const void* w, int64_t n_cols, int64_t ldw,
                                      void* c, int64_t ldc, const ub_overlap_cfg_t* cfg,
                                      ub_stream_t stream) {
  const TraceRange range("ub_gemm_ag_chunked");
  return ag_call(h, nullptr, 0, w, n_cols, ldw, c, ldc, cfg, stream);
}

UB_API ub_status_t ub_gemm_ag_arrival(ub_handle_t h, const void* src, int32_t src_on_host,
                                      const void* w, int64_t n_cols, int64_t ldw, void* c,
                                      int64_t ldc, const ub_overlap_cfg_t* cfg,
                                      ub_stream_t stream) {
  const TraceRange range("ub_gemm_ag_arrival");
  if (!h) return UB_ERR_NOT_INITIALIZED;
  if (!src) return fail(h, UB_ERR_INVALID_ARG, "src is NULL");
  return ag_call(h, src, src_on_host != 0, w, n_cols, ldw, c, ldc, cfg, stream);
}

UB_API ub_status_t ub_deliver_chunks(ub_handle_t h, const void* src, int32_t src_on_host,
                                     const ub_overlap_cfg_t* cfg, ub_stream_t stream) {
  const TraceRange range("ub_deliver_chunks");
  if (!h) return UB_ERR_NOT_INITIALIZED;
  ub_status_t st = need_dtype(h, UB_DTYPE_BF16, "ub_deliver_chunks");
  if (st != UB_OK) return st;
  if ((st = check_cfg_common(h, cfg)) != UB_OK) return st;
  if ((st = check_arrival(h, src, src_on_host != 0, cfg)) != UB_OK) return st;
  if ((st = ubx::build_plan(h->T, h->tp, *cfg, UB_OP_AG, &h->plan, &h->last_error)) != UB_OK)
    return st;
  if ((st = ensure_device(h, 1)) != UB_OK) return st;
  hipStream_t caller = static_cast<hipStream_t>(stream);
  const ChunkMap m = chunk_map(h, cfg);
  if ((st = start_deliveries(h, m.n, caller)) != UB_OK) return st;
  for (const ub_plan_unit_t& u : h->plan.units)
    if ((st = deliver_unit(h, static_cast<const uint16_t*>(src), src_on_host != 0, cfg, m, u)) !=
        UB_OK)
      return st;
  return join_deliveries(h, caller);
}

UB_API ub_status_t ub_quantize_in(ub_handle_t h, const void* src, int64_t rows,
                                  int64_t row_offset, float scale, ub_stream_t stream) {
  const TraceRange range("ub_quantize_in");
  if (!h) return UB_ERR_NOT_INITIALIZED;
  ub_status_t st = need_dtype(h, UB_DTYPE_FP8_E4M3, "ub_quantize_in");
  if (st != UB_OK) return st;
  if (!src || !aligned16(src)) return fail(h, UB_ERR_INVALID_ARG, "src must be 16-byte aligned");
  if (!std::isfinite(scale)) return fail(h, UB_ERR_INVALID_ARG, "scale must be finite");
  if (rows < 0 || row_offset < 0 || row_offset + rows > h->T)
    return fail(h, UB_ERR_INVALID_ARG,
                "quantizing %lld rows at row %lld does not fit the active T=%lld",
                (long long)rows, (long long)row_offset, (long long)h->T);
  if (rows == 0) return UB_OK;
  if ((st = ensure_device(h, 1)) != UB_OK) return st;
  const int64_t H = h->hidden;
  hipError_t e = ubx::launch_quantize_e4m3(static_cast<const uint16_t*>(src), H,
                                           h->ub8 + row_offset * H, H, rows, H, scale,
                                           static_cast<hipStream_t>(stream));
  return e == hipSuccess ? UB_OK : hip_fail(h, e, "quantize launch");
}

UB_API ub_status_t ub_quantize_e4m3(const void* src, int64_t lds, void* dst, int64_t ldd,
                                    int64_t rows, int64_t cols, float scale, ub_stream_t stream) {
  if (!src || !dst || !aligned16(src) || !aligned16(dst)) return UB_ERR_INVALID_ARG;
  if (rows < 0 || cols < 0 || cols % 8 != 0 || lds % 8 != 0 || ldd % 8 != 0 || lds < cols ||
      ldd < cols || !std::isfinite(scale))
    return UB_ERR_INVALID_ARG;
  if (rows == 0 || cols == 0) return UB_OK;
  hipError_t e = ubx::launch_quantize_e4m3(static_cast<const uint16_t*>(src), lds,
                                           static_cast<uint8_t*>(dst), ldd, rows, cols, scale,
                                           static_cast<hipStream_t>(stream));
  return e == hipSuccess ? UB_OK : UB_ERR_HIP;
}

UB_API ub_status_t ub_gemm_ag_chunked_fp8(ub_handle_t h, const void* w, int64_t n_cols,
                                          int64_t ldw, float scale_inv_a, float scale_inv_w,
                                          void* c, int64_t ldc, const ub_overlap_cfg_t* cfg,
                                          ub_stream_t stream) {
  const TraceRange range("ub_gemm_ag_chunked_fp8");
  if (!h) return UB_ERR_NOT_INITIALIZED;
  ub_status_t st = need_dtype(h, UB_DTYPE_FP8_E4M3, "ub_gemm_ag_chunked_fp8");
  if (st != UB_OK) return st;
  if ((st = check_cfg_common(h, cfg)) != UB_OK) return st;
  const int64_t H = h->hidden;
  if (!w || !c || !aligned16(w) || !aligned16(c))
    return fail(h, UB_ERR_INVALID_ARG, "w and c must be non-NULL and 16-byte aligned");
  if (n_cols <= 0 || n_cols % 8 != 0 || n_cols > INT32_MAX)
    return fail(h, UB_ERR_INVALID_ARG, "n_cols=%lld must be > 0 and a multiple of 8",
                (long long)n_cols);
  if (ldw < H || ldw % 16 != 0)
    return fail(h, UB_ERR_INVALID_ARG, "ldw=%lld must be >= hidden=%lld and a multiple of 16",
                (long long)ldw, (long long)H);
  if ((st = check_ld(h, "ldc", ldc, n_cols)) != UB_OK) return st;
  if (!std::isfinite(scale_inv_a) || !std::isfinite(scale_inv_w))
    return fail(h, UB_ERR_INVALID_ARG, "scales must be finite");
  if (H % ubx::kGemmF8KStep != 0)
    return fail(h, UB_ERR_UNSUPPORTED, "hidden=%lld must be a multiple of %d", (long long)H,
                ubx::kGemmF8KStep);
  if ((st = check_forced_tile(h, true)) != UB_OK) return st;
  h->last_plan = ubx::TilePlanRecord{};
  ubx::GemmF8Args g{};
  g.dbg = &h->dbg;
  g.plan_out = &h->last_plan;
  g.a = h->ub8;
  g.lda = H;
  g.b = static_cast<const uint8_t*>(w);
  g.ldb = ldw;
  g.c = static_cast<uint16_t*>(c);
  g.ldc = ldc;
  g.n = static_cast<int32_t>(n_cols);
  g.k = static_cast<int32_t>(H);
  g.scale = scale_inv_a * scale_inv_w;  // one fp32 product
  if (!ubx::gemm_fp8_shape_supported(g)) return fail(h, UB_ERR_UNSUPPORTED, "ldw too large");
  if ((st = ubx::build_plan(h->T, h->tp, *cfg, UB_OP_AG, &h->plan, &h->last_error)) != UB_OK)
    return st;
  hipStream_t caller = static_cast<hipStream_t>(stream);
  if (cfg->atomic_gemm) {
    ubx::GemmUnits units;
    if ((st = plan_units(h, &units)) != UB_OK) return st;
    if ((st = ensure_device(h, 1)) != UB_OK) return st;
    g.concurrency = 1;
    return timed_launch(h, caller, 0, 2.0 * h->T * H * n_cols,
                        double(h->T * H + H * n_cols + 2 * h->T * n_cols),
                        [&] { return ubx::launch_gemm_fp8_units(g, units, caller); },
                        "fp8 GEMM launch");
  }
  const int S = h->plan.n_streams;
  if ((st = ensure_device(h, S)) != UB_OK) return st;
  if ((st = fork_streams(h, caller, S)) != UB_OK) return st;
  g.concurrency = S;
  for (const ub_plan_unit_t& u : h->plan.units) {
    const int64_t rows = u.row1 - u.row0;
    if (rows <= 0) continue;
    if (rows > kMaxRowsPerUnit) return fail(h, UB_ERR_UNSUPPORTED, "unit too large");
    hipStream_t s = u.stream == 0 ? caller : h->streams[u.stream];
    ubx::GemmUnits one;
    one.n = 1;
    one.row0[0] = static_cast<int32_t>(u.row0);
    one.rows[0] = static_cast<int32_t>(rows);
    st = timed_launch(h, s, 0, 2.0 * rows * H * n_cols,
                      double(rows * H + H * n_cols + 2 * rows * n_cols),
                      [&] { return ubx::launch_gemm_fp8_units(g, one, s); }, "fp8 GEMM launch");
    if (st != UB_OK) return st;
  }
  return join_streams(h, caller, S);
}

namespace {

// Where a reduce-scatter call puts its partial slots (tp slots of T x hidden, packed from
// the active T) and its fused-sum tile counters (all of them, and each compute stream's
// range): the registered workspace, or the fixed scratch of ub_gemm_rs_chunked_noalloc.
struct RsTarget {
  uint16_t* ws;
  uint32_t* counters;
  int64_t counters_n;
  int64_t stream_words;
};

// Checks of a bf16 reduce-scatter call, before any HIP call; builds the plan.
ub_status_t check_rs_call(ub_ctx* h, const void* a, int64_t k, int64_t lda, const void* w,
                          int64_t ldw, const void* out, int64_t ldo, const ub_overlap_cfg_t* cfg,
                          bool need_ws) {
  ub_status_t st = need_dtype(h, UB_DTYPE_BF16, "the reduce-scatter GEMM");
  if (st != UB_OK) return st;
  if ((st = check_cfg_common(h, cfg)) != UB_OK) return st;
  if (need_ws && !h->ws)
    return fail(h, UB_ERR_NOT_INITIALIZED, "no reduce-scatter workspace registered");
  if (!a || !w || !out) return fail(h, UB_ERR_INVALID_ARG, "a, w and out must be non-NULL");
  if (!aligned16(a) || !aligned16(w) || !aligned16(out))
    return fail(h, UB_ERR_INVALID_ARG, "a, w and out must be 16-byte aligned");
  if (k <= 0 || k % h->tp != 0 || k > INT32_MAX)
    return fail(h, UB_ERR_INVALID_ARG, "k=%lld must be > 0 and divisible by tp_size %d",
                (long long)k, h->tp);
  const int64_t ks = k / h->tp;
  if (ks % ubx::kGemmKStep != 0)
    return fail(h, UB_ERR_UNSUPPORTED, "k / tp_size = %lld must be a multiple of %d",
                (long long)ks, ubx::kGemmKStep);
  if ((st = check_forced_tile(h, false)) != UB_OK) return st;
  const int64_t H = h->hidden;
  if ((st = check_ld(h, "lda", lda, k)) != UB_OK) return st;
  if ((st = check_ld(h, "ldw", ldw, H)) != UB_OK) return st;
  if ((st = check_ld(h, "ldo", ldo, H)) != UB_OK) return st;
  return ubx::build_plan(h->T, h->tp, *cfg, UB_OP_RS, &h->plan, &h->last_error);
}

// Body of both bf16 reduce-scatter entry points, after check_rs_call.
// Rows [lo, hi) of the units, in the same order (empty pieces dropped).
ubx::GemmUnits clip_rows(const ubx::GemmUnits& u, int64_t lo, int64_t hi) {
  ubx::GemmUnits out;
  out.n = 0;
  for (int i = 0; i < u.n; ++i) {
    const int64_t r0 = std::max<int64_t>(u.row0[i], lo);
    const int64_t r1 = std::min<int64_t>((int64_t)u.row0[i] + u.rows[i], hi);
    if (r1 <= r0) continue;
    out.row0[out.n] = static_cast<int32_t>(r0);
    out.rows[out.n] = static_cast<int32_t>(r1 - r0);
    ++out.n;
  }
  return out;
}

// Row pieces of the pipelined device-side reduce-scatter: piece p's slice GEMMs run on the
// caller's stream, then its reduction on worker stream 1 while the next piece's GEMMs run.
// Cuts fall on multiples of 1280 rows (whole bands of the 256- and 320-row tiles), as near
// to p T / P as that allows; returns the number of pieces (cuts[0] = 0, cuts[n] = T).
int rs_cuts(int64_t T, int P, int64_t* cuts) {
  constexpr int64_t kBand = 1280;
  int n = 0;
  cuts[0] = 0;
  for (int p = 1; p < P; ++p) {
    const int64_t c = (T * p / P + kBand / 2) / kBand * kBand;
    if (c > cuts[n] && c < T) cuts[++n] = c;
  }
  cuts[++n] = T;
  return n;
}

// Pieces of the device-side reduce-scatter at the active T: forced by the debug settings,
// else 1 (one launch of every slice GEMM, then one reduction).
int rs_pieces(const ub_ctx* h) {
  if (h->dbg.rs_pieces > 0) return h->dbg.rs_pieces;
  return 1;
}

ub_status_t rs_call(ub_ctx* h, const RsTarget& tg, const void* a, int64_t k, int64_t lda,
                    const void* w, int64_t ldw, void* out, int64_t ldo,
                    const ub_overlap_cfg_t* cfg, hipStream_t caller) {
  ub_status_t st;
  const int64_t H = h->hidden;
  const int64_t ks = k / h->tp;
  const int64_t T = h->T;
  const int32_t tp = h->tp;
  const bool ring = cfg->reduce_order == UB_REDUCE_RING;
  const bool fuse = cfg->fuse_reduce != 0;
  h->last_plan = ubx::TilePlanRecord{};
  // Fused reduction: each compute stream's launches run one after another and leave
  // their counters at zero, so each stream counts in its own range; the device-side loop
  // uses the whole array.
  auto set_fuse = [&](ubx::GemmArgs& g, int64_t row0, int stream_index) {
    if (!fuse) return;
    g.fuse_out = static_cast<uint16_t*>(out) + row0 * ldo;
    g.fuse_ldo = ldo;
    g.fuse_nslots = tp;
    g.fuse_ring = ring;
    g.fuse_row0 = row0;
    g.fuse_shard_rows = T / tp;
    if (stream_index < 0) {
      g.counters = tg.counters;
      g.counters_n = tg.counters_n;
    } else {
      g.counters = tg.counters + stream_index * tg.stream_words;
      g.counters_n = tg.stream_words;
    }
  };
  const double fused_flops = double(tp - 1) * H;  // per row: the reduction's adds
  const double fused_bytes = 2.0 * (tp + 1) * H;  // per row: the reduction's reads and write

  if (cfg->atomic_gemm) {
    // One launch computes every unit's tp slice partials in plan order, then one
    // reduction sums the whole active prefix (or the launch's tiles sum them).
    ubx::GemmUnits units;
    if ((st = plan_units(h, &units)) != UB_OK) return st;
    if ((st = ensure_device(h, 1)) != UB_OK) return st;
    ubx::GemmArgs g{};
    g.dbg = &h->dbg;
    g.plan_out = &h->last_plan;
    g.a = static_cast<const uint16_t*>(a);
    g.lda = lda;
    g.a_batch_stride = ks;
    g.b = static_cast<const uint16_t*>(w);
    g.ldb = ldw;
    g.b_batch_stride = ks * ldw;
    g.c = tg.ws;
    g.ldc = H;
    g.c_batch_stride = T * H;
    g.n = static_cast<int32_t>(H);
    g.k = static_cast<int32_t>(ks);
    g.batch = tp;
    g.concurrency = 1;
    set_fuse(g, 0, -1);
    int64_t cuts[kMaxRsPieces + 1];
    const int np = fuse ? 1 : rs_cuts(T, rs_pieces(h), cuts);
    if (np <= 1) {
      st = timed_launch(h, caller, 0, 2.0 * T * k * H + (fuse ? fused_flops * T : 0.0),
                        2.0 * (T * k + k * H + tp * T * H) + (fuse ? fused_bytes * T : 0.0),
                        [&] { return ubx::launch_gemm_bf16_units(g, units, caller); },
                        "slice GEMM launch");
      if (st != UB_OK || fuse) return st;
      const ubx::ReduceArgs r = reduce_args(h, 0, T, out, ldo, ring, tg.ws);
      return timed_launch(h, caller, 1, double(tp - 1) * T * H, 2.0 * (tp + 1) * T * H,
                          [&] { return ubx::launch_reduce_partials(r, caller); }, "reduce launch");
    }
    // pipelined: piece p's GEMMs on the caller's stream, its reduction on worker stream 1
    // after an event, overlapping piece p + 1's GEMMs; the caller joins stream 1 at the end
    if ((st = ensure_device(h, 2)) != UB_OK) return st;
    hipStream_t rs = h->streams[1];
    h->last_plan.rs_pieces = np;
    for (int p = 0; p < np; ++p) {
      const int64_t lo = cuts[p], rows = cuts[p + 1] - cuts[p];
      const ubx::GemmUnits pu = clip_rows(units, lo, cuts[p + 1]);
      st = timed_launch(h, caller, 0, 2.0 * rows * k * H, 2.0 * (rows * k + k * H + tp * rows * H),
                        [&] { return ubx::launch_gemm_bf16_units(g, pu, caller); },
                        "slice GEMM launch");
      if (st != UB_OK) return st;
      hipError_t e = hipEventRecord(h->ev_piece[p], caller);
      if (e == hipSuccess) e = hipStreamWaitEvent(rs, h->ev_piece[p], 0);
      if (e != hipSuccess) return hip_fail(h, e, "piece event");
      const ubx::ReduceArgs r = reduce_args(h, lo, rows, out, ldo, ring, tg.ws);
      st = timed_launch(h, rs, 1, double(tp - 1) * rows * H, 2.0 * (tp + 1) * rows * H,
                        [&] { return ubx::launch_reduce_partials(r, rs); }, "reduce launch");
      if (st != UB_OK) return st;
    }
    return join_streams(h, caller, 2);
  }

  const int S = h->plan.n_streams;
  if ((st = ensure_device(h, S)) != UB_OK) return st;
  if ((st = fork_streams(h, caller, S)) != UB_OK) return st;
  for (size_t ui = 0; ui < h->plan.units.size(); ++ui) {
    const ub_plan_unit_t& u = h->plan.units[ui];
    const int64_t rows = u.row1 - u.row0;
    if (rows <= 0) continue;
    if (rows > kMaxRowsPerUnit) return fail(h, UB_ERR_UNSUPPORTED, "unit too large");
    hipStream_t s = u.stream == 0 ? caller : h->streams[u.stream];
    // tp slice GEMMs of this chunk in one batched launch; slot s of the packed active
    // prefix starts at workspace element s*T*H (offsets from the active T).
    ubx::GemmArgs g{};
    g.dbg = &h->dbg;
    g.plan_out = &h->last_plan;
    g.a = static_cast<const uint16_t*>(a) + u.row0 * lda;
    g.lda = lda;
    g.a_batch_stride = ks;
    g.b = static_cast<const uint16_t*>(w);
    g.ldb = ldw;
    g.b_batch_stride = ks * ldw;
    g.c = tg.ws + u.row0 * H;
    g.ldc = H;
    g.c_batch_stride = T * H;
    g.m = static_cast<int32_t>(rows);
    g.n = static_cast<int32_t>(H);
    g.k = static_cast<int32_t>(ks);
    g.batch = tp;
    g.concurrency = S;
    if (fuse) set_fuse(g, u.row0, u.stream);
    const double flops = 2.0 * rows * k * H + (fuse ? fused_flops * rows : 0.0);
    const double gbytes = 2.0 * (rows * k + k * H + tp * rows * H) + (fuse ? fused_bytes * rows : 0.0);
    st = timed_launch(h, s, 0, flops, gbytes, [&] { return ubx::launch_gemm_bf16(g, s); },
                      "slice GEMM launch");
    if (st != UB_OK) return st;
    if (fuse) continue;
    // the reduction of this chunk follows its GEMMs on the same stream
    const ubx::ReduceArgs r = reduce_args(h, u.row0, rows, out, ldo, ring, tg.ws);
    const double rbytes = 2.0 * (tp + 1) * rows * H;
    st = timed_launch(h, s, 1, double(tp - 1) * rows * H, rbytes,
                      [&] { return ubx::launch_reduce_partials(r, s); }, "reduce launch");
    if (st != UB_OK) return st;
  }
  return join_streams(h, caller, S);
}

}  // namespace

UB_API ub_status_t ub_gemm_rs_chunked(ub_handle_t h, const void* a, int64_t k, int64_t lda,
                                      const void* w, int64_t ldw, void* out, int64_t ldo,
                                      const ub_overlap_cfg_t* cfg, ub_stream_t stream) {
  const TraceRange range("ub_gemm_rs_chunked");
  if (!h) return UB_ERR_NOT_INITIALIZED;
  ub_status_t st = check_rs_call(h, a, k, lda, w, ldw, out, ldo, cfg, true);
  if (st != UB_OK) return st;
  const RsTarget tg{h->ws, h->fuse_counters, h->fuse_counters_n,
                    ubx::fuse_counter_stream_words(h->capacity, h->hidden)};
  return rs_call(h, tg, a, k, lda, w, ldw, out, ldo, cfg, static_cast<hipStream_t>(stream));
}

UB_API ub_status_t ub_gemm_rs_chunked_noalloc(ub_handle_t h, const void* a, int64_t k,
                                              int64_t lda, const void* w, int64_t ldw, void* out,
                                              int64_t ldo, const ub_overlap_cfg_t* cfg,
                                              ub_stream_t stream) {
  const TraceRange range("ub_gemm_rs_chunked_noalloc");
  if (!h) return UB_ERR_NOT_INITIALIZED;
  ub_status_t st = check_rs_call(h, a, k, lda, w, ldw, out, ldo, cfg, false);
  if (st != UB_OK) return st;
  // the workspace's layout, sized for the active T, in the fixed scratch
  const int64_t T = h->T, H = h->hidden;
  const size_t parts = static_cast<size_t>(h->tp) * static_cast<size_t>(T * H) * 2;
  const size_t counter_off = (parts + 255) / 256 * 256;
  const int64_t words = cfg->fuse_reduce ? ubx::fuse_counter_words(T, H) : 0;
  const size_t need = counter_off + static_cast<size_t>(words) * sizeof(uint32_t);
  if (need > ubx::kStaticScratchBytes)
    return fail(h, UB_ERR_BUFFER_TOO_SMALL,
                "this call needs %zu bytes of scratch (tp * T * hidden bf16 partials%s); the "
                "fixed scratch holds %zu",
                need, cfg->fuse_reduce ? " and fused-sum counters" : "", ubx::kStaticScratchBytes);
  if ((st = ensure_device(h, 1)) != UB_OK) return st;
  hipError_t e = hipSuccess;
  unsigned char* base = ubx::static_scratch_base(&e);
  if (!base) return hip_fail(h, e, "hipGetSymbolAddress(static scratch)");
  hipStream_t caller = static_cast<hipStream_t>(stream);
  uint32_t* counters = reinterpret_cast<uint32_t*>(base + counter_off);
  if (words > 0) {  // another call may have left the shared array in any state
    e = ubx::launch_clear_words(counters, words, caller);
    if (e != hipSuccess) return hip_fail(h, e, "scratch counter clear");
  }
  const RsTarget tg{reinterpret_cast<uint16_t*>(base), counters, words,
                    ubx::fuse_counter_stream_words(T, H)};
  return rs_call(h, tg, a, k, lda, w, ldw, out, ldo, cfg, caller);
}

UB_API ub_status_t ub_gemm_rs_chunked_fp8(ub_handle_t h, const void* a, int64_t k, int64_t lda,
                                          const void* w, int64_t ldw, float scale_inv_a,
                                          float scale_inv_w, void* out, int64_t ldo,
                                          const ub_overlap_cfg_t* cfg, ub_stream_t stream) {
  const TraceRange range("ub_gemm_rs_chunked_fp8");
  if (!h) return UB_ERR_NOT_INITIALIZED;
  ub_status_t st = need_dtype(h, UB_DTYPE_BF16, "the reduce-scatter GEMM (bf16 partials)");
  if (st != UB_OK) return st;
  if ((st = check_cfg_common(h, cfg)) != UB_OK) return st;
  if (cfg->fuse_reduce)
    return fail(h, UB_ERR_UNSUPPORTED, "fuse_reduce is implemented for bf16 operands only");
  if (!h->ws) return fail(h, UB_ERR_NOT_INITIALIZED, "no reduce-scatter workspace registered");
  if (!a || !w || !out) return fail(h, UB_ERR_INVALID_ARG, "a, w and out must be non-NULL");
  if (!aligned16(a) || !aligned16(w) || !aligned16(out))
    return fail(h, UB_ERR_INVALID_ARG, "a, w and out must be 16-byte aligned");
  if (k <= 0 || k % h->tp != 0 || k > INT32_MAX)
    return fail(h, UB_ERR_INVALID_ARG, "k=%lld must be > 0 and divisible by tp_size %d",
                (long long)k, h->tp);
  const int64_t ks = k / h->tp;
  if (ks % ubx::kGemmF8KStep != 0)
    return fail(h, UB_ERR_UNSUPPORTED, "k / tp_size = %lld must be a multiple of %d",
                (long long)ks, ubx::kGemmF8KStep);
  if ((st = check_forced_tile(h, true)) != UB_OK) return st;
  const int64_t H = h->hidden;
  if (lda < k || lda % 16 != 0)
    return fail(h, UB_ERR_INVALID_ARG, "lda=%lld must be >= k=%lld and a multiple of 16",
                (long long)lda, (long long)k);
  if (ldw < k || ldw % 16 != 0)
    return fail(h, UB_ERR_INVALID_ARG, "ldw=%lld must be >= k=%lld and a multiple of 16",
                (long long)ldw, (long long)k);
  if ((st = check_ld(h, "ldo", ldo, H)) != UB_OK) return st;
  if (!std::isfinite(scale_inv_a) || !std::isfinite(scale_inv_w))
    return fail(h, UB_ERR_INVALID_ARG, "scales must be finite");
  const int64_t T = h->T;
  const int32_t tp = h->tp;
  // slice s: columns [s*ks, (s+1)*ks) of A's rows and of W's rows; partial s at workspace
  // element s*T*H (offsets from the active T)
  h->last_plan = ubx::TilePlanRecord{};
  ubx::GemmF8Args g{};
  g.dbg = &h->dbg;
  g.plan_out = &h->last_plan;
  g.a = static_cast<const uint8_t*>(a);
  g.lda = lda;
  g.a_batch_stride = ks;
  g.b = static_cast<const uint8_t*>(w);
  g.ldb = ldw;
  g.b_batch_stride = ks;
  g.c = h->ws;
  g.ldc = H;
  g.c_batch_stride = T * H;
  g.n = static_cast<int32_t>(H);
  g.k = static_cast<int32_t>(ks);
  g.batch = tp;
  g.scale = scale_inv_a * scale_inv_w;  // one fp32 product
  if (!ubx::gemm_fp8_shape_supported(g))
    return fail(h, UB_ERR_UNSUPPORTED, "lda or ldw too large");
  st = ubx::build_plan(T, tp, *cfg, UB_OP_RS, &h->plan, &h->last_error);
  if (st != UB_OK) return st;
  hipStream_t caller = static_cast<hipStream_t>(stream);
  const bool ring = cfg->reduce_order == UB_REDUCE_RING;

  if (cfg->atomic_gemm) {
    ubx::GemmUnits units;
    if ((st = plan_units(h, &units)) != UB_OK) return st;
    if ((st = ensure_device(h, 1)) != UB_OK) return st;
    g.concurrency = 1;
    int64_t cuts[kMaxRsPieces + 1];
    const int np = rs_cuts(T, rs_pieces(h), cuts);
    if (np <= 1) {
      st = timed_launch(h, caller, 0, 2.0 * T * k * H, double(T * k + k * H + 2 * tp * T * H),
                        [&] { return ubx::launch_gemm_fp8_units(g, units, caller); },
                        "fp8 slice GEMM launch");
      if (st != UB_OK) return st;
      const ubx::ReduceArgs r = reduce_args(h, 0, T, out, ldo, ring);
      return timed_launch(h, caller, 1, double(tp - 1) * T * H, 2.0 * (tp + 1) * T * H,
                          [&] { return ubx::launch_reduce_partials(r, caller); }, "reduce launch");
    }
    // pipelined as the bf16 call: piece p's slice GEMMs on the caller's stream, its
    // reduction on worker stream 1 after an event, overlapping piece p + 1's GEMMs
    if ((st = ensure_device(h, 2)) != UB_OK) return st;
    hipStream_t rs = h->streams[1];
    for (int p = 0; p < np; ++p) {
      const int64_t lo = cuts[p], rows = cuts[p + 1] - cuts[p];
      const ubx::GemmUnits pu = clip_rows(units, lo, cuts[p + 1]);
      st = timed_launch(h, caller, 0, 2.0 * rows * k * H, double(rows * k + k * H + 2 * tp * rows * H),
                        [&] { return ubx::launch_gemm_fp8_units(g, pu, caller); },
                        "fp8 slice GEMM launch");
      if (st != UB_OK) return st;
      hipError_t e = hipEventRecord(h->ev_piece[p], caller);
      if (e == hipSuccess) e = hipStreamWaitEvent(rs, h->ev_piece[p], 0);
      if (e != hipSuccess) return hip_fail(h, e, "piece event");
      const ubx::ReduceArgs r = reduce_args(h, lo, rows, out, ldo, ring);
      st = timed_launch(h, rs, 1, double(tp - 1) * rows * H, 2.0 * (tp + 1) * rows * H,
                        [&] { return ubx::launch_reduce_partials(r, rs); }, "reduce launch");
      if (st != UB_OK) return st;
    }
    h->last_plan.rs_pieces = np;
    return join_streams(h, caller, 2);
  }

  const int S = h->plan.n_streams;
  if ((st = ensure_device(h, S)) != UB_OK) return st;
  if ((st = fork_streams(h, caller, S)) != UB_OK) return st;
  g.concurrency = S;
  for (const ub_plan_unit_t& u : h->plan.units) {
    const int64_t rows = u.row1 - u.row0;
    if (rows <= 0) continue;
    if (rows > kMaxRowsPerUnit) return fail(h, UB_ERR_UNSUPPORTED, "unit too large");
    hipStream_t s = u.stream == 0 ? caller : h->streams[u.stream];
    ubx::GemmUnits one;
    one.n = 1;
    one.row0[0] = static_cast<int32_t>(u.row0);
    one.rows[0] = static_cast<int32_t>(rows);
    st = timed_launch(h, s, 0, 2.0 * rows * k * H, double(rows * k + k * H + 2 * tp * rows * H),
                      [&] { return ubx::launch_gemm_fp8_units(g, one, s); },
                      "fp8 slice GEMM launch");
    if (st != UB_OK) return st;
    const ubx::ReduceArgs r = reduce_args(h, u.row0, rows, out, ldo, ring);
    st = timed_launch(h, s, 1, double(tp - 1) * rows * H, 2.0 * (tp + 1) * rows * H,
                      [&] { return ubx::launch_reduce_partials(r, s); }, "reduce launch");
    if (st != UB_OK) return st;
  }
  return join_streams(h, caller, S);
}

UB_API ub_status_t ub_reduce_partials(ub_handle_t h, void* out, int64_t ldo,
                                      int32_t reduce_order, ub_stream_t stream) {
  const TraceRange range("ub_reduce_partials");
  if (!h) return UB_ERR_NOT_INITIALIZED;
  if (need_dtype(h, UB_DTYPE_BF16, "ub_reduce_partials") != UB_OK) return UB_ERR_DTYPE;
  if (!h->ws) return fail(h, UB_ERR_NOT_INITIALIZED, "no reduce-scatter workspace registered");
  if (!out || !aligned16(out)) return fail(h, UB_ERR_INVALID_ARG, "out must be 16-byte aligned");
  if (reduce_order != UB_REDUCE_ASCENDING && reduce_order != UB_REDUCE_RING)
    return fail(h, UB_ERR_INVALID_ARG, "reduce_order=%d is not a ub_reduce_order_t", reduce_order);
  ub_status_t st = check_ld(h, "ldo", ldo, h->hidden);
  if (st != UB_OK) return st;
  if ((st = ensure_device(h, 1)) != UB_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const ubx::ReduceArgs r = reduce_args(h, 0, h->T, out, ldo, reduce_order == UB_REDUCE_RING);
  const double rbytes = 2.0 * (h->tp + 1) * h->T * h->hidden;
  return timed_launch(h, s, 1, double(h->tp - 1) * h->T * h->hidden, rbytes,
                      [&] { return ubx::launch_reduce_partials(r, s); }, "reduce launch");
}

UB_API ub_status_t ub_set_kernel_timing(ub_handle_t h, int32_t enable) {
  if (!h) return UB_ERR_NOT_INITIALIZED;
  if (enable < 0 || enable > 2)
    return fail(h, UB_ERR_INVALID_ARG, "enable=%d must be 0 (off), 1 (per launch) or 2 (chained)",
                enable);
  clear_chain(h);
  h->timing = enable;
  return UB_OK;
}

UB_API ub_status_t ub_get_kernel_timing(ub_handle_t h, ub_kernel_stats_t* gemm,
                                        ub_kernel_stats_t* reduce) {
  if (!h) return UB_ERR_NOT_INITIALIZED;
  ub_status_t st = harvest(h);
  if (st != UB_OK) return st;
  clear_chain(h);
  if (gemm) *gemm = h->stats[0];
  if (reduce) *reduce = h->stats[1];
  h->stats[0] = ub_kernel_stats_t{};
  h->stats[1] = ub_kernel_stats_t{};
  return UB_OK;
}

UB_API ub_status_t ub_arrival_timeouts(ub_handle_t h, uint32_t* count) {
  if (!h) return UB_ERR_NOT_INITIALIZED;
  if (!count) return fail(h, UB_ERR_INVALID_ARG, "count must be non-NULL");
  *count = 0;
  if (!h->ready) return UB_OK;
  hipError_t e = hipMemcpy(count, h->ready + ubx::kReadyTimeoutWord, sizeof(uint32_t),
                           hipMemcpyDeviceToHost);
  return e == hipSuccess ? UB_OK : hip_fail(h, e, "hipMemcpy(arrival timeouts)");
}

UB_API ub_status_t ub_prepare_streams(ub_handle_t h, int32_t num_max_streams,
                                      int32_t copy_stream) {
  if (!h) return UB_ERR_NOT_INITIALIZED;
  if (num_max_streams < 1)
    return fail(h, UB_ERR_INVALID_ARG, "num_max_streams=%d must be >= 1", num_max_streams);
  ub_status_t st = ensure_device(h, std::min<int32_t>(num_max_streams, UB_MAX_STREAMS));
  if (st != UB_OK || !copy_stream) return st;
  return ensure_arrival(h, 0);
}

UB_API ub_status_t ub_debug_set(ub_handle_t h, const char* key, int64_t value) {
  if (!h) return UB_ERR_NOT_INITIALIZED;
  if (!key) return fail(h, UB_ERR_INVALID_ARG, "key is NULL");
  ubx::DebugOpts& d = h->dbg;
  const std::string k(key);
  if (k == "tile_m" || k == "tile_n") {
    if (value < 0 || value > 4096) return fail(h, UB_ERR_INVALID_ARG, "%s=%lld", key, (long long)value);
    (k == "tile_m" ? d.tile_m : d.tile_n) = static_cast<int32_t>(value);
    return UB_OK;
  }
  if (k == "cut_row") {
    if (value < 0 || value > (int64_t(1) << 31)) return fail(h, UB_ERR_INVALID_ARG, "cut_row=%lld", (long long)value);
    d.cut_row = value;
    return UB_OK;
  }
  if (k == "tail_tile_m" || k == "tail_tile_n") {
    if (value < 0 || value > 4096) return fail(h, UB_ERR_INVALID_ARG, "%s=%lld", key, (long long)value);
    (k == "tail_tile_m" ? d.tail_m : d.tail_n) = static_cast<int32_t>(value);
    return UB_OK;
  }
  if (k == "seg_row") {
    if (value < 0 || value > (int64_t(1) << 31)) return fail(h, UB_ERR_INVALID_ARG, "seg_row=%lld", (long long)value);
    d.seg_row = value;
    return UB_OK;
  }
  if (k == "nseg") {
    if (value < 0 || value > 64) return fail(h, UB_ERR_INVALID_ARG, "nseg=%lld", (long long)value);
    d.nseg = static_cast<int32_t>(value);
    return UB_OK;
  }
  if (k == "rs_pieces") {
    if (value < 0 || value > kMaxRsPieces)
      return fail(h, UB_ERR_INVALID_ARG, "rs_pieces=%lld", (long long)value);
    d.rs_pieces = static_cast<int32_t>(value);
    return UB_OK;
  }
  if (k == "seg_reduce") {
    if (value < 0 || value > 2) return fail(h, UB_ERR_INVALID_ARG, "seg_reduce=%lld", (long long)value);
    d.seg_reduce = static_cast<int32_t>(value);
    return UB_OK;
  }
  if (k == "seg_tile_m" || k == "seg_tile_n") {
    if (value < 0 || value > 1024) return fail(h, UB_ERR_INVALID_ARG, "%s=%lld", key, (long long)value);
    (k == "seg_tile_m" ? d.seg_m : d.seg_n) = static_cast<int32_t>(value);
    return UB_OK;
  }
  if (k == "tile_group") {
    if (value < 0 || value > 4096) return fail(h, UB_ERR_INVALID_ARG, "tile_group=%lld", (long long)value);
    d.tile_group = static_cast<int32_t>(value);
    return UB_OK;
  }
  if (k == "arrival_wait_us") {
    if (value < 0 || value > 60000000) return fail(h, UB_ERR_INVALID_ARG, "arrival_wait_us=%lld", (long long)value);
    d.arrival_wait_us = value;
    return UB_OK;
  }
  if (k == "arrival_drop_flags") {
    if (value != 0 && value != 1) return fail(h, UB_ERR_INVALID_ARG, "arrival_drop_flags=%lld", (long long)value);
    d.arrival_drop_flags = static_cast<int32_t>(value);
    return UB_OK;
  }
  return fail(h, UB_ERR_INVALID_ARG, "unknown debug key '%s'", key);
}

UB_API ub_status_t ub_debug_last_plan(ub_handle_t h, ub_tile_plan_t* out) {
  if (!h) return UB_ERR_NOT_INITIALIZED;
  if (!out) return fail(h, UB_ERR_INVALID_ARG, "out is NULL");
  out->tile_m = h->last_plan.tile_m;
  out->tile_n = h->last_plan.tile_n;
  out->cut_row = h->last_plan.cut;
  out->tail_tile_m = h->last_plan.tail_m;
  out->tail_tile_n = h->last_plan.tail_n;
  out->seg_row = h->last_plan.seg_row;
  out->nseg = h->last_plan.nseg;
  out->split = h->last_plan.split;
  out->seg_tile_m = h->last_plan.seg_m;
  out->seg_tile_n = h->last_plan.seg_n;
  out->dispatches = h->last_plan.dispatches;
  out->rs_pieces = h->last_plan.rs_pieces;
  return UB_OK;
}

UB_API ub_status_t ub_register_scratch(ub_handle_t h, void* buf, size_t bytes) {
  if (!h) return UB_ERR_NOT_INITIALIZED;
  if (!buf && bytes == 0) {  // unregister
    h->split_counters = nullptr;
    h->split_parts = nullptr;
    h->split_counters_n = h->split_parts_n = 0;
    return UB_OK;
  }
  if (!buf || !aligned16(buf)) return fail(h, UB_ERR_INVALID_ARG, "scratch must be 16-byte aligned");
  if (bytes < UB_SCRATCH_MIN_BYTES)
    return fail(h, UB_ERR_BUFFER_TOO_SMALL, "scratch of %zu bytes, at least %d needed", bytes,
                UB_SCRATCH_MIN_BYTES);
  unsigned char* b = static_cast<unsigned char*>(buf);
  h->split_counters = reinterpret_cast<uint32_t*>(b);
  h->split_counters_n = UB_SCRATCH_COUNTER_BYTES / 4;
  h->split_parts = reinterpret_cast<float*>(b + UB_SCRATCH_COUNTER_BYTES);
  h->split_parts_n = static_cast<int64_t>((bytes - UB_SCRATCH_COUNTER_BYTES) / sizeof(float));
  return UB_OK;
}

UB_API ub_status_t ub_destroy(ub_handle_t h) {
  if (!h) return UB_OK;
  if (h->device >= 0) {
    int cur = -1;
    (void)hipGetDevice(&cur);
    if (cur != h->device) (void)hipSetDevice(h->device);
    harvest(h);
    clear_chain(h);
    for (int i = 1; i < h->n_streams_created; ++i) {
      (void)hipStreamSynchronize(h->streams[i]);
      (void)hipStreamDestroy(h->streams[i]);
      (void)hipEventDestroy(h->ev_join[i]);
    }
    if (h->ev_fork) (void)hipEventDestroy(h->ev_fork);
    if (h->copy_stream) {
      (void)hipStreamSynchronize(h->copy_stream);
      (void)hipStreamDestroy(h->copy_stream);
      (void)hipEventDestroy(h->ev_copy_join);
    }
    for (hipEvent_t ev : h->ev_arrive)
      if (ev) (void)hipEventDestroy(ev);
    for (hipEvent_t ev : h->ev_piece)
      if (ev) (void)hipEventDestroy(ev);
    for (hipEvent_t ev : h->free_events) (void)hipEventDestroy(ev);
    if (h->ready) {  // the next handle to take this slot starts with no counted timeouts
      const uint32_t zero = 0;
      (void)hipMemcpy(h->ready + ubx::kReadyTimeoutWord, &zero, sizeof(zero), hipMemcpyHostToDevice);
    }
    if (cur >= 0 && cur != h->device) (void)hipSetDevice(cur);
  }
  release_ready_slot(h);
  delete h;
  return UB_OK;
}

}  // extern "C"
