/*
 * ub.h -- C ABI of the chunked tensor-parallel overlap GEMMs over a capacity UserBuffer,
 * for AMD Instinct MI355X (gfx950).
 *
 * Pages cited by title:
 *   [TE#3564] "[Feature Request] Support dynamic token counts in TP communication/GEMM
 *             overlap" (Transformer Engine issue 3564): "Problem", "Proposed API",
 *             "Implementation approach in the prototype".
 *   [TE#1344] "How to setup TP Overlap configs" (Transformer Engine issue 1344): the
 *             maintainer's option list.
 *   [MLM#1240] "[QUESTION] Do tp overlap support thd, whose sequence length is flexible?"
 *             (Megatron-LM discussion 1240): the QKV and MLP shape diagrams and the
 *             "Why doesn't the hidden dimension appear" answer.
 *
 * What the library does.  A UserBuffer (UB) is registered once at a fixed capacity
 * [capacity, hidden] of bf16 ([TE#3564] "Proposed API"); every microbatch then sets an
 * active shape [T, hidden] whose data is the contiguous prefix of the buffer, and all
 * views, chunk offsets and counts are recomputed from T without any allocation
 * ([TE#3564] "Implementation approach in the prototype").  Two chunked bf16 GEMMs read
 * the buffer by offset:
 *   - the all-gather side: a column-parallel GEMM (QKV, MLP fc1; [MLM#1240] diagrams)
 *     whose input is the gathered activation tensor held in the UB, cut into token
 *     chunks that run in ring, pipeline or bulk order on min(num_splits, num_max_streams)
 *     HIP streams ([TE#1344] "method", "num_splits", "num_max_streams", "aggregate");
 *   - the reduce-scatter side: a row-parallel GEMM (MLP fc2) whose tp K-slice partial
 *     products are written as bf16 into a workspace and summed into tp shards of
 *     [T/tp, hidden] ([MLM#1240] MLP diagram; [TE#3564]: reduce-scatter keeps its extra
 *     per-rank chunks inside its own allocation).
 * One process drives one GPU; the library moves no data between GPUs.  The UB holds what
 * a rank would have after the all-gather; the caller fills its active prefix, or lets
 * ub_gemm_ag_arrival deliver the other ranks' chunks while the chunk GEMMs run.
 * Extensions beyond the pages' first scope: a device-side chunk loop (option
 * atomic_gemm, [TE#1344]), the reduce-scatter sum in ring order with a bf16 rounding per
 * hop (reduce_order), and FP8 (E4M3) UserBuffers on the all-gather side.
 *
 * Conventions for every entry point.
 *   - Tensors are row-major bf16 (2 bytes, IEEE binary32 upper half), or E4M3 codes (1
 *     byte) where an entry point says so.  Device pointers must be 16-byte aligned;
 *     leading dimensions and the hidden size are counted in elements and must be
 *     multiples of 8 (16-byte rows; 16 for fp8).
 *   - Every device buffer is owned by the caller (allocated by PyTorch or hipMalloc) and
 *     must outlive the handle.  The library never allocates, frees or registers device
 *     memory, and no call makes a device-wide wait.  A handle owns only host state and its
 *     HIP streams and events (created by ub_prepare_streams, or on first use;
 *     ub_gemm_ag_arrival adds a copy stream and one event per chunk).  The library's only
 *     device memory of its own is a fixed array of arrival flags in its code object.
 *   - Functions return a ub_status_t; no C++ exception crosses the ABI.  Arguments are
 *     checked before anything is launched; a rejected call changes no state and enqueues
 *     nothing.  ub_last_error() returns a message for the last failure on a handle.
 *   - GEMM calls are asynchronous on the caller's stream: their results are ordered
 *     after work already on `stream` and before work enqueued on it afterwards.  No
 *     host synchronisation happens inside them.  Device faults surface at the caller's
 *     next synchronisation.
 *   - A handle is not thread-safe.  The caller must not modify the UB prefix, the
 *     weights or the outputs while a call that uses them is in flight.
 *   - Rounding: products are accumulated in fp32 (MFMA) and each stored result is
 *     rounded once to bf16, round-to-nearest-even (the reduce-scatter partials once
 *     each, then their sum once, or once per hop in ring order).  An output element
 *     depends only on its own input row and weight column: results are bit-identical
 *     for every chunk count, stream count, order, aggregate setting, atomic_gemm,
 *     capacity and buffer offset.
 */
#ifndef CHUNKED_TP_OVERLAP_AMD_UB_H
#define CHUNKED_TP_OVERLAP_AMD_UB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define UB_API __attribute__((visibility("default")))

/* Largest number of compute streams a handle uses; num_max_streams above it is clamped. */
#define UB_MAX_STREAMS 8
/* Largest tensor-parallel size (number of K slices on the reduce-scatter side). */
#define UB_MAX_TP 64

typedef struct ub_ctx* ub_handle_t;
/* A hipStream_t passed as an opaque pointer; NULL is the device's null stream. */
typedef void* ub_stream_t;

typedef enum {
  UB_OK = 0,
  UB_ERR_INVALID_ARG = 1,       /* null pointer, bad size, misalignment, bad option */
  UB_ERR_NDIM = 2,              /* active shape is not 2-D                    [TE#3564] */
  UB_ERR_ZERO_DIM = 3,          /* active shape has a dimension <= 0          [TE#3564] */
  UB_ERR_CAPACITY = 4,          /* active T exceeds the registered capacity   [TE#3564] */
  UB_ERR_HIDDEN_MISMATCH = 5,   /* active hidden differs from the registered  [TE#3564] */
  UB_ERR_TP_DIVISIBILITY = 6,   /* T (or capacity) not divisible by tp_size   [TE#3564] */
  UB_ERR_DTYPE = 7,             /* not bf16 or fp8 E4M3, or the wrong one for the call */
  UB_ERR_UNSUPPORTED = 8,       /* a valid request the library does not implement */
  UB_ERR_BUFFER_TOO_SMALL = 9,  /* a registered byte size is below what the shape needs */
  UB_ERR_NOT_INITIALIZED = 10,  /* null handle, or a reduce-scatter call without workspace */
  UB_ERR_HIP = 11               /* a HIP runtime call failed; see ub_last_error */
} ub_status_t;

/* Element type of a UserBuffer.  The pages scope the prototype to unquantized 2-byte
 * bf16 buffers and name quantized (FP8) ones as outside that first scope ([TE#3564]
 * "Implementation approach", last paragraph).  UB_DTYPE_BF16 is the main path;
 * UB_DTYPE_FP8_E4M3 is the extension to quantized buffers (OCP E4M3 codes, one byte per
 * element) on the all-gather side: ub_quantize_in, ub_gemm_ag_chunked_fp8.  On the
 * reduce-scatter side the communicated partials stay bf16, so ub_gemm_rs_chunked_fp8
 * takes E4M3 operands on a bf16 handle.  FP16 and E5M2 are rejected with UB_ERR_DTYPE. */
typedef enum {
  UB_DTYPE_BF16 = 0,
  UB_DTYPE_FP16 = 1,
  UB_DTYPE_FP8_E4M3 = 2,
  UB_DTYPE_FP8_E5M2 = 3,
  UB_DTYPE_INT32_RANGE_ = 0x7FFFFFFF /* not a type: any int32 value may be passed and is checked */
} ub_dtype_t;

/* Overlap method ([TE#1344] "method"). */
typedef enum {
  UB_RING_EXCHANGE = 0, /* chunk count forced to tp_size; ring order from `rank` */
  UB_PIPELINE = 1,      /* num_splits chunks in natural order */
  UB_BULK = 2           /* num_splits chunks in natural order */
} ub_method_t;

/* Which side of the overlap a plan describes. */
typedef enum { UB_OP_AG = 0, UB_OP_RS = 1, UB_OP_INT32_RANGE_ = 0x7FFFFFFF } ub_op_t;

/* Per-call overlap options: the keys of [TE#1344]'s option list.
 *   num_splits       chunks the GEMM is cut into (>= 1); ignored for ring exchange,
 *                    which uses tp_size chunks.
 *   num_max_streams  compute streams = min(chunks, num_max_streams, UB_MAX_STREAMS), >= 1.
 *                    Default 3.  The handle's worker streams overlap with the caller's
 *                    stream only on hardware queues of their own: HIP places streams on
 *                    GPU_MAX_HW_QUEUES queues (4 by default) in creation order, and streams
 *                    that share one run in issue order.  ub_prepare_streams creates them
 *                    right after registration, before the process's other streams, so that
 *                    they take queues of their own; otherwise the first call that needs
 *                    them creates them.
 *   aggregate        all-gather side only: chunks {2u, 2u+1} are merged into one launch.
 *   atomic_gemm      0: one kernel launch per unit from a host loop on the compute
 *                    streams; 1: one kernel on the caller's stream whose workgroups walk
 *                    the units on the device in plan order (at most 64 non-empty units,
 *                    else UB_ERR_UNSUPPORTED).  The units' rows are cut into tiles from
 *                    the first active row, each tile going to the unit that holds its
 *                    last row, so a tile may read rows of two neighbouring units.
 *                    Results are bit-identical to the host loop ([TE#1344]
 *                    "atomic_gemm").
 *   rank             this rank in [0, tp_size): sets the ring order.
 *   use_ce           ub_gemm_ag_arrival / ub_deliver_chunks only: deliveries from device
 *                    memory go on the SDMA engines (1, the default) or through the
 *                    runtime's copy kernel (0).  Ignored elsewhere.
 *   num_sm, set_sm_margin  accepted for compatibility and ignored: on one GPU there is no
 *                    communication kernel to reserve compute units for.
 *   reduce_order     reduce-scatter side only (ub_reduce_order_t).  UB_REDUCE_ASCENDING
 *                    (default): out = bf16(sum of the tp bf16 partials in fp32, slice 0
 *                    first), one rounding.  UB_REDUCE_RING: the sum a ring
 *                    reduce-scatter computes ([TE#1344] "ring_exchange" moves chunks
 *                    between neighbours): for shard r the partial of slice r+1 starts,
 *                    slices r+2, ..., r (mod tp) are added one per hop in fp32 and the
 *                    running value is rounded to bf16 after every hop.
 *   fuse_reduce      reduce-scatter side, bf16 operands only (ignored on the all-gather
 *                    side; 1 with ub_gemm_rs_chunked_fp8 -> UB_ERR_UNSUPPORTED).  0: the
 *                    sum runs as its own launch after each unit's slice GEMMs.  1: inside
 *                    the slice-GEMM launch, the last of the tp slice tiles of each output
 *                    tile to finish sums the tp partials ([TE#1344] "pipeline": the
 *                    GEMM chunks feed the reduce-scatter; here with no separate pass).  The
 *                    partials still go through the workspace, and out is bit-identical to
 *                    fuse_reduce 0 for either reduce_order.  The tiles count their arrival
 *                    in the workspace's counter region (see ub_required_bytes), which every
 *                    launch leaves at zero; nothing is allocated or cleared on the call, so
 *                    any fused call may be captured into a graph. */
typedef enum { UB_REDUCE_ASCENDING = 0, UB_REDUCE_RING = 1 } ub_reduce_order_t;

typedef struct {
  int32_t method;
  int32_t num_splits;
  int32_t num_max_streams;
  int32_t aggregate;
  int32_t atomic_gemm;
  int32_t rank;
  int32_t use_ce;
  int32_t num_sm;
  int32_t set_sm_margin;
  int32_t reduce_order;
  int32_t fuse_reduce;
} ub_overlap_cfg_t;

/* One unit of an execution plan: rows [row0, row1) of the active T, at position `pos`
 * of the execution order, on compute stream `stream` (0 = the caller's stream). */
typedef struct {
  int32_t pos;
  int32_t unit;
  int64_t row0;
  int64_t row1;
  int32_t stream;
  int32_t reserved;
} ub_plan_unit_t;

/* Accumulated per-launch kernel timings (see ub_set_kernel_timing). */
typedef struct {
  int64_t launches;   /* kernel launches measured */
  double total_ms;    /* sum of per-launch durations, HIP events on the launch stream */
  double flops;       /* algorithmic floating-point operations of those launches */
  double bytes;       /* algorithmic HBM bytes of those launches */
} ub_kernel_stats_t;

/* Fill `cfg` with the defaults of [TE#1344]: ring exchange, num_splits 1,
 * num_max_streams 3, use_ce 1, aggregate 0, atomic_gemm 0, set_sm_margin 0, num_sm 0,
 * rank 0, reduce_order UB_REDUCE_ASCENDING, fuse_reduce 0. */
UB_API void ub_overlap_cfg_default(ub_overlap_cfg_t* cfg);

/* Bytes the caller must allocate for a registration of [capacity, hidden] over
 * tp_size ranks: the UB itself (capacity * hidden * element size: 2 for bf16, 1 for
 * fp8) and the reduce-scatter workspace (0 for fp8, which has no reduce-scatter side).
 * The workspace holds the tp_size bf16 partial slots (tp_size * capacity * hidden * 2
 * bytes, [TE#3564] "Implementation approach": reduce-scatter keeps its per-rank chunks in
 * its own capacity-sized allocation) and, from the next 256-byte boundary, the fused
 * reduction's tile counters: 4 bytes per 128 x 128 output tile of a launch over up to
 * capacity rows, one range per compute stream (UB_MAX_STREAMS of them), sized once here
 * from the capacity (~129 KiB for capacity 16384, hidden 4096).  Same validation as
 * ub_init.  Either output pointer may be NULL. */
UB_API ub_status_t ub_required_bytes(int64_t capacity, int64_t hidden, int32_t tp_size,
                                     ub_dtype_t dtype, size_t* ub_bytes,
                                     size_t* rs_workspace_bytes);

/* Register a UserBuffer at its maximum token capacity ([TE#3564] "Proposed API":
 * initialize at [max_tokens, hidden_size] with tp_size, unquantized, bf16).
 *   capacity, hidden  > 0; hidden % 8 == 0 (bf16) or % 16 == 0 (fp8); capacity %
 *                     tp_size == 0 (so that the initial active shape, which equals the
 *                     capacity shape, is valid).
 *   tp_size           1 .. UB_MAX_TP.
 *   dtype             UB_DTYPE_BF16 or UB_DTYPE_FP8_E4M3, else UB_ERR_DTYPE.
 *   ub_buf, ub_bytes  device memory of at least capacity*hidden*element-size bytes
 *                     (16-byte aligned), else UB_ERR_BUFFER_TOO_SMALL / UB_ERR_INVALID_ARG.
 *   rs_ws, rs_ws_bytes reduce-scatter workspace of at least the size ub_required_bytes
 *                     reports, or NULL/0 when the reduce-scatter side is not used (always
 *                     NULL/0 for fp8, else UB_ERR_INVALID_ARG).  Its counter region (the
 *                     bytes past the partial slots) must be zero at registration, e.g.
 *                     allocated with torch.zeros; every call leaves it zero.
 * Records the pointers and sizes; allocates no device memory and makes no HIP call
 * (streams and events are created by ub_prepare_streams or on the first GEMM call, on the
 * device current then).  On success *out is a new handle whose active shape is
 * [capacity, hidden]. */
UB_API ub_status_t ub_init(ub_handle_t* out, int64_t capacity, int64_t hidden,
                           int32_t tp_size, ub_dtype_t dtype, void* ub_buf, size_t ub_bytes,
                           void* rs_ws, size_t rs_ws_bytes);

/* Set the active shape for the next microbatch ([TE#3564] "Proposed API" and
 * "Implementation approach"): shape = {T, hidden}, ndim = 2.  Checks, in the order the
 * pages list the constraints, returning the first that fails: ndim != 2 -> NDIM; any
 * dimension <= 0 -> ZERO_DIM; T > capacity -> CAPACITY; hidden != registered ->
 * HIDDEN_MISMATCH; T % tp_size != 0 -> TP_DIVISIBILITY.  On success only host-side views
 * change (T, element counts, chunk/shard/partial offsets); nothing is allocated, freed,
 * re-registered or launched.  On failure the previous active shape is kept. */
UB_API ub_status_t ub_set_active_shape(ub_handle_t h, const int64_t* shape, int32_t ndim);

/* Active and capacity shapes ([TE#3564]: per-communicator active/capacity getters). */
UB_API ub_status_t ub_get_active_shape(ub_handle_t h, int64_t shape_out[2]);
UB_API ub_status_t ub_get_capacity_shape(ub_handle_t h, int64_t shape_out[2]);

/* Execution plan a GEMM call with `cfg` would follow at the current active T
 * ([TE#1344] "num_splits", "num_max_streams", "aggregate", "method").  Writes up to
 * max_units entries to `out` (may be NULL when max_units is 0) and the unit and stream
 * counts to *n_units / *n_streams.  Host-only. */
UB_API ub_status_t ub_get_plan(ub_handle_t h, const ub_overlap_cfg_t* cfg, ub_op_t op,
                               ub_plan_unit_t* out, int32_t max_units, int32_t* n_units,
                               int32_t* n_streams);

/* Copy `rows` rows of [*, hidden] elements (bf16, or fp8 codes for an fp8 buffer) from
 * device memory `src` (row stride hidden) into
 * active rows [row_offset, row_offset + rows) of the UB, asynchronously on `stream`
 * (this is where a rank's own shard enters the buffer).  The copy-size check is against
 * the active T, not the capacity ([TE#3564]: copy-size checks use the active element
 * count): row_offset + rows > T -> UB_ERR_INVALID_ARG. */
UB_API ub_status_t ub_copy_in(ub_handle_t h, const void* src, int64_t rows,
                              int64_t row_offset, ub_stream_t stream);

/* All-gather-side column-parallel GEMM over the active prefix ([MLM#1240] QKV / MLP fc1
 * diagrams; [TE#1344] option list; [TE#3564] offsets from the active T):
 *   C[t, j] = bf16( sum_k UB[t, k] * W[k, j] ),  t in [0, T), j in [0, n_cols),
 * with UB the active [T, hidden] prefix (row stride hidden), W [hidden, n_cols] with row
 * stride ldw >= n_cols, C [T, n_cols] with row stride ldc >= n_cols.  The rows are cut
 * into the plan's units; unit u is one GEMM reading the UB at byte offset
 * row0_u * hidden * 2.  Reads no UB byte beyond T*hidden elements; writes only C rows
 * [0, T).  n_cols, ldw, ldc and hidden multiples of 8 (16-byte rows); a hidden that is not
 * a multiple of the kernel's 32-deep k-step is handled by masking the last step's
 * k-chunks past hidden.  aggregate is honoured; W and C are caller memory.  Needs a bf16
 * handle, as do ub_gemm_ag_arrival, ub_deliver_chunks, ub_gemm_rs_chunked and
 * ub_reduce_partials (else UB_ERR_DTYPE). */
UB_API ub_status_t ub_gemm_ag_chunked(ub_handle_t h, const void* w, int64_t n_cols,
                                      int64_t ldw, void* c, int64_t ldc,
                                      const ub_overlap_cfg_t* cfg, ub_stream_t stream);

/* FP8 (E4M3) UserBuffers: the extension to quantized buffers that [TE#3564]
 * ("Implementation approach", last paragraph) leaves outside the first scope.  The pages
 * give no format or scaling rule; the reading taken: OCP E4M3 codes (bias 7, 3 significand
 * bits, largest finite 448, no infinities) with one scale per tensor.
 *
 * ub_quantize_in: rows [row_offset, row_offset + rows) of the fp8 UB receive
 *   q = sat(RNE_e4m3(fp32(x * scale))) of the bf16 rows `src` ([rows, hidden] packed,
 *   16-byte aligned device memory): one fp32 multiply, round to the nearest E4M3 value
 *   with ties to even, magnitudes beyond 448 saturate to 448, NaN stays NaN.  The size
 *   check is against the active T, as for ub_copy_in.  scale must be finite.  Needs an
 *   fp8 handle (else UB_ERR_DTYPE).  Asynchronous on `stream`. */
UB_API ub_status_t ub_quantize_in(ub_handle_t h, const void* src, int64_t rows,
                                  int64_t row_offset, float scale, ub_stream_t stream);

/* ub_gemm_ag_chunked_fp8: the all-gather-side chunked GEMM over an fp8 UB, with the same
 * plan, options, streams and device-side chunk loop as ub_gemm_ag_chunked:
 *   C[t, j] = bf16_rne( (scale_inv_a * scale_inv_w) * sum_k UB[t, k] * W[j, k] )
 * for t < T, with fp32 accumulation and the two dequantization factors multiplied once in
 * fp32.  W is [n_cols, hidden] E4M3 codes, row stride ldw bytes (>= hidden, multiple of
 * 16; the weight stored N x K, as FP8 GEMMs take it); C is [T, n_cols] bf16 (ldc >= n_cols,
 * multiple of 8).  hidden must be a multiple of 64 (else UB_ERR_UNSUPPORTED).  Needs an
 * fp8 handle (else UB_ERR_DTYPE). */
UB_API ub_status_t ub_gemm_ag_chunked_fp8(ub_handle_t h, const void* w, int64_t n_cols,
                                          int64_t ldw, float scale_inv_a, float scale_inv_w,
                                          void* c, int64_t ldc, const ub_overlap_cfg_t* cfg,
                                          ub_stream_t stream);

/* Arrival stand-in for the all-gather side ([TE#1344] "ring_exchange": the other ranks'
 * chunks arrive by point-to-point copies, "use_ce": on the Copy Engine, without compute
 * units; each GEMM chunk runs once its data is there).
 *
 * Same result as ub_gemm_ag_chunked, but the UB prefix is completed while the call runs:
 * `src` ([T, hidden] bf16 packed, 16-byte aligned; device memory, or pinned host memory
 * when src_on_host is nonzero) holds the active rows as the other ranks would send them,
 * and the non-local chunks are copied from src into the UB rows they belong to on the
 * handle's copy stream, in plan order (each unit's chunks ascending), one event per
 * chunk.  A unit's copies are issued just before its GEMM, and each unit's GEMM waits on
 * the events of its own chunks only, so GEMMs on arrived chunks overlap the remaining
 * copies.
 *   Local chunk: with method ring exchange, chunk `rank` (rows [rank*T/tp,
 *     (rank+1)*T/tp)) is this rank's own shard, already in the UB (ub_copy_in); its rows
 *     of src are never read.  With pipeline or bulk every chunk is delivered.
 *   Copy kind: host source: hipMemcpyHostToDevice over PCIe (SDMA engines; src must be
 *     pinned, e.g. hipHostMalloc).  Device source: use_ce = 1 -> hipMemcpyDeviceToDeviceNoCU
 *     (SDMA engines, no compute units), use_ce = 0 -> hipMemcpyDeviceToDevice (the
 *     runtime's copy kernel, which shares the compute units with the GEMMs).  Measured on
 *     MI355X with ROCm 7.2: all three kinds run alongside the GEMMs of other streams; an
 *     SDMA copy costs about 80 us whatever its size.
 *   atomic_gemm = 1: the device-side chunk loop ([TE#1344] "atomic_gemm") gated by a
 *     ready flag per chunk.  After each chunk's copy, the copy stream writes the call's
 *     epoch to the chunk's flag (hipStreamWriteValue32; the local chunk's flag first).
 *     The GEMM's tiles (one launch, or two when a ragged last round is cut off) wait for
 *     the flags of the chunks whose rows they read,
 *     acquire at system scope, then load.  The copy stream's work is all issued before
 *     the GEMM, so streams that share a hardware queue serialise rather than wait on each
 *     other.
 *     - Deliveries must be SDMA copies: use_ce = 1 or a host source.  Otherwise
 *       UB_ERR_UNSUPPORTED, because the runtime's copy kernel would need CUs that waiting
 *       tiles hold.
 *     - A tile's wait is bounded (~0.5 s); past it the tile stores bf16 NaN (0x7FC0)
 *       over its whole output instead of computing from rows that may not have arrived,
 *       and counts one timeout (ub_arrival_timeouts).
 *     - The flags live in a fixed device array of 64 slots, one per handle, taken on its
 *       first such call and returned by ub_destroy; a 65th handle gets
 *       UB_ERR_UNSUPPORTED.
 *   More than 64 chunks -> UB_ERR_UNSUPPORTED.
 *   Hardware queues: the call keeps up to four streams busy (the caller's, two workers,
 *     the copy stream).  HIP maps a process's streams onto GPU_MAX_HW_QUEUES hardware
 *     queues (4 by default), and streams that share a queue run in issue order: with
 *     other streams in the process, copies and GEMMs then serialise (measured on qkv:
 *     0.30 instead of 0.22 ms per call with three other streams and 4 queues, 0.22 ms with
 *     8 queues).  A process that overlaps arrivals should raise GPU_MAX_HW_QUEUES.
 * The copies start when the caller's stream reaches the call; the call as a whole is
 * ordered on `stream`.  The caller must not touch the UB prefix or src until then. */
UB_API ub_status_t ub_gemm_ag_arrival(ub_handle_t h, const void* src, int32_t src_on_host,
                                      const void* w, int64_t n_cols, int64_t ldw, void* c,
                                      int64_t ldc, const ub_overlap_cfg_t* cfg,
                                      ub_stream_t stream);

/* Number of tiles of the device-side chunk loop of ub_gemm_ag_arrival whose wait hit the
 * time bound on this handle's flag slot since the handle took the slot (0 if the handle
 * never gated on arrivals; ub_destroy clears the count, so a slot handed to a later handle
 * starts from zero).  Split-K rows (ub_register_scratch) summed by a second launch count
 * once per K segment whose wait ran out; summed in the kernel, once per tile.  A nonzero
 * count means a chunk's flag never came; those tiles hold NaN.  Synchronous (copies one
 * word from the device). */
UB_API ub_status_t ub_arrival_timeouts(ub_handle_t h, uint32_t* count);

/* The deliveries of ub_gemm_ag_arrival alone (same copies, order, stream and kind, no
 * GEMM), ordered on `stream`: for measuring how long the arrivals take by themselves. */
UB_API ub_status_t ub_deliver_chunks(ub_handle_t h, const void* src, int32_t src_on_host,
                                     const ub_overlap_cfg_t* cfg, ub_stream_t stream);

/* Reduce-scatter-side row-parallel GEMM ([MLM#1240] MLP diagram, RowParallelLinear;
 * [TE#3564]: partial chunks inside the workspace's allocation, offsets from active T):
 * with Ks = k / tp_size, for every plan unit (rows [r0, r1)) and slice s:
 *   P_s[t, j] = bf16( sum_{k in [s Ks, (s+1) Ks)} A[t, k] * W[k, j] )
 * written to the workspace at element (s*T + t) * hidden + j (the packed active prefix
 * of tp_size slots), then
 *   out[t, j] = bf16( sum_{s = 0..tp_size-1} P_s[t, j] )   (fp32 sum, ascending s)
 * or, with cfg->reduce_order = UB_REDUCE_RING, the ring-order sum with a bf16 rounding
 * per hop (see ub_overlap_cfg_t), so that rank r's shard is out rows
 * [r T/tp, (r+1) T/tp), contiguous.
 * A is [T, k] (row stride lda >= k), W is [k, hidden] (row stride ldw >= hidden), out is
 * [T, hidden] (row stride ldo >= hidden).  k % tp_size == 0 (else INVALID_ARG) and
 * Ks % 8 == 0, so that every slice starts on a 16-byte boundary (else UNSUPPORTED).
 * Requires a registered workspace (else
 * NOT_INITIALIZED).  aggregate is ignored (it is an all-gather option).  Writes nothing
 * beyond tp_size*T*hidden workspace elements or beyond T rows of out. */
UB_API ub_status_t ub_gemm_rs_chunked(ub_handle_t h, const void* a, int64_t k, int64_t lda,
                                      const void* w, int64_t ldw, void* out, int64_t ldo,
                                      const ub_overlap_cfg_t* cfg, ub_stream_t stream);

/* ub_gemm_rs_chunked for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation), also on a handle
 * registered without a workspace: same arguments, checks, plan, kernels and results (bit
 * for bit), but the tp partial slots ([tp, T, hidden] bf16, packed from the active T) and,
 * with fuse_reduce, the tile counters live in the library's fixed device scratch of 32 MiB
 * (kept by each GPU the library runs on until the process ends) instead of the registered
 * workspace.  Calls needing more than 32 MiB (tp * T * hidden * 2 bytes of partials, plus
 * the counters) return UB_ERR_BUFFER_TOO_SMALL before anything is enqueued.  Allocates
 * nothing and calls no allocating routine; with fuse_reduce it first clears the counters
 * with a fill kernel on `stream`.  Every call on one GPU shares the scratch: calls that
 * overlap on a GPU (other streams, other handles, other threads) race and must be ordered
 * by the caller.  The partials are not left in the handle's workspace, so
 * ub_reduce_partials does not see them. */
UB_API ub_status_t ub_gemm_rs_chunked_noalloc(ub_handle_t h, const void* a, int64_t k,
                                              int64_t lda, const void* w, int64_t ldw, void* out,
                                              int64_t ldo, const ub_overlap_cfg_t* cfg,
                                              ub_stream_t stream);

/* FP8 (E4M3) reduce-scatter GEMM: ub_gemm_rs_chunked with E4M3 operands and one
 * dequantization factor per tensor (the reading of [TE#3564]'s quantized buffers taken
 * for ub_gemm_ag_chunked_fp8).  The partials and the sum are bf16, as in
 * ub_gemm_rs_chunked, so the handle is a bf16 one with a registered workspace.  With
 * Ks = k / tp_size, for every plan unit and slice s:
 *   P_s[t, j] = bf16_rne( (scale_inv_a * scale_inv_w) * sum_{k in [s Ks, (s+1) Ks)} A[t, k] * W[j, k] )
 * (fp32 accumulation; the two factors multiplied once in fp32), written to the workspace
 * at element (s*T + t) * hidden + j, then summed into out exactly as ub_gemm_rs_chunked
 * sums (cfg->reduce_order).
 *   A   [T, k] E4M3 codes, row stride lda bytes (>= k, multiple of 16), device memory;
 *   W   [hidden, k] E4M3 codes, row j = output column j, row stride ldw bytes (>= k,
 *       multiple of 16): the weight stored N x K, as FP8 GEMMs take it;
 *   out [T, hidden] bf16, row stride ldo elements (>= hidden, multiple of 8).
 * k % tp_size == 0 (else INVALID_ARG), Ks % 64 == 0 (else UNSUPPORTED); scales finite
 * (else INVALID_ARG); a bf16 handle (else UB_ERR_DTYPE) with a workspace (else
 * NOT_INITIALIZED).  Plan, streams, atomic_gemm and the write bounds as for
 * ub_gemm_rs_chunked. */
UB_API ub_status_t ub_gemm_rs_chunked_fp8(ub_handle_t h, const void* a, int64_t k, int64_t lda,
                                          const void* w, int64_t ldw, float scale_inv_a,
                                          float scale_inv_w, void* out, int64_t ldo,
                                          const ub_overlap_cfg_t* cfg, ub_stream_t stream);

/* E4M3 quantization of a bf16 matrix into caller memory, with no handle: the operands of
 * ub_gemm_rs_chunked_fp8 (and weights for ub_gemm_ag_chunked_fp8).
 *   dst[r, c] = sat(RNE_e4m3(fp32(src[r, c] * scale)))   for r < rows, c < cols,
 * the rule of ub_quantize_in.  src is bf16 with row stride lds elements, dst is E4M3 with
 * row stride ldd bytes; both device memory and 16-byte aligned; cols, lds and ldd
 * multiples of 8 with lds, ldd >= cols; rows, cols >= 0; scale finite (else
 * UB_ERR_INVALID_ARG; there is no handle, so no message).  rows == 0 or cols == 0 does
 * nothing.  Asynchronous on `stream`. */
UB_API ub_status_t ub_quantize_e4m3(const void* src, int64_t lds, void* dst, int64_t ldd,
                                    int64_t rows, int64_t cols, float scale, ub_stream_t stream);

/* The reduce-scatter sum alone: out[t, :] for all active rows t in [0, T) from the
 * tp_size partial slots currently in the workspace (as left by ub_gemm_rs_chunked at the
 * same T), summed in the order `reduce_order` (ub_reduce_order_t, as in
 * ub_overlap_cfg_t; anything else -> UB_ERR_INVALID_ARG).  One launch on `stream`.  For
 * measuring the reduction by itself ([TE#1344] "pipeline": the reduce-scatter that the
 * GEMM chunks feed). */
UB_API ub_status_t ub_reduce_partials(ub_handle_t h, void* out, int64_t ldo,
                                      int32_t reduce_order, ub_stream_t stream);

/* Per-launch kernel timing.  enable 1: every GEMM and reduction launch is bracketed by HIP
 * events on the stream it is launched on: a start event recorded before it, and an end
 * event that the call's last kernel launch takes (hipExtLaunchKernel's stop event, the
 * kernel's own completion time, no separate event record).
 * enable 2, chained: a launch's start is the end event of the previous launch timed on
 * the same stream since the last ub_get_kernel_timing or ub_set_kernel_timing, so no
 * event record of its own after the first (a record costs a few microseconds of GPU
 * time); the caller
 * promises that nothing else runs on that stream between the calls it measures, or that
 * work counts as the next launch's time (back-to-back calls on one stream; not the host
 * loop's worker streams, whose launches wait for the caller's).  enable 0 (the default):
 * off.  ub_get_kernel_timing waits for the measured launches and returns the accumulated
 * durations with their algorithmic FLOPs and bytes, then clears the counters and ends the
 * chains.  Other values of enable -> UB_ERR_INVALID_ARG. */
UB_API ub_status_t ub_set_kernel_timing(ub_handle_t h, int32_t enable);
UB_API ub_status_t ub_get_kernel_timing(ub_handle_t h, ub_kernel_stats_t* gemm,
                                        ub_kernel_stats_t* reduce);

/* Create the handle's compute streams now, on the current device: the worker streams
 * (and events) that calls with up to num_max_streams streams use (clamped to
 * UB_MAX_STREAMS), and, when copy_stream is nonzero, the copy stream of
 * ub_gemm_ag_arrival.  Optional: a call creates what it needs the first time; creating
 * them right after registration gives them hardware queues of their own before the
 * process's other streams take them (see num_max_streams).  num_max_streams < 1 ->
 * UB_ERR_INVALID_ARG; a handle is bound to the device current at its first HIP call. */
UB_API ub_status_t ub_prepare_streams(ub_handle_t h, int32_t num_max_streams,
                                      int32_t copy_stream);

/* Tile plan of the last GEMM launch group of a handle (ub_debug_last_plan). */
typedef struct {
  int32_t tile_m, tile_n;            /* tile of the (first) launch */
  int64_t cut_row;                   /* -1: one launch; else the first row of a second launch */
  int32_t tail_tile_m, tail_tile_n;  /* tile of the second launch (0 without one) */
  int64_t seg_row;                   /* first K-segmented row of the launch group, or -1 */
  int32_t nseg;                      /* K segments of those rows (0 or >= 2) */
  int32_t split;                     /* the segments ran as separate workgroups (split-K),
                                        summed in the kernel (1) or by a second launch (2);
                                        0: one workgroup per tile */
  int32_t seg_tile_m, seg_tile_n;    /* tile of the segmented rows' launch */
  int32_t dispatches;                /* GEMM kernels the last call launched, every launch
                                        group counted (reductions not counted) */
  int32_t rs_pieces;                 /* row pieces of a pipelined device-side
                                        reduce-scatter (0: not pipelined) */
} ub_tile_plan_t;

/* Split-K scratch of a handle (optional; all-gather side).  When a call's shape leaves the
 * chip underused -- few rows (small T), or a last round of tiles that would hold only a
 * few -- the library sums the rows concerned in K segments: for those rows,
 *   C = bf16( ((P_0 + P_1) + ...) + P_{nseg-1} )  in fp32,  P_s = the products of k-steps
 *   [s nk / nseg, (s+1) nk / nseg) (32-deep steps) accumulated from zero,
 * a choice made from (T, n_cols, hidden) alone while scratch is registered (nothing is
 * segmented without it), so that every schedule (chunk count, stream count, order,
 * atomic_gemm, arrivals) computes the same bits.  The segments run as separate workgroups
 * that write fp32 partial tiles to the scratch; a launch that needs more partial space than
 * it has (the host loop gives each of its streams an equal share) falls back to one
 * workgroup per tile summing the segments in the same order: the same bits, slower.  The
 * library segments at most 1024 tiles' worth of partials (64 MiB) in one call, so
 * UB_SCRATCH_COUNTER_BYTES + 64 MiB covers every choice of the device-side chunk loop.
 * Layout: the first UB_SCRATCH_COUNTER_BYTES hold 32-bit counters that must be zero at
 * registration (e.g. torch.zeros) and are left zero; the rest holds partials.  The buffer
 * is caller-owned and must outlive its registration; calls of the handle must not overlap
 * on different streams (they share it).  buf NULL and bytes 0 unregisters; bytes <
 * UB_SCRATCH_MIN_BYTES -> UB_ERR_BUFFER_TOO_SMALL; a buf not 16-byte aligned ->
 * UB_ERR_INVALID_ARG. */
#define UB_SCRATCH_COUNTER_BYTES (256 * 1024)
#define UB_SCRATCH_MIN_BYTES (UB_SCRATCH_COUNTER_BYTES + 64 * 1024)
UB_API ub_status_t ub_register_scratch(ub_handle_t h, void* buf, size_t bytes);

/* Debug and tuning settings of one handle, for tests and tile tuning; each starts at 0,
 * which leaves every choice to the library.  No environment variable changes what the
 * library computes.  Keys:
 *   "tile_m", "tile_n"     force this tile shape for every GEMM launch of the handle (one
 *                          launch per unit group, no cut).  Calls fail with
 *                          UB_ERR_INVALID_ARG if their kernel has no such tile (bf16:
 *                          320x256, 256x256, 128x256, 128x128; fp8: 256x256, 128x256).
 *                          Results do not depend on the tile.
 *   "cut_row"              > 0: a bf16 launch group whose rows span this row (a band
 *                          boundary of its first tile) runs as two launches, the rows from
 *                          cut_row on with the tile "tail_tile_m" x "tail_tile_n" (default
 *                          128x128); the first launch takes the forced tile, or 256x256.
 *                          Results do not depend on the cut.
 *   "nseg", "seg_row"      K segmentation of the all-gather side: nseg 0 (default) lets the
 *                          shape decide (see ub_register_scratch); 1 turns it off; >= 2
 *                          sums rows from seg_row on (call rows, default 0) in nseg
 *                          segments (clamped to the number of 32-deep k-steps).
 *   "seg_tile_m", "seg_tile_n"  tile of forced split pieces (default 256 x 256; any of the
 *                          bf16 tiles).
 *   "rs_pieces"            device-side reduce-scatter (atomic_gemm; bf16 with fuse_reduce 0,
 *                          and fp8) in P row pieces: piece p's slice GEMMs on the caller's stream, its
 *                          reduction on a worker stream overlapping piece p + 1's GEMMs;
 *                          0 (default) the library's choice, 1..8 forced.  The results do
 *                          not change.
 *   "seg_reduce"           sum of forced split pieces: 1 the tile's last piece sums in the
 *                          kernel (per-tile counters in the scratch); 2 (default) a second
 *                          launch sums every tile over the whole chip.
 *   "tile_group"           row tiles per group in the workgroup -> tile map (>= 1).
 *   "arrival_wait_us"      bound of a gated tile's wait in ub_gemm_ag_arrival, in
 *                          microseconds (0: ~0.5 s).
 *   "arrival_drop_flags"   1: write no ready flag after the delivered chunks, so that the
 *                          tiles that need them run into the bound (a test of that path).
 * Unknown keys and out-of-range values -> UB_ERR_INVALID_ARG. */
UB_API ub_status_t ub_debug_set(ub_handle_t h, const char* key, int64_t value);
UB_API ub_status_t ub_debug_last_plan(ub_handle_t h, ub_tile_plan_t* out);

/* Destroy a handle: waits for the handle's own streams, then releases its streams,
 * events and arrival-flag slot.  The caller's streams are not waited for: work of this
 * handle still queued there must have finished (the caller synchronises first), or a
 * device-side loop of a gated arrival could wait on a slot that another handle has taken
 * (it would end at its time bound, with wrong results).  Caller buffers are untouched.
 * NULL is accepted. */
UB_API ub_status_t ub_destroy(ub_handle_t h);

/* Static name of a status code ("UB_OK", "UB_ERR_CAPACITY", ...). */
UB_API const char* ub_status_string(ub_status_t s);
/* Message describing the last failure on h ("" if none); valid until the next call on h. */
UB_API const char* ub_last_error(ub_handle_t h);

#ifdef __cplusplus
}
#endif

#endif /* CHUNKED_TP_OVERLAP_AMD_UB_H */
