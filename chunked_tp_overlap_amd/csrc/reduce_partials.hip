// Partial-sum reduction of the reduce-scatter side.
//
// The row-parallel GEMM (MLP fc2 in "[QUESTION] Do tp overlap support thd, whose sequence
// length is flexible?", Megatron-LM discussion 1240, MLP diagram) leaves tp bf16 partial
// products of [rows, cols] in the workspace, slot s at parts + s * slot_stride; their sum,
// rounded once to bf16, is the reduce-scatter result whose tp row blocks are the ranks'
// shards ("How to setup TP Overlap configs", Transformer Engine issue 1344, "pipeline":
// the GEMM chunks feed a reduce-scatter).
//
//   out[r, c] = bf16( ((0 + P_0[r, c]) + P_1[r, c]) + ... + P_{tp-1}[r, c] )   in fp32
//
// or, in ring order (the sum a ring reduce-scatter computes: the partials of shard q
// start at rank q+1 and each hop adds one rank's bf16 partial in fp32 and rounds to bf16
// before passing it on, "How to setup TP Overlap configs", "ring_exchange"):
//
//   acc = P_{q+1};  acc = bf16(acc + P_{q+i}) for i = 2 .. tp (slot indices mod tp),
//
// with q = (row0 + r) / shard_rows the shard of row r.
//
// HBM-bound: every element is read tp times and written once (2 (tp + 1) bytes per output
// element).  Each lane handles V 16-byte vectors (8 elements each) of one workgroup's
// chunk of V * 256 consecutive vectors, and walks the slots in ascending order: V loads of
// slot s, add them into the V fp32 accumulators, then slot s + 1.  Many short chunks with
// this slot-major order stream faster on MI355X than long per-workgroup ranges or a
// grid-stride walk with every slot's loads in flight (measured on 8 slots of
// [16384, 4096]: about 6.1 TB/s against 5.1 - 5.7).  V = 4, except for small sums (at most
// 2^21 vectors), where V = 2 gives twice the workgroups: measured with the MALL flushed,
// 8 slots of [2048, 4096] at 5.6 TB/s against 5.1 - 5.2 with V = 4, while V = 2 loses
// 6% at [16384, 4096] and V = 8 loses everywhere.  The partials are read exactly once,
// so loads and stores are non-temporal.  When the partial rows and the output rows are
// both packed (leading dimension == cols) the vectors are one flat run; otherwise each
// vector's row is recovered by division.
#include <hip/hip_runtime.h>

#include "ub_internal.h"

namespace ubx {
namespace {

constexpr int THREADS = 256;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
#define GLOBAL_PTR(T, p) ((__attribute__((address_space(1))) T*)(p))

__device__ inline float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ inline uint32_t pack2(float a, float b) {
  const uint32_t x = __builtin_bit_cast(uint16_t, static_cast<__bf16>(a));  // RNE
  const uint32_t y = __builtin_bit_cast(uint16_t, static_cast<__bf16>(b));
  return x | (y << 16);
}

__device__ inline void add8(float (&acc)[8], u32x4 x) {
  acc[0] += lo_bf16(x[0]); acc[1] += hi_bf16(x[0]);
  acc[2] += lo_bf16(x[1]); acc[3] += hi_bf16(x[1]);
  acc[4] += lo_bf16(x[2]); acc[5] += hi_bf16(x[2]);
  acc[6] += lo_bf16(x[3]); acc[7] += hi_bf16(x[3]);
}

__device__ inline u32x4 pack8(const float (&acc)[8]) {
  u32x4 o;
  o[0] = pack2(acc[0], acc[1]);
  o[1] = pack2(acc[2], acc[3]);
  o[2] = pack2(acc[4], acc[5]);
  o[3] = pack2(acc[6], acc[7]);
  return o;
}


// fp32 -> nearest bf16 (ties to even), returned as the fp32 of the same value.
__device__ inline float round_bf16(float x) {
  return __uint_as_float((uint32_t)__builtin_bit_cast(uint16_t, static_cast<__bf16>(x)) << 16);
}

// One ring hop for 8 elements: acc = bf16(acc + x), or acc = x for the first partial.
__device__ inline void hop8(float (&acc)[8], u32x4 x, bool first) {
  const float v[8] = {lo_bf16(x[0]), hi_bf16(x[0]), lo_bf16(x[1]), hi_bf16(x[1]),
                      lo_bf16(x[2]), hi_bf16(x[2]), lo_bf16(x[3]), hi_bf16(x[3])};
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = first ? v[i] : round_bf16(acc[i] + v[i]);
}

// acc[j] += the V vectors of one slot (loads first, then the adds).
template <int V>
__device__ inline void add_slot(float (&acc)[V][8], const bool (&ok)[V], const int64_t (&ein)[V],
                                const uint16_t* slot) {
  u32x4 x[V];
#pragma unroll
  for (int j = 0; j < V; ++j)
    if (ok[j]) x[j] = __builtin_nontemporal_load(GLOBAL_PTR(const u32x4, slot + ein[j]));
#pragma unroll
  for (int j = 0; j < V; ++j)
    if (ok[j]) add8(acc[j], x[j]);
}

// Ring hop i for the V vectors: slot (first[j] + i) mod nslots of each vector j.
template <int NS, int V>
__device__ inline void hop_slot(float (&acc)[V][8], const bool (&ok)[V], const int64_t (&ein)[V],
                                const int (&first)[V], int i, const ReduceArgs& r) {
  u32x4 x[V];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    int s = first[j] + i;
    if (s >= (NS > 0 ? NS : r.nslots)) s -= (NS > 0 ? NS : r.nslots);
    if (ok[j]) x[j] = __builtin_nontemporal_load(GLOBAL_PTR(const u32x4, r.parts + s * r.slot_stride + ein[j]));
  }
#pragma unroll
  for (int j = 0; j < V; ++j)
    if (ok[j]) hop8(acc[j], x[j], i == 0);
}

// Workgroup b reduces vectors [b * V * THREADS, (b + 1) * V * THREADS) clipped to nvec; lane t
// takes vectors t, t + THREADS, ...  PACKED: vector v is at element 8 v of every slot and
// of out; otherwise at row v / vpr, column 8 (v % vpr).  NS = 0: nslots at run time.
template <int NS, bool PACKED, bool RING, int V>
__global__ __launch_bounds__(THREADS) void reduce_chunks(ReduceArgs r, int64_t nvec, int64_t vpr) {
  const int64_t base = (int64_t)blockIdx.x * (V * THREADS) + threadIdx.x;
  int64_t ein[V], eout[V];
  int first[V];  // ring order: slot of the first partial of each vector's shard
  bool ok[V];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int64_t v = base + j * THREADS;
    ok[j] = v < nvec;
    const int64_t row = v / vpr;
    if (PACKED) {
      ein[j] = eout[j] = v * 8;
    } else {
      const int64_t col = (v - row * vpr) * 8;
      ein[j] = row * r.ldp + col;
      eout[j] = row * r.ldo + col;
    }
    if (RING) {
      const int q = (int)((r.row0 + row) / r.shard_rows);
      const int ns = NS > 0 ? NS : r.nslots;
      first[j] = (q + 1) % ns;
    }
  }
  float acc[V][8];
#pragma unroll
  for (int j = 0; j < V; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[j][i] = 0.0f;
  if constexpr (RING) {
    if constexpr (NS > 0) {
#pragma unroll
      for (int i = 0; i < NS; ++i) hop_slot<NS, V>(acc, ok, ein, first, i, r);
    } else {
      for (int i = 0; i < r.nslots; ++i) hop_slot<NS, V>(acc, ok, ein, first, i, r);
    }
  } else if constexpr (NS > 0) {
#pragma unroll
    for (int s = 0; s < NS; ++s) add_slot<V>(acc, ok, ein, r.parts + s * r.slot_stride);
  } else {
    for (int s = 0; s < r.nslots; ++s) add_slot<V>(acc, ok, ein, r.parts + s * r.slot_stride);
  }
#pragma unroll
  for (int j = 0; j < V; ++j)
    if (ok[j]) __builtin_nontemporal_store(pack8(acc[j]), GLOBAL_PTR(u32x4, r.out + eout[j]));
}

template <int NS, int V>
hipError_t launch_nsv(const ReduceArgs& r, int64_t nvec, int64_t vpr, hipStream_t stream) {
  const int64_t blocks = (nvec + V * THREADS - 1) / (V * THREADS);
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const bool packed = r.ldp == r.cols && r.ldo == r.cols;
  const dim3 grid((unsigned)blocks), block(THREADS);
  if (r.ring)
    return packed ? launch_k(&reduce_chunks<NS, true, true, V>, grid, block, 0, stream, r, nvec, vpr)
                  : launch_k(&reduce_chunks<NS, false, true, V>, grid, block, 0, stream, r, nvec, vpr);
  return packed ? launch_k(&reduce_chunks<NS, true, false, V>, grid, block, 0, stream, r, nvec, vpr)
                : launch_k(&reduce_chunks<NS, false, false, V>, grid, block, 0, stream, r, nvec, vpr);
}

constexpr int64_t kSmallSumVectors = int64_t(1) << 21;

template <int NS>
hipError_t launch_ns(const ReduceArgs& r, hipStream_t stream) {
  const int64_t vpr = r.cols / 8;
  const int64_t nvec = r.rows * vpr;
  return nvec <= kSmallSumVectors ? launch_nsv<NS, 2>(r, nvec, vpr, stream)
                                  : launch_nsv<NS, 4>(r, nvec, vpr, stream);
}

}  // namespace

hipError_t launch_reduce_partials(const ReduceArgs& r, hipStream_t stream) {
  if (r.rows <= 0 || r.cols <= 0 || r.nslots <= 0) return hipSuccess;
  if (r.cols % 8 != 0 || r.ldp % 8 != 0 || r.ldo % 8 != 0) return hipErrorInvalidValue;
  // ring order: every row's shard index must lie in [0, nslots)
  if (r.ring && (r.shard_rows <= 0 || r.row0 < 0 || (r.row0 + r.rows - 1) / r.shard_rows >= r.nslots))
    return hipErrorInvalidValue;
  switch (r.nslots) {
    case 1: return launch_ns<1>(r, stream);
    case 2: return launch_ns<2>(r, stream);
    case 4: return launch_ns<4>(r, stream);
    case 8: return launch_ns<8>(r, stream);
    default: return launch_ns<0>(r, stream);
  }
}

}  // namespace ubx
