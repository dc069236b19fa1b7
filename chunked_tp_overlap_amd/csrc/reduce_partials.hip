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
// HBM-bound: every element is read tp times and written once (2 (tp + 1) bytes per output
// element).  Each lane handles 16-byte vectors (8 elements); consecutive lanes take
// consecutive vectors; every lane keeps two vectors' worth of loads (2 tp x 16 bytes) in
// flight.  The partials are read exactly once, so loads and stores are non-temporal.  When
// the partial rows and the output rows are both packed (leading dimension == cols) the
// region is one flat range of vectors; otherwise each vector's row is recovered by
// division.
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

// Sum of the NS (or nslots, when NS == 0) partials of the vector at element offset `e`.
template <int NS>
__device__ inline u32x4 reduce_vec(const uint16_t* parts, int64_t slot_stride, int nslots,
                                   int64_t e) {
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.0f;
  if constexpr (NS > 0) {
    u32x4 x[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s)
      x[s] = __builtin_nontemporal_load(GLOBAL_PTR(const u32x4, parts + s * slot_stride + e));
#pragma unroll
    for (int s = 0; s < NS; ++s) add8(acc, x[s]);
  } else {
    for (int s = 0; s < nslots; ++s)
      add8(acc, __builtin_nontemporal_load(GLOBAL_PTR(const u32x4, parts + s * slot_stride + e)));
  }
  return pack8(acc);
}

// Packed rows: vectors v = 0 .. nvec-1 at element offset 8 v in every slot and in out.
template <int NS>
__global__ __launch_bounds__(THREADS) void reduce_packed(ReduceArgs r, int64_t nvec) {
  const int64_t stride = (int64_t)gridDim.x * THREADS;
  int64_t v = (int64_t)blockIdx.x * THREADS + threadIdx.x;
  for (; v + stride < nvec; v += 2 * stride) {
    const u32x4 a = reduce_vec<NS>(r.parts, r.slot_stride, r.nslots, v * 8);
    const u32x4 b = reduce_vec<NS>(r.parts, r.slot_stride, r.nslots, (v + stride) * 8);
    __builtin_nontemporal_store(a, GLOBAL_PTR(u32x4, r.out + v * 8));
    __builtin_nontemporal_store(b, GLOBAL_PTR(u32x4, r.out + (v + stride) * 8));
  }
  if (v < nvec)
    __builtin_nontemporal_store(reduce_vec<NS>(r.parts, r.slot_stride, r.nslots, v * 8),
                                GLOBAL_PTR(u32x4, r.out + v * 8));
}

// Strided rows (ldp or ldo != cols).
template <int NS>
__global__ __launch_bounds__(THREADS) void reduce_strided(ReduceArgs r) {
  const int64_t vpr = r.cols >> 3;  // 16-byte vectors per row
  const int64_t total = r.rows * vpr;
  for (int64_t v = (int64_t)blockIdx.x * THREADS + threadIdx.x; v < total;
       v += (int64_t)gridDim.x * THREADS) {
    const int64_t row = v / vpr;
    const int64_t col = (v - row * vpr) * 8;
    __builtin_nontemporal_store(reduce_vec<NS>(r.parts, r.slot_stride, r.nslots, row * r.ldp + col),
                                GLOBAL_PTR(u32x4, r.out + row * r.ldo + col));
  }
}

template <int NS>
hipError_t launch_ns(const ReduceArgs& r, hipStream_t stream) {
  const int64_t nvec = r.rows * (r.cols / 8);
  // enough waves to cover HBM latency: up to 16 workgroups of 4 waves per CU
  int64_t blocks = (nvec + THREADS - 1) / THREADS;
  if (blocks > 256 * 16) blocks = 256 * 16;
  if (r.ldp == r.cols && r.ldo == r.cols)
    hipLaunchKernelGGL(reduce_packed<NS>, dim3((unsigned)blocks), dim3(THREADS), 0, stream, r, nvec);
  else
    hipLaunchKernelGGL(reduce_strided<NS>, dim3((unsigned)blocks), dim3(THREADS), 0, stream, r);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_reduce_partials(const ReduceArgs& r, hipStream_t stream) {
  if (r.rows <= 0 || r.cols <= 0 || r.nslots <= 0) return hipSuccess;
  if (r.cols % 8 != 0 || r.ldp % 8 != 0 || r.ldo % 8 != 0) return hipErrorInvalidValue;
  switch (r.nslots) {
    case 1: return launch_ns<1>(r, stream);
    case 2: return launch_ns<2>(r, stream);
    case 4: return launch_ns<4>(r, stream);
    case 8: return launch_ns<8>(r, stream);
    default: return launch_ns<0>(r, stream);
  }
}

}  // namespace ubx
