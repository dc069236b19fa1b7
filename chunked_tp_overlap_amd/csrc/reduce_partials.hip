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
// HBM-bound: every element is read tp times and written once, 16 bytes per lane per
// access, consecutive lanes on consecutive 16-byte vectors of a row.
#include <hip/hip_runtime.h>

#include "ub_internal.h"

namespace ubx {
namespace {

constexpr int THREADS = 256;

__device__ inline float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ inline uint32_t pack2(float a, float b) {
  const uint32_t x = __builtin_bit_cast(uint16_t, static_cast<__bf16>(a));  // RNE
  const uint32_t y = __builtin_bit_cast(uint16_t, static_cast<__bf16>(b));
  return x | (y << 16);
}

__global__ __launch_bounds__(THREADS) void reduce_partials_v8(ReduceArgs r) {
  const int64_t vpr = r.cols >> 3;  // 8-element vectors per row
  const int64_t total = r.rows * vpr;
  for (int64_t v = (int64_t)blockIdx.x * THREADS + threadIdx.x; v < total;
       v += (int64_t)gridDim.x * THREADS) {
    const int64_t row = v / vpr;
    const int64_t col = (v - row * vpr) * 8;
    const uint16_t* p = r.parts + row * r.ldp + col;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
    for (int s = 0; s < r.nslots; ++s) {
      const uint4 x = *reinterpret_cast<const uint4*>(p + s * r.slot_stride);
      acc[0] += lo_bf16(x.x); acc[1] += hi_bf16(x.x);
      acc[2] += lo_bf16(x.y); acc[3] += hi_bf16(x.y);
      acc[4] += lo_bf16(x.z); acc[5] += hi_bf16(x.z);
      acc[6] += lo_bf16(x.w); acc[7] += hi_bf16(x.w);
    }
    uint4 o;
    o.x = pack2(acc[0], acc[1]);
    o.y = pack2(acc[2], acc[3]);
    o.z = pack2(acc[4], acc[5]);
    o.w = pack2(acc[6], acc[7]);
    *reinterpret_cast<uint4*>(r.out + row * r.ldo + col) = o;
  }
}

}  // namespace

hipError_t launch_reduce_partials(const ReduceArgs& r, hipStream_t stream) {
  if (r.rows <= 0 || r.cols <= 0 || r.nslots <= 0) return hipSuccess;
  if (r.cols % 8 != 0) return hipErrorInvalidValue;
  const int64_t total = r.rows * (r.cols / 8);
  int64_t blocks = (total + THREADS - 1) / THREADS;
  if (blocks > 256 * 16) blocks = 256 * 16;
  hipLaunchKernelGGL(reduce_partials_v8, dim3(static_cast<unsigned>(blocks)), dim3(THREADS), 0,
                     stream, r);
  return hipGetLastError();
}

}  // namespace ubx
