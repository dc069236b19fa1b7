// bf16 -> FP8 (E4M3) quantization of UserBuffer rows with a per-tensor scale.
//
// Quantized UserBuffers: "[Feature Request] Support dynamic token counts in TP
// communication/GEMM overlap" (Transformer Engine issue 3564), "Implementation approach in
// the prototype", names them and leaves them outside the first scope; the reading taken
// for this extension (the pages give no format or rule):
//
//   q = sat(RNE_e4m3(fp32(x * scale)))
//
// x * scale is one IEEE fp32 multiply; the result is rounded to the nearest OCP E4M3 value
// (bias 7, 3 significand bits, subnormal spacing 2^-9), ties to even; magnitudes beyond
// 448 (and infinities) saturate to 448; NaN stays NaN (0x7F with its sign); zeros keep
// their sign.  The rounding is done on the fp32 bits with integer operations, so it is
// exactly that definition for every input.
//
// HBM-bound: 2 bytes read and 1 written per element; a lane converts 8 elements (16 bytes
// in, 8 out) per vector, four vectors per lane, one short chunk of rows per workgroup.
#include <hip/hip_runtime.h>

#include "ub_internal.h"

namespace ubx {
namespace {

constexpr int THREADS = 256;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
#define GLOBAL_PTR(T, p) ((__attribute__((address_space(1))) T*)(p))

__device__ inline uint32_t e4m3(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;                 // NaN
  if (a >= 0x43E00000u) return sign | 0x7Eu;                // >= 448 (and inf): saturate
  if (a >= 0x3C800000u) {                                   // >= 2^-6: normal E4M3
    // round the 23-bit fp32 significand to 3 bits, ties to even (a carry moves the
    // exponent up), then rebias the exponent from 127 to 7
    const uint32_t r = (a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20;
    return sign | (r - (120u << 3));
  }
  // subnormal range: multiples of 2^-9 (8 * 2^-9 = 2^-6 is code 0x08, the smallest normal)
  return sign | (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.0f);
}

constexpr int V = 4;  // vectors per lane

__device__ inline u32x2 quantize8(u32x4 x, float scale) {
  uint32_t q[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    q[2 * i] = e4m3(__uint_as_float(x[i] << 16) * scale);
    q[2 * i + 1] = e4m3(__uint_as_float(x[i] & 0xFFFF0000u) * scale);
  }
  u32x2 o;
  o[0] = q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24);
  o[1] = q[4] | (q[5] << 8) | (q[6] << 16) | (q[7] << 24);
  return o;
}

// dst row r (stride ldd bytes) = quantized src row r (stride lds elements), cols elements.
// Workgroup b converts vectors [b V THREADS, (b + 1) V THREADS) of 8 elements each; lane t
// takes vectors t, t + THREADS, ... (all V loads in flight before the conversions).
__global__ __launch_bounds__(THREADS) void quantize_rows(const uint16_t* src, int64_t lds,
                                                         uint8_t* dst, int64_t ldd, int64_t rows,
                                                         int64_t cols, float scale) {
  const int64_t vpr = cols / 8;
  const int64_t total = rows * vpr;
  const int64_t base = (int64_t)blockIdx.x * (V * THREADS) + threadIdx.x;
  u32x4 x[V];
  int64_t row[V], col[V];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int64_t v = base + j * THREADS;
    row[j] = v / vpr;
    col[j] = (v - row[j] * vpr) * 8;
    if (v < total)
      x[j] = __builtin_nontemporal_load(GLOBAL_PTR(const u32x4, src + row[j] * lds + col[j]));
  }
#pragma unroll
  for (int j = 0; j < V; ++j)
    if (base + j * THREADS < total)
      __builtin_nontemporal_store(quantize8(x[j], scale),
                                  GLOBAL_PTR(u32x2, dst + row[j] * ldd + col[j]));
}

}  // namespace

hipError_t launch_quantize_e4m3(const uint16_t* src, int64_t lds, uint8_t* dst, int64_t ldd,
                                int64_t rows, int64_t cols, float scale, hipStream_t stream) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  if (cols % 8 != 0 || lds % 8 != 0 || ldd % 8 != 0) return hipErrorInvalidValue;
  const int64_t blocks = (rows * (cols / 8) + V * THREADS - 1) / (V * THREADS);
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  return launch_k(&quantize_rows, dim3((unsigned)blocks), dim3(THREADS), 0, stream, src, lds, dst,
                  ldd, rows, cols, scale);
}

}  // namespace ubx
