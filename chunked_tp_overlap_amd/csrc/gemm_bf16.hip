// bf16 GEMM on gfx950 matrix cores: C = bf16(A * B), fp32 accumulation.
//
// This is the per-chunk GEMM of the overlap schedule ("How to setup TP Overlap configs",
// Transformer Engine issue 1344, "num_splits": the GEMM is cut into chunks, each a GEMM
// of its own).  A chunk's A operand is read in place from the capacity-sized UserBuffer at
// the chunk's row offset ("[Feature Request] Support dynamic token counts in TP
// communication/GEMM overlap", Transformer Engine issue 3564, "Implementation approach in
// the prototype": offsets from the active first dimension).
//
// All operands row-major.  A [m, k] (lda), B [k, n] (ldb), C [m, n] (ldc); blockIdx.z
// selects a batch entry at the given element strides (the reduce-scatter side's K slices).
//
// Tiling: a 256-thread workgroup (4 waves of 64) computes a 128x128 tile of C; each wave
// owns a 64x64 quadrant as 2x2 blocks of v_mfma_f32_32x32x16_bf16.  K advances 64 at a
// time through LDS.  Every tile shape uses the same instruction and the same ascending-K
// order, so an output element's bits depend only on its own A row and B column: the
// chunking, the row offset and the tile position never change a result.
#include <hip/hip_runtime.h>

#include "ub_internal.h"

namespace ubx {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128;
constexpr int BN = 128;
constexpr int BK = 64;
constexpr int THREADS = 256;
constexpr int LDA_S = BK + 8;  // A tile row in LDS (elements); +16 B keeps b128 reads conflict-free
constexpr int LDB_S = BN + 8;  // B tile row in LDS (k-major)

struct Params {
  const uint16_t* a;
  const uint16_t* b;
  uint16_t* c;
  int64_t lda, sa, ldb, sb, ldc, sc;
  int32_t m, n, k;
};

__device__ inline uint16_t bf16_bits(float f) {
  // fptrunc to bfloat lowers to gfx950's v_cvt_pk_bf16_f32: round to nearest even.
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__global__ __launch_bounds__(THREADS) void gemm_bf16_tile128(Params p) {
  __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDA_S];
  __shared__ __attribute__((aligned(16))) uint16_t Bs[BK * LDB_S];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;
  const int wn = wave & 1;
  const int m0 = blockIdx.y * BM;
  const int n0 = blockIdx.x * BN;
  const uint16_t* A = p.a + blockIdx.z * p.sa;
  const uint16_t* B = p.b + blockIdx.z * p.sb;
  uint16_t* C = p.c + blockIdx.z * p.sc;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  const uint4 zero = make_uint4(0, 0, 0, 0);
  for (int k0 = 0; k0 < p.k; k0 += BK) {
    uint4 ra[4], rb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // A tile: 128 rows x 64 k, 8 k per lane
      const int v = tid + i * THREADS;
      const int r = v >> 3, cc = (v & 7) * 8;
      const int gm = m0 + r;
      ra[i] = gm < p.m ? *reinterpret_cast<const uint4*>(A + (int64_t)gm * p.lda + k0 + cc) : zero;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {  // B tile: 64 k x 128 cols, 8 cols per lane
      const int v = tid + i * THREADS;
      const int r = v >> 4, cc = (v & 15) * 8;
      const int gn = n0 + cc;
      rb[i] = gn < p.n ? *reinterpret_cast<const uint4*>(B + (int64_t)(k0 + r) * p.ldb + gn) : zero;
    }
    __syncthreads();  // the previous step's LDS reads are done
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v = tid + i * THREADS;
      *reinterpret_cast<uint4*>(&As[(v >> 3) * LDA_S + (v & 7) * 8]) = ra[i];
      *reinterpret_cast<uint4*>(&Bs[(v >> 4) * LDB_S + (v & 15) * 8]) = rb[i];
    }
    __syncthreads();

#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      bf16x8 af[2], bfr[2];
      const int kl = kk + (lane >> 5) * 8;  // this lane's 8 consecutive k
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const int row = wm * 64 + mi * 32 + (lane & 31);
        af[mi] = *reinterpret_cast<const bf16x8*>(&As[row * LDA_S + kl]);
      }
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int col = wn * 64 + ni * 32 + (lane & 31);
        u16x8 t;
#pragma unroll
        for (int e = 0; e < 8; ++e) t[e] = Bs[(kl + e) * LDB_S + col];
        bfr[ni] = __builtin_bit_cast(bf16x8, t);
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
    }
  }

  // 32x32 accumulator layout: lane holds column (lane & 31); element e holds row
  // 8*(e/4) + 4*(lane/32) + (e%4).
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
      const int col = n0 + wn * 64 + ni * 32 + (lane & 31);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm * 64 + mi * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
        if (row < p.m && col < p.n) C[(int64_t)row * p.ldc + col] = bf16_bits(acc[mi][ni][e]);
      }
    }
}

}  // namespace

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t stream) {
  if (g.m <= 0 || g.n <= 0 || g.batch <= 0) return hipSuccess;
  if (g.k <= 0 || g.k % BK != 0 || g.n % 8 != 0) return hipErrorInvalidValue;
  const int64_t gy = (g.m + BM - 1) / BM;
  if (gy > 65535 || g.batch > 65535) return hipErrorInvalidValue;
  Params p{g.a, g.b, g.c, g.lda, g.a_batch_stride, g.ldb, g.b_batch_stride,
           g.ldc, g.c_batch_stride, g.m, g.n, g.k};
  dim3 grid((g.n + BN - 1) / BN, static_cast<unsigned>(gy), g.batch);
  hipLaunchKernelGGL(gemm_bf16_tile128, grid, dim3(THREADS), 0, stream, p);
  return hipGetLastError();
}

}  // namespace ubx
