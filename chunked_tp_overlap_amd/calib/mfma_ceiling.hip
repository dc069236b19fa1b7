// Matrix-core ceiling of this part under its power limit (a calibration program, not part of
// the GEMM path).
//
// Every wave runs a GEMM's inner work without its memory side, repeated `iters` times over
// register operands drawn from random data:
//   bf16: the 16 v_mfma_f32_32x32x16_bf16 of one 32-deep k-step of a 128 x 64 wave tile
//         (4 x 2 blocks of 32 x 32, two 16-deep sub-steps);
//   fp8:  the 8 v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 x E4M3, unit scales) of one 64-deep
//         k-step of the same wave tile, as the FP8 GEMM;
//   bf16_16x16x32: the 32 v_mfma_f32_16x16x32_bf16 (8 x 4 blocks of 16 x 16) that cover the
//         same bf16 step with the smaller instruction, as the bf16 GEMM.
// Every variant is compiled for at most 256 registers per lane (two waves per SIMD), so one
// and two waves per SIMD run the same code.  One workgroup per CU (its LDS request leaves
// room for no second), 4 or 8 waves (one or two per SIMD, as the GEMMs' four-wave and
// ping-pong kernels), on a chosen number of CUs.  What this sustains is the most any GEMM built on
// this instruction can reach with that many CUs busy, whatever its memory side does.
//
// Lane 0 of each workgroup records the shader clock counter (s_memtime) and the constant
// 100 MHz counter (s_memrealtime) before and after the loop; their ratio is the shader
// clock the workgroup ran at.  Prints one JSON line per (instruction, waves, CUs).
//
// Usage: mfma_ceiling [seconds_per_sustained_run [busy_cu_count ...]]
//        (defaults: 0.5 s; 142, 192 and every CU of the device)
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int FM = 4, FN = 2, SUBS = 2;          // the GEMM's 128 x 64 wave tile, BK = 32
enum Kind { kBf16 = 0, kFp8 = 1, kBf16Small = 2 };
// flops per wave per iteration: bf16 a 32-deep step, fp8 a 64-deep step of the wave tile
constexpr double flop_per_iter_wave(int kind) { return 2.0 * 128 * 64 * (kind == kFp8 ? 64 : 32); }
constexpr double PEAK[3] = {2516.6, 5033.2, 2516.6};  // dense TFLOP/s
const char* const KIND_NAME[3] = {"bf16", "fp8", "bf16_16x16x32"};
constexpr size_t LDS_FORCE_ONE_PER_CU = 96 * 1024;  // two would need 192 KiB of 160

#define CHECK(x)                                                                       \
  do {                                                                                 \
    hipError_t e_ = (x);                                                               \
    if (e_ != hipSuccess) {                                                            \
      std::fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_)); \
      std::exit(1);                                                                    \
    }                                                                                  \
  } while (0)

template <int WAVES, int KIND>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mfma_loop(const bf16x8* src, float* sink, unsigned long long* clk, int iters) {
  extern __shared__ unsigned char lds[];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // fragments: 12 distinct 16-byte vectors per lane, from a 64-lane x 12 table per wave
  // slot; fp8 operands are 32 bytes, two neighbouring vectors
  const bf16x8* s = src + ((size_t)(wave % 8) * 64 + lane) * (SUBS * (FM + FN));
  bf16x8 a[SUBS][FM], b[SUBS][FN];
#pragma unroll
  for (int u = 0; u < SUBS; ++u) {
#pragma unroll
    for (int i = 0; i < FM; ++i) a[u][i] = s[u * (FM + FN) + i];
#pragma unroll
    for (int j = 0; j < FN; ++j) b[u][j] = s[u * (FM + FN) + FM + j];
  }
  i32x8 a8[FM], b8[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
    a8[i] = __builtin_shufflevector(__builtin_bit_cast(i32x4_t, a[0][i]),
                                    __builtin_bit_cast(i32x4_t, a[1][i]), 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
  for (int j = 0; j < FN; ++j)
    b8[j] = __builtin_shufflevector(__builtin_bit_cast(i32x4_t, b[0][j]),
                                    __builtin_bit_cast(i32x4_t, b[1][j]), 0, 1, 2, 3, 4, 5, 6, 7);
  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  f32x4 acc4[2 * FM][2 * FN];  // bf16_16x16x32: 16 x 16 blocks over the same wave tile
#pragma unroll
  for (int i = 0; i < 2 * FM; ++i)
#pragma unroll
    for (int j = 0; j < 2 * FN; ++j) acc4[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  lds[threadIdx.x] = 0;  // the LDS request only limits occupancy
  __syncthreads();
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
    if constexpr (KIND == kBf16Small) {
      // a 16-row block takes row block i/2 and k half i%2 of the 32 x 32 operands' vectors:
      // any 8 bf16 per lane serve, the operand values only set the data the units switch
#pragma unroll
      for (int i = 0; i < 2 * FM; ++i)
#pragma unroll
        for (int j = 0; j < 2 * FN; ++j)
          acc4[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i & 1][i >> 1], b[j & 1][j >> 1],
                                                               acc4[i][j], 0, 0, 0);
    } else if constexpr (KIND == kFp8) {
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a8[i], b8[j], acc[i][j], 0, 0,
                                                                      0, 127, 0, 127);
    } else {
#pragma unroll
      for (int u = 0; u < SUBS; ++u)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[u][i], b[u][j], acc[i][j], 0, 0, 0);
    }
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < 2 * FM; ++i)
#pragma unroll
    for (int j = 0; j < 2 * FN; ++j) sum += acc4[i][j][0] + acc4[i][j][1] + acc4[i][j][2] + acc4[i][j][3];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) sum += acc[i][j][e];
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = sum;
  if (threadIdx.x == 0) {
    clk[blockIdx.x * 4 + 0] = t0;
    clk[blockIdx.x * 4 + 1] = t1;
    clk[blockIdx.x * 4 + 2] = r0;
    clk[blockIdx.x * 4 + 3] = r1;
  }
}

struct Result {
  double seconds, tflops, clock_mhz;
};

// `launches` back-to-back launches of `iters` iterations on `cus` workgroups.
template <int WAVES, int KIND>
Result run(const bf16x8* src, float* sink, unsigned long long* clk, int cus, int iters,
           int launches) {
  const dim3 grid(cus), block(64 * WAVES);
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  CHECK(hipEventRecord(e0, 0));
  for (int l = 0; l < launches; ++l)
    hipLaunchKernelGGL((mfma_loop<WAVES, KIND>), grid, block, LDS_FORCE_ONE_PER_CU, 0, src, sink,
                       clk, iters);
  CHECK(hipGetLastError());
  CHECK(hipEventRecord(e1, 0));
  CHECK(hipEventSynchronize(e1));
  float ms = 0.0f;
  CHECK(hipEventElapsedTime(&ms, e0, e1));
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  // clock of the last launch: shader-clock ticks over 100 MHz ticks, averaged over workgroups
  std::vector<unsigned long long> h((size_t)cus * 4);
  CHECK(hipMemcpy(h.data(), clk, h.size() * sizeof(unsigned long long), hipMemcpyDeviceToHost));
  double ratio = 0.0;
  int n = 0;
  for (int w = 0; w < cus; ++w) {
    const double dt = (double)(h[w * 4 + 1] - h[w * 4 + 0]);
    const double dr = (double)(h[w * 4 + 3] - h[w * 4 + 2]);
    if (dr > 0) {
      ratio += dt / dr;
      ++n;
    }
  }
  Result r;
  r.seconds = ms * 1e-3;
  r.tflops = flop_per_iter_wave(KIND) * WAVES * cus * (double)iters * launches / r.seconds / 1e12;
  r.clock_mhz = n ? 100.0 * ratio / n : 0.0;
  return r;
}

int main(int argc, char** argv) {
  const double sustained_s = argc > 1 ? std::atof(argv[1]) : 0.5;
  if (!(sustained_s > 0.0 && sustained_s <= 10.0)) {
    std::fprintf(stderr, "seconds_per_sustained_run must be in (0, 10]\n");
    return 2;
  }
  int dev = 0, ncu = 0;
  CHECK(hipGetDevice(&dev));
  CHECK(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev));
  std::vector<int> busy;
  for (int i = 2; i < argc; ++i) {
    const int c = std::atoi(argv[i]);
    if (c < 1 || c > ncu) {
      std::fprintf(stderr, "busy_cu_count must be in [1, %d]\n", ncu);
      return 2;
    }
    busy.push_back(c);
  }
  if (busy.empty()) busy = {std::min(142, ncu), std::min(192, ncu), ncu};
  for (const void* k : {reinterpret_cast<const void*>(&mfma_loop<4, kBf16>),
                        reinterpret_cast<const void*>(&mfma_loop<8, kBf16>),
                        reinterpret_cast<const void*>(&mfma_loop<4, kFp8>),
                        reinterpret_cast<const void*>(&mfma_loop<8, kFp8>),
                        reinterpret_cast<const void*>(&mfma_loop<4, kBf16Small>),
                        reinterpret_cast<const void*>(&mfma_loop<8, kBf16Small>)})
    CHECK(hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize,
                              (int)LDS_FORCE_ONE_PER_CU));

  // random bf16 operands in [-1, 1): 8 wave slots x 64 lanes x 12 vectors x 8 values
  const size_t nvec = 8 * 64 * SUBS * (FM + FN);
  std::vector<uint16_t> host(nvec * 8);
  std::mt19937 gen(20261202u);
  std::uniform_real_distribution<float> dist(-1.0f, 1.0f);
  for (auto& v : host) {
    const float f = dist(gen);
    uint32_t u;
    std::memcpy(&u, &f, 4);
    v = (uint16_t)(u >> 16);
    // read as E4M3 bytes too: no byte may be a NaN code (S.1111.111)
    if ((v & 0x7F) == 0x7F) v ^= 1;
    if (((v >> 8) & 0x7F) == 0x7F) v ^= 0x100;
  }
  bf16x8* src = nullptr;
  float* sink = nullptr;
  unsigned long long* clk = nullptr;
  CHECK(hipMalloc(&src, host.size() * 2));
  CHECK(hipMalloc(&sink, (size_t)ncu * 512 * sizeof(float)));
  CHECK(hipMalloc(&clk, (size_t)ncu * 4 * sizeof(unsigned long long)));
  CHECK(hipMemcpy(src, host.data(), host.size() * 2, hipMemcpyHostToDevice));

  // iterations per microsecond at 2.4 GHz with two waves per SIMD: 16 MFMAs of 32 cycles per
  // wave per iteration, two waves -> 1024 cycles per iteration
  const double iters_per_us = 2400.0 / 1024.0;
  run<8, kBf16>(src, sink, clk, ncu, 100, 10);  // warm-up
  for (int kind : {kBf16, kFp8, kBf16Small}) {
    for (int waves : {8, 4}) {
      for (int cus : busy) {
        const double per_wave = waves == 8 ? 1.0 : 2.0;  // one wave per SIMD issues half as often
        // bursts: 32 launches of ~80 us (one qkv step's launches)
        const int it_b = (int)(80.0 * iters_per_us * per_wave);
        // sustained: one launch of the requested length
        const int it_s = (int)(sustained_s * 1e6 * iters_per_us * per_wave);
        // the sustained run first, so that the bursts start with the clock already settled
        // (after an idle gap the clock takes milliseconds to ramp up)
        auto go = [&](int iters, int launches) {
          if (kind == kBf16Small)
            return waves == 8 ? run<8, kBf16Small>(src, sink, clk, cus, iters, launches)
                              : run<4, kBf16Small>(src, sink, clk, cus, iters, launches);
          if (kind == kFp8)
            return waves == 8 ? run<8, kFp8>(src, sink, clk, cus, iters, launches)
                              : run<4, kFp8>(src, sink, clk, cus, iters, launches);
          return waves == 8 ? run<8, kBf16>(src, sink, clk, cus, iters, launches)
                            : run<4, kBf16>(src, sink, clk, cus, iters, launches);
        };
        const Result s = go(it_s, 1);
        const Result b = go(it_b, 32);
        const double peak = PEAK[kind];
        std::printf("{\"kind\": \"%s\", \"peak_tflops\": %.1f, \"waves_per_simd\": %d, \"cus\": %d, "
                    "\"bursts_32x80us\": {\"tflops\": %.1f, \"pct_of_peak\": %.1f, \"clock_mhz\": %.0f, \"ms\": %.3f}, "
                    "\"sustained\": {\"tflops\": %.1f, \"pct_of_peak\": %.1f, \"clock_mhz\": %.0f, \"ms\": %.1f}}\n",
                    KIND_NAME[kind], peak, waves / 4, cus, b.tflops,
                    100.0 * b.tflops / peak, b.clock_mhz, b.seconds * 1e3, s.tflops,
                    100.0 * s.tflops / peak, s.clock_mhz, s.seconds * 1e3);
        std::fflush(stdout);
      }
    }
  }
  CHECK(hipFree(src));
  CHECK(hipFree(sink));
  CHECK(hipFree(clk));
  return 0;
}
