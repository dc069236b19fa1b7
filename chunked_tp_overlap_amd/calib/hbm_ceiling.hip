// HBM bandwidth ceiling of this part for the reduce-scatter sum's access pattern (a
// calibration program, not part of the reduction path).
//
// Three streaming kernels, each with 16-byte non-temporal accesses, 256 threads per
// workgroup and V vectors per lane in short per-workgroup chunks (the partial-sum
// reduction's launch shape):
//   read   every lane reads its vectors of S slots and folds them with XOR into one word
//          per lane, written once (reads only, in effect);
//   mix    the reduction's pattern without its arithmetic: S slot reads of each vector,
//          one 16-byte write of their XOR (S + 1 streams, S : 1 reads to writes);
//   copy   one read and one write per vector.
// Each is timed with HIP events over single launches, with a 512 MiB write between
// launches so that the 256 MiB last-level cache (MALL) holds none of the input, and the
// median is reported as algorithmic bytes / time.  Prints one JSON line per (kernel, size).
//
// Usage: hbm_ceiling [rows ...]   (default 2048 16384: [rows, 4096] bf16 slots, 8 slots)
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#define CHECK(x)                                                                            \
  do {                                                                                      \
    hipError_t e_ = (x);                                                                    \
    if (e_ != hipSuccess) {                                                                 \
      std::fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #x, hipGetErrorString(e_)); \
      std::exit(1);                                                                         \
    }                                                                                       \
  } while (0)

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
#define GLOBAL_PTR(T, p) ((__attribute__((address_space(1))) T*)(p))

constexpr int THREADS = 256;
constexpr int SLOTS = 8;
constexpr int COLS = 4096;
constexpr int64_t FLUSH_BYTES = int64_t(512) << 20;

// Workgroup b covers vectors [b V THREADS, (b + 1) V THREADS) of each slot, clipped to nvec.
template <int V>
__global__ __launch_bounds__(THREADS) void read_kernel(const u32x4* src, int64_t slot_vec,
                                                       int64_t nvec, uint32_t* sink) {
  const int64_t base = (int64_t)blockIdx.x * (V * THREADS) + threadIdx.x;
  uint32_t x = 0;
  for (int s = 0; s < SLOTS; ++s) {
    u32x4 v[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int64_t i = base + j * THREADS;
      v[j] = i < nvec ? __builtin_nontemporal_load(GLOBAL_PTR(const u32x4, src + s * slot_vec + i))
                      : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < V; ++j) x ^= v[j][0] ^ v[j][1] ^ v[j][2] ^ v[j][3];
  }
  sink[(int64_t)blockIdx.x * THREADS + threadIdx.x] = x;
}

template <int V>
__global__ __launch_bounds__(THREADS) void mix_kernel(const u32x4* src, int64_t slot_vec,
                                                      int64_t nvec, u32x4* dst) {
  const int64_t base = (int64_t)blockIdx.x * (V * THREADS) + threadIdx.x;
  u32x4 acc[V];
#pragma unroll
  for (int j = 0; j < V; ++j) acc[j] = u32x4{0, 0, 0, 0};
  for (int s = 0; s < SLOTS; ++s) {
    u32x4 v[V];
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int64_t i = base + j * THREADS;
      v[j] = i < nvec ? __builtin_nontemporal_load(GLOBAL_PTR(const u32x4, src + s * slot_vec + i))
                      : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < V; ++j) acc[j] ^= v[j];
  }
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int64_t i = base + j * THREADS;
    if (i < nvec) __builtin_nontemporal_store(acc[j], GLOBAL_PTR(u32x4, dst + i));
  }
}

template <int V>
__global__ __launch_bounds__(THREADS) void copy_kernel(const u32x4* src, int64_t nvec, u32x4* dst) {
  const int64_t base = (int64_t)blockIdx.x * (V * THREADS) + threadIdx.x;
  u32x4 v[V];
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int64_t i = base + j * THREADS;
    v[j] = i < nvec ? __builtin_nontemporal_load(GLOBAL_PTR(const u32x4, src + i)) : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int j = 0; j < V; ++j) {
    const int64_t i = base + j * THREADS;
    if (i < nvec) __builtin_nontemporal_store(v[j], GLOBAL_PTR(u32x4, dst + i));
  }
}

__global__ void flush_kernel(u32x4* p, int64_t n, uint32_t salt) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = u32x4{salt, (uint32_t)i, salt, (uint32_t)(i >> 32)};
}

template <class F>
double median_us(F launch, u32x4* flush, int reps) {
  hipEvent_t e0, e1;
  CHECK(hipEventCreate(&e0));
  CHECK(hipEventCreate(&e1));
  std::vector<double> t;
  for (int r = 0; r < reps + 3; ++r) {
    hipLaunchKernelGGL(flush_kernel, dim3(4096), dim3(256), 0, 0, flush,
                       FLUSH_BYTES / 16, (uint32_t)r);
    CHECK(hipGetLastError());
    CHECK(hipEventRecord(e0, 0));
    launch();
    CHECK(hipGetLastError());
    CHECK(hipEventRecord(e1, 0));
    CHECK(hipEventSynchronize(e1));
    float ms = 0.0f;
    CHECK(hipEventElapsedTime(&ms, e0, e1));
    if (r >= 3) t.push_back(ms * 1e3);  // the first three are warm-up
  }
  CHECK(hipEventDestroy(e0));
  CHECK(hipEventDestroy(e1));
  std::sort(t.begin(), t.end());
  return t[t.size() / 2];
}

int main(int argc, char** argv) {
  std::vector<int64_t> rows;
  for (int i = 1; i < argc; ++i) {
    const long long r = std::atoll(argv[i]);
    if (r < 8 || r > 32768) {
      std::fprintf(stderr, "rows must be in [8, 32768]\n");
      return 2;
    }
    rows.push_back(r);
  }
  if (rows.empty()) rows = {2048, 16384};
  const int64_t max_rows = *std::max_element(rows.begin(), rows.end());
  const int64_t slot_vec_max = max_rows * COLS / 8;  // 16-byte vectors per slot
  u32x4 *src = nullptr, *dst = nullptr, *flush = nullptr;
  uint32_t* sink = nullptr;
  CHECK(hipMalloc(&src, (size_t)(SLOTS * slot_vec_max) * 16));
  CHECK(hipMalloc(&dst, (size_t)slot_vec_max * 16));
  CHECK(hipMalloc(&flush, (size_t)FLUSH_BYTES));
  CHECK(hipMalloc(&sink, (size_t)(slot_vec_max / THREADS + 1) * THREADS * 4));
  hipLaunchKernelGGL(flush_kernel, dim3(4096), dim3(256), 0, 0, src, SLOTS * slot_vec_max, 7u);
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  constexpr int V = 4;
  for (const int64_t r : rows) {
    const int64_t nvec = r * COLS / 8;  // vectors per slot at this size
    const unsigned blocks = (unsigned)((nvec + V * THREADS - 1) / (V * THREADS));
    const double rd = median_us([&] {
      hipLaunchKernelGGL(read_kernel<V>, dim3(blocks), dim3(THREADS), 0, 0, src, slot_vec_max, nvec, sink);
    }, flush, 20);
    const double mx = median_us([&] {
      hipLaunchKernelGGL(mix_kernel<V>, dim3(blocks), dim3(THREADS), 0, 0, src, slot_vec_max, nvec, dst);
    }, flush, 20);
    const double cp = median_us([&] {
      hipLaunchKernelGGL(copy_kernel<V>, dim3(blocks), dim3(THREADS), 0, 0, src, nvec, dst);
    }, flush, 20);
    const double b_rd = (double)SLOTS * nvec * 16, b_mx = (double)(SLOTS + 1) * nvec * 16,
                 b_cp = 2.0 * nvec * 16;
    std::printf("{\"rows\": %lld, \"cols\": %d, \"slots\": %d, "
                "\"read\": {\"bytes\": %.0f, \"us\": %.2f, \"tbs\": %.3f}, "
                "\"mix_8_1\": {\"bytes\": %.0f, \"us\": %.2f, \"tbs\": %.3f}, "
                "\"copy\": {\"bytes\": %.0f, \"us\": %.2f, \"tbs\": %.3f}}\n",
                (long long)r, COLS, SLOTS, b_rd, rd, b_rd / rd / 1e6, b_mx, mx, b_mx / mx / 1e6, b_cp,
                cp, b_cp / cp / 1e6);
    std::fflush(stdout);
  }
  CHECK(hipFree(src));
  CHECK(hipFree(dst));
  CHECK(hipFree(flush));
  CHECK(hipFree(sink));
  return 0;
}
