// The library's fixed device scratch for callers that cannot allocate: a file-scope device
// array that holds the reduce-scatter partial slots and the fused sum's tile counters of
// ub_gemm_rs_chunked_noalloc (the same layout the registered workspace has), and the fill
// kernel that clears its counter words before a fused call.
//
// The array lives in the code object, one copy per GPU, for as long as the process: no call
// allocates it.  Host code never uses the array's name as an address (on the host it is a
// stand-in, not device memory): static_scratch_base() takes each device's address once
// with hipGetSymbolAddress, with that device current, and the kernels receive that pointer.
// Every call on one GPU shares the array, so calls that overlap on a GPU race.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>

#include "ub_internal.h"

namespace ubx {
namespace {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

__global__ void clear_words(uint32_t* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

}  // namespace

unsigned char* static_scratch_base(hipError_t* err) {
  static std::mutex mu;
  static std::map<int, unsigned char*> by_device;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *err = e;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  auto it = by_device.find(dev);
  if (it != by_device.end()) return it->second;
  void* ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !ptr) {
    *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
    return nullptr;
  }
  by_device[dev] = static_cast<unsigned char*>(ptr);
  return by_device[dev];
}

hipError_t launch_clear_words(uint32_t* p, int64_t n, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  constexpr int kThreads = 256;
  const int64_t blocks = (n + kThreads - 1) / kThreads;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  return launch_k(&clear_words, dim3((unsigned)blocks), dim3(kThreads), 0, stream, p, n);
}

}  // namespace ubx
