// Host-only stand-ins for the library's device-side entry points, for the sanitizer build
// of the C ABI's host code (ub_api.cpp, ub_plan.cpp) on a machine without a GPU.  Every
// launcher reports hipErrorNotSupported; the argument checks under test run before any of
// them.  The tile lists answer for one shape only (256 x 256), enough to exercise the
// forced-tile check's rejection path.
#include "ub_internal.h"

namespace ubx {

uint32_t* ready_flags_base(hipError_t* err) {
  *err = hipErrorNotSupported;
  return nullptr;
}
hipError_t launch_gemm_bf16(const GemmArgs&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_gemm_bf16_units(const GemmArgs&, const GemmUnits&, hipStream_t) {
  return hipErrorNotSupported;
}
bool gemm_bf16_tile_supported(int tile_m, int tile_n) { return tile_m == 256 && tile_n == 256; }
bool gemm_fp8_tile_supported(int tile_m, int tile_n) { return tile_m == 256 && tile_n == 256; }
bool gemm_fp8_shape_supported(const GemmF8Args&) { return true; }
hipError_t launch_gemm_fp8_units(const GemmF8Args&, const GemmUnits&, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_quantize_e4m3(const uint16_t*, int64_t, uint8_t*, int64_t, int64_t, int64_t,
                                float, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_reduce_partials(const ReduceArgs&, hipStream_t) { return hipErrorNotSupported; }
unsigned char* static_scratch_base(hipError_t* err) {
  *err = hipErrorNotSupported;
  return nullptr;
}
hipError_t launch_clear_words(uint32_t*, int64_t, hipStream_t) { return hipErrorNotSupported; }
SegPlan choose_segmentation(int64_t, int64_t, int64_t, int32_t) { return SegPlan{}; }

}  // namespace ubx
