// The C ABI's host-side argument checking under AddressSanitizer and UndefinedBehavior-
// Sanitizer, on the CPU: registration, the active-shape constraint list, plans, the GEMM
// entry points' rejections (which come before any HIP call), debug settings and messages,
// then a randomized sweep of arguments through every entry point.  Device pointers are
// fake (never dereferenced by host code); calls that pass every check reach a HIP call,
// which fails without a GPU (UB_ERR_HIP) or reaches a stubbed launcher.  Any sanitizer
// report aborts the process (halt_on_error).
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>

#include "ub.h"

#define CHECK(cond)                                                      \
  do {                                                                   \
    if (!(cond)) {                                                       \
      std::printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #cond);        \
      return 1;                                                          \
    }                                                                    \
  } while (0)

static void* fake(uintptr_t off = 0) { return reinterpret_cast<void*>(uintptr_t(1) << 40 | off); }

int main() {
  size_t ub_bytes = 0, ws_bytes = 0;
  CHECK(ub_required_bytes(512, 256, 2, UB_DTYPE_BF16, &ub_bytes, &ws_bytes) == UB_OK);
  CHECK(ub_bytes == 512 * 256 * 2 && ws_bytes > 2 * 512 * 256 * 2);
  CHECK(ub_required_bytes(510, 256, 4, UB_DTYPE_BF16, nullptr, nullptr) == UB_ERR_TP_DIVISIBILITY);
  CHECK(ub_required_bytes(512, 256, 2, UB_DTYPE_FP16, nullptr, nullptr) == UB_ERR_DTYPE);
  CHECK(ub_required_bytes(int64_t(1) << 40, 1 << 20, 2, UB_DTYPE_BF16, nullptr, nullptr) ==
        UB_ERR_INVALID_ARG);

  ub_handle_t h = nullptr;
  CHECK(ub_init(&h, 512, 256, 2, UB_DTYPE_BF16, fake(), ub_bytes - 2, nullptr, 0) ==
        UB_ERR_BUFFER_TOO_SMALL);
  CHECK(ub_init(&h, 512, 256, 2, UB_DTYPE_BF16, fake(2), ub_bytes, nullptr, 0) == UB_ERR_INVALID_ARG);
  CHECK(ub_init(&h, 512, 256, 2, UB_DTYPE_BF16, fake(), ub_bytes, fake(), ws_bytes - 1) ==
        UB_ERR_BUFFER_TOO_SMALL);
  CHECK(ub_init(&h, 512, 256, 2, UB_DTYPE_BF16, fake(), ub_bytes, fake(), ws_bytes) == UB_OK);

  // the active-shape constraint list, in its order; state unchanged on error
  int64_t shape[2] = {256, 256}, got[2];
  CHECK(ub_set_active_shape(h, shape, 3) == UB_ERR_NDIM);
  int64_t zero[2] = {0, 256};
  CHECK(ub_set_active_shape(h, zero, 2) == UB_ERR_ZERO_DIM);
  int64_t big[2] = {1024, 256};
  CHECK(ub_set_active_shape(h, big, 2) == UB_ERR_CAPACITY);
  int64_t hid[2] = {256, 128};
  CHECK(ub_set_active_shape(h, hid, 2) == UB_ERR_HIDDEN_MISMATCH);
  int64_t odd[2] = {255, 256};
  CHECK(ub_set_active_shape(h, odd, 2) == UB_ERR_TP_DIVISIBILITY);
  CHECK(ub_get_active_shape(h, got) == UB_OK && got[0] == 512);
  CHECK(std::strlen(ub_last_error(h)) > 0);
  CHECK(ub_set_active_shape(h, shape, 2) == UB_OK);

  ub_overlap_cfg_t cfg;
  ub_overlap_cfg_default(&cfg);
  ub_plan_unit_t units[16];
  int32_t nu = 0, ns = 0;
  CHECK(ub_get_plan(h, &cfg, UB_OP_AG, units, 16, &nu, &ns) == UB_OK && nu == 2);
  CHECK(ub_get_plan(h, &cfg, UB_OP_AG, nullptr, 4, &nu, &ns) == UB_ERR_INVALID_ARG);

  // GEMM rejections before any HIP call
  CHECK(ub_gemm_ag_chunked(h, nullptr, 384, 384, fake(), 384, &cfg, nullptr) == UB_ERR_INVALID_ARG);
  CHECK(ub_gemm_ag_chunked(h, fake(), 380, 384, fake(), 384, &cfg, nullptr) == UB_ERR_INVALID_ARG);
  CHECK(ub_gemm_ag_chunked(h, fake(), 384, 384, fake(), 384, nullptr, nullptr) == UB_ERR_INVALID_ARG);
  CHECK(ub_gemm_rs_chunked(h, fake(), 255, 256, fake(), 256, fake(), 256, &cfg, nullptr) ==
        UB_ERR_INVALID_ARG);
  CHECK(ub_gemm_rs_chunked(h, fake(), 36, 40, fake(), 256, fake(), 256, &cfg, nullptr) ==
        UB_ERR_UNSUPPORTED);
  ub_overlap_cfg_t bad = cfg;
  bad.fuse_reduce = 2;
  CHECK(ub_gemm_rs_chunked(h, fake(), 256, 256, fake(), 256, fake(), 256, &bad, nullptr) ==
        UB_ERR_INVALID_ARG);
  bad = cfg;
  bad.method = 9;
  CHECK(ub_gemm_ag_chunked(h, fake(), 384, 384, fake(), 384, &bad, nullptr) == UB_ERR_INVALID_ARG);
  CHECK(ub_copy_in(h, fake(), 300, 0, nullptr) == UB_ERR_INVALID_ARG);  // past the active T

  // debug settings
  CHECK(ub_debug_set(h, "nope", 1) == UB_ERR_INVALID_ARG);
  CHECK(ub_debug_set(h, nullptr, 1) == UB_ERR_INVALID_ARG);
  CHECK(ub_debug_set(h, "tile_m", 192) == UB_OK && ub_debug_set(h, "tile_n", 128) == UB_OK);
  CHECK(ub_gemm_ag_chunked(h, fake(), 384, 384, fake(), 384, &cfg, nullptr) == UB_ERR_INVALID_ARG);
  CHECK(std::strstr(ub_last_error(h), "192x128") != nullptr);
  CHECK(ub_debug_set(h, "tile_m", 0) == UB_OK && ub_debug_set(h, "tile_n", 0) == UB_OK);
  ub_tile_plan_t plan;
  CHECK(ub_debug_last_plan(h, &plan) == UB_OK && plan.cut_row == -1);
  CHECK(ub_prepare_streams(h, 0, 0) == UB_ERR_INVALID_ARG);
  CHECK(ub_debug_set(h, "nseg", 65) == UB_ERR_INVALID_ARG && ub_debug_set(h, "seg_row", -1) == UB_ERR_INVALID_ARG);
  CHECK(ub_debug_set(h, "nseg", 4) == UB_OK && ub_debug_set(h, "seg_row", 128) == UB_OK);
  CHECK(ub_debug_set(h, "nseg", 0) == UB_OK && ub_debug_set(h, "seg_row", 0) == UB_OK);
  CHECK(ub_register_scratch(h, fake(), UB_SCRATCH_MIN_BYTES - 16) == UB_ERR_BUFFER_TOO_SMALL);
  CHECK(ub_register_scratch(h, nullptr, 1 << 26) == UB_ERR_INVALID_ARG);
  CHECK(ub_register_scratch(h, fake(), 1 << 26) == UB_OK);
  CHECK(ub_register_scratch(h, nullptr, 0) == UB_OK);
  CHECK(ub_register_scratch(nullptr, fake(), 1 << 26) == UB_ERR_NOT_INITIALIZED);
  for (int s = 0; s <= 11; ++s) CHECK(ub_status_string(static_cast<ub_status_t>(s))[0] == 'U');
  CHECK(ub_destroy(h) == UB_OK);
  CHECK(ub_destroy(nullptr) == UB_OK);

  // randomized arguments through every entry point: no sanitizer report, statuses in range
  std::mt19937_64 rng(7);
  auto pick = [&](std::initializer_list<int64_t> v) {
    return *(v.begin() + rng() % v.size());
  };
  long calls = 0;
  for (int it = 0; it < 4000; ++it) {
    const int64_t cap = pick({-8, 0, 8, 64, 520, 4096, int64_t(1) << 33});
    const int64_t H = pick({-8, 0, 8, 72, 256, 4100, int64_t(1) << 31});
    const int32_t tp = static_cast<int32_t>(pick({-1, 0, 1, 2, 8, 65}));
    const ub_dtype_t dt = static_cast<ub_dtype_t>(pick({0, 1, 2, 3, 7, 1000}));
    size_t ub_b = 0, ws_b = 0;
    const ub_status_t rq = ub_required_bytes(cap, H, tp, dt, &ub_b, &ws_b);
    CHECK(rq >= UB_OK && rq <= UB_ERR_HIP);
    ub_handle_t hh = nullptr;
    const bool with_ws = dt == UB_DTYPE_BF16 && (rng() & 1);
    const ub_status_t st = ub_init(&hh, cap, H, tp, dt, fake(), ub_b + (rng() % 3) * 16 - 16,
                                   with_ws ? fake() : nullptr, with_ws ? ws_b : 0);
    ++calls;
    if (st != UB_OK) {
      CHECK(hh == nullptr);
      continue;
    }
    for (int j = 0; j < 8; ++j) {
      int64_t sh[2] = {pick({-1, 0, 8, 16, 64, 512, 4096, cap, cap + 8}), pick({H, H + 8, 0})};
      const ub_status_t s2 = ub_set_active_shape(hh, sh, static_cast<int32_t>(pick({1, 2, 2, 2})));
      CHECK(s2 >= UB_OK && s2 <= UB_ERR_HIP);
      ub_overlap_cfg_t c;
      ub_overlap_cfg_default(&c);
      c.method = static_cast<int32_t>(pick({0, 1, 2, 5}));
      c.num_splits = static_cast<int32_t>(pick({-1, 0, 1, 3, 8, 65, 1000}));
      c.num_max_streams = static_cast<int32_t>(pick({0, 1, 3, 9}));
      c.aggregate = static_cast<int32_t>(pick({0, 1}));
      c.atomic_gemm = static_cast<int32_t>(pick({0, 1}));
      c.rank = static_cast<int32_t>(pick({-1, 0, 1, 7, 64}));
      c.reduce_order = static_cast<int32_t>(pick({0, 1, 3}));
      c.fuse_reduce = static_cast<int32_t>(pick({0, 1, 2}));
      ub_plan_unit_t pu[8];
      int32_t n1 = 0, n2 = 0;
      const ub_status_t s3 = ub_get_plan(hh, &c, static_cast<ub_op_t>(pick({0, 1, 2})), pu, 8, &n1, &n2);
      CHECK(s3 >= UB_OK && s3 <= UB_ERR_HIP);
      const int64_t n = pick({-8, 0, 8, 260, 1024});
      const int64_t ld = pick({n, n + 8, n - 8, 3});
      const ub_status_t s4 = ub_gemm_ag_chunked(hh, rng() & 7 ? fake() : nullptr, n, ld, fake(), ld, &c, nullptr);
      const ub_status_t s5 = ub_gemm_rs_chunked(hh, fake(), pick({-16, 0, 16, 256, 4104}), pick({16, 256, 4104}),
                                                fake(), pick({H, H + 8, 0}), fake(), H, &c, nullptr);
      const ub_status_t s6 = ub_reduce_partials(hh, fake(), pick({H, 1}), static_cast<int32_t>(pick({0, 1, 2})), nullptr);
      const ub_status_t s7 = ub_copy_in(hh, fake(), pick({-1, 0, 8, 1 << 20}), pick({-1, 0, 8}), nullptr);
      for (ub_status_t s : {s4, s5, s6, s7}) CHECK(s >= UB_OK && s <= UB_ERR_HIP);
      calls += 6;
    }
    CHECK(ub_destroy(hh) == UB_OK);
  }
  std::printf("ok: %ld calls\n", calls);
  return 0;
}
