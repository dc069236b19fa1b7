// Device helpers shared by the GEMM kernels (bf16 and fp8): buffer resources and
// direct-to-LDS loads, the A-side swizzle, waits, bf16 packing and the workgroup -> tile
// mapping of the device-side chunk loop.  See gemm_bf16.hip for the design.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace ubx {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))
#define GLOBAL_PTR(T, p) ((__attribute__((address_space(1))) T*)(p))

constexpr int NUM_XCD = 8;
constexpr int RSRC_WORD3 = 0x00020000;   // gfx9-family raw buffer: 32-bit data format
constexpr uint32_t OOB = 0x80000000u;    // an offset beyond every resource size used here

// Swizzles (see the design notes at the top of gemm_bf16.hip).
template <int CPR>
__device__ constexpr int a_swz(int R) {
  return CPR == 8 ? ((R ^ (R >> 1)) & 7) : (((R >> 1) ^ (R >> 2)) & 3);
}
__device__ constexpr int b_swz(int r) { return (2 * (r & 3)) ^ (4 * (r & 3)); }

// Raw buffer resource (base, num_records bytes) in scalar registers.
__device__ inline i32x4 make_rsrc(const void* base, uint32_t num_records) {
  const uint64_t b = (uint64_t)base;
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  r[1] = __builtin_amdgcn_readfirstlane((int)((b >> 32) & 0xFFFF));
  r[2] = __builtin_amdgcn_readfirstlane((int)num_records);
  r[3] = RSRC_WORD3;
  return r;
}

// 16 bytes per lane from rsrc + voffset into LDS at lds_addr + 16 * lane (see gemm_bf16.hip
// comment for why this is inline asm).
__device__ inline void dma16(i32x4 rsrc, uint32_t lds_addr, uint32_t voffset) {
  __asm__ volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                   ::"s"(lds_addr), "v"(voffset), "s"(rsrc)
                   : "memory");
}

__device__ inline uint32_t lds_addr(const void* p) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(size_t)LDS_PTR(const void, p));
}

template <int N>
__device__ inline void wait_vmcnt_and_barrier() {
  // this wave's direct loads older than the newest N have landed and its LDS reads are
  // done; then the same for every wave of the workgroup
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __asm__ volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  // fptrunc to bfloat lowers to gfx950's v_cvt_pk_bf16_f32: round to nearest even.
  const uint32_t a = __builtin_bit_cast(uint16_t, static_cast<__bf16>(lo));
  const uint32_t b = __builtin_bit_cast(uint16_t, static_cast<__bf16>(hi));
  return a | (b << 16);
}

// Tile of workgroup `wg` of a batch entry.  The workgroup index is first remapped so that a
// contiguous block of tile indices lands on each XCD; the index then selects its row unit
// (units are laid out in processing order) and, inside the unit, tiles are walked in
// groups of G tile-rows so neighbours share B columns.  Returns the unit's row range.
template <class P>
__device__ inline void tile_of(const P& p, int wg, int bm, int& m0, int& m_end, int& tn) {
  const int total = p.unit_tile0[p.n_units];
  int t = wg;
  if (total >= NUM_XCD * 2) {
    const int per = total / NUM_XCD;   // full share of each XCD
    const int full = per * NUM_XCD;
    if (wg < full) t = (wg % NUM_XCD) * per + wg / NUM_XCD;
  }
  int u = 0;
  while (u + 1 < p.n_units && p.unit_tile0[u + 1] <= t) ++u;
  const int local = t - p.unit_tile0[u];
  const int tiles_m = (p.unit_rows[u] + bm - 1) / bm;
  constexpr int G = 4;
  const int group = local / (G * p.tiles_n);
  const int first_m = group * G;
  const int gm = min(G, tiles_m - first_m);
  const int r = local - group * G * p.tiles_n;
  m0 = p.unit_row0[u] + (first_m + r % gm) * bm;
  m_end = p.unit_row0[u] + p.unit_rows[u];
  tn = r / gm;
}

}  // namespace
}  // namespace ubx
