// Device helpers shared by the GEMM kernels (bf16 and fp8): buffer resources and
// direct-to-LDS loads, the A-side swizzle, waits, bf16 packing and the workgroup -> tile
// mapping of the device-side chunk loop.  See gemm_bf16.hip for the design.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <set>
#include <utility>

namespace ubx {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
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
// B: k-rows r and r + 8 (read by the two 16-lane halves of one 32-lane LDS cycle of the
// transposing reads) get column-chunk sets that differ by XOR 2, disjoint banks.
__device__ constexpr int b_swz(int r) { return ((2 * (r & 3)) ^ (4 * (r & 3))) ^ (((r >> 3) & 1) << 1); }

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

// Tile of workgroup `wg` of a batch entry.  The row tiles of all units, in processing order,
// form one list of R row tiles (unit u owns row tiles [unit_tile0[u] / C, unit_tile0[u+1] /
// C), C = tile columns); the tiles are listed in groups of p.group row tiles, each group
// column by column, so that neighbours share B columns.  The dispatcher deals workgroups
// round-robin over the 8 XCDs, each with its own L2: XCD x = wg % 8 takes a balanced
// contiguous block of that list (total / 8 tiles, the remainder spread over the first
// XCDs), so an XCD's tiles share A rows.  Returns the tile's first row and the end of its
// unit's rows; false for a workgroup past the last tile.
//
// Group size: a launch whose tiles all run at once (no more tiles than workgroup slots)
// gains nothing from column groups and lists its tiles row by row (group 1), which keeps
// each XCD's block on the fewest A rows; so does a launch with few tile columns (at most
// 8); other larger launches use groups of 4.  Measured on MI355X, interleaved per point:
// the GQA shape (5 tile columns) at T = 23376 ... 32520 runs 2-4% faster with 1 than with
// 4; qkv shapes ~1-2% faster with 1; fc2's batched slices (16 columns) 3-10% and 8192^3 and
// 16384 x 3584 x 4096 3-5% faster with 4.  forced > 0 (a handle's debug setting) overrides
// the choice.
inline int tile_group(int64_t tiles, int tiles_n, int per_cu, int forced) {
  if (forced >= 1) return forced;
  return tiles <= 256 * (int64_t)per_cu || tiles_n <= 8 ? 1 : 4;
}

// Sets a kernel's dynamic-LDS limit on the current device, once per (device, kernel):
// HIP keeps the attribute per device, and launches from several host threads may come
// first at the same time, hence the lock.
inline hipError_t ensure_lds_attr(const void* kernel, int bytes) {
  static std::mutex mu;
  static std::set<std::pair<int, const void*>> done;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  if (done.count({dev, kernel})) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.insert({dev, kernel});
  return e;
}

// Workgroup wg's place in that order: its row tile (in the list of all units' row tiles)
// and its tile column, for `total` tiles of C columns listed in groups of G row tiles.
__host__ __device__ __attribute__((always_inline)) inline void tile_position(int wg, int total, int C, int G, int& row_tile,
                                              int& tn) {
  const int R = total / C;
  const int q = total / NUM_XCD, rem = total % NUM_XCD;
  const int x = wg % NUM_XCD, k = wg / NUM_XCD;
  const int t = x * q + (x < rem ? x : rem) + k;  // XCD x holds [x q + min(x, rem), ...)
  const int group = t / (G * C);
  const int first = group * G;
  const int gm = G < R - first ? G : R - first;
  const int r = t - group * G * C;
  row_tile = first + r % gm;
  tn = r / gm;
}

template <class P>
__host__ __device__ __attribute__((always_inline)) inline bool tile_of(const P& p, int wg, int bm, int& m0, int& m_end, int& tn) {
  const int C = p.tiles_n;
  const int total = p.unit_tile0[p.n_units];
  if (wg >= total) return false;
  int row_tile;
  tile_position(wg, total, C, p.group, row_tile, tn);
  int u = 0;
  while (u + 1 < p.n_units && p.unit_tile0[u + 1] / C <= row_tile) ++u;
  m0 = p.unit_row0[u] + (row_tile - p.unit_tile0[u] / C) * bm;
  m_end = p.unit_row0[u] + p.unit_rows[u];
  return true;
}

// tile_of as a wave computes it in a kernel: the same tile, with the unit table read by one
// load per lane (lane j: unit j) and the unit found by a ballot, instead of a scan whose
// every step waits on a scalar load.  unit_tile0 is non-decreasing and a multiple of C, so
// the units that start at or before the row tile are a prefix of the lanes, and its length
// is the scan's answer.  At the start of a launch every workgroup reads the table at once;
// there the scan's chain of dependent loads took most of a ~6k-cycle prologue.
struct UnitLanes {
  int t0, t1, r0, nr;  // lane j: unit j's first tile, unit j + 1's, unit j's first row, rows
};

template <class P>
__device__ __attribute__((always_inline)) inline UnitLanes unit_lanes(const P& p) {
  static_assert(sizeof(p.unit_row0) == 64 * sizeof(p.unit_row0[0]), "one lane per unit");
  const int lane = __lane_id();
  return UnitLanes{p.unit_tile0[lane], p.unit_tile0[lane + 1], p.unit_row0[lane], p.unit_rows[lane]};
}

// nu units, C tile columns, G row tiles per group, total tiles: the launch's n_units,
// tiles_n, group and unit_tile0[n_units].  A workgroup past the last tile (none is launched)
// ends here; an early return instead, after the lanes' loads, makes the compiler treat the
// kernel's exit as divergent and keep the tile's addresses in VGPRs.
__device__ __attribute__((always_inline)) inline void tile_of_lanes(const UnitLanes& l, int nu,
                                                                     int C, int G, int total,
                                                                     int wg, int bm, int& m0,
                                                                     int& m_end, int& tn) {
  if (wg >= total) __builtin_amdgcn_endpgm();
  int row_tile;
  tile_position(wg, total, C, G, row_tile, tn);
  const int lane = __lane_id();
  const int u = __popcll(__ballot(lane + 1 < nu && l.t1 <= row_tile * C));
  const int r0 = __builtin_amdgcn_readlane(l.r0, u);
  m0 = r0 + (row_tile - __builtin_amdgcn_readlane(l.t0, u) / C) * bm;
  m_end = r0 + __builtin_amdgcn_readlane(l.nr, u);
}

template <class P>
__device__ __attribute__((always_inline)) inline void tile_of_wave(const P& p, int wg, int bm,
                                                                    int& m0, int& m_end, int& tn) {
  tile_of_lanes(unit_lanes(p), p.n_units, p.tiles_n, p.group, p.tiles_total, wg, bm, m0, m_end,
                tn);
}

// Marks values loaded from the kernel arguments as needed here: their loads issue before
// this point, together, and are waited for once (the compiler otherwise places each load
// at its first use, behind the branches before it, one round trip each).
template <class T>
__device__ inline void arg_here(const T& v) {
  __asm__ volatile("" ::"s"(v));
}
template <class... T>
__device__ inline void args_here(const T&... v) {
  (arg_here(v), ...);
}
__device__ inline void lanes_here(const UnitLanes& l) {
  __asm__ volatile("" ::"v"(l.t0), "v"(l.t1), "v"(l.r0), "v"(l.nr));
}

}  // namespace
}  // namespace ubx
