// FP8 (E4M3) GEMM on gfx950 matrix cores: C = bf16(scale * (A * B^T)), fp32 accumulation.
//
// The all-gather-side chunk GEMM over a quantized UserBuffer, and the reduce-scatter
// side's K-slice GEMMs on quantized operands (batch entries, bf16 partials).  "[Feature Request] Support
// dynamic token counts in TP communication/GEMM overlap" (Transformer Engine issue 3564),
// "Implementation approach in the prototype", names quantized (FP8) buffers and leaves
// them outside the prototype's first scope; this is that extension, with the plain
// reading: OCP E4M3 operands with one dequantization factor per tensor, the weight stored
// [N, K] (K contiguous) as FP8 GEMMs conventionally take it, bf16 output.
//
//   A [m, k] E4M3 codes, row stride lda bytes (the UserBuffer rows of a chunk);
//   B [n, k] E4M3 codes, row stride ldb bytes (weight row j = output column j);
//   C [m, n] bf16, row stride ldc elements;  C = bf16_rne(scale * sum_k A[t, k] B[j, k]).
//
// Design (CDNA4), the bf16 kernel's (gemm_bf16.hip) with both operands K-contiguous:
//  - v_mfma_scale_f32_32x32x64_f8f6f4 with E4M3 on both sides and unit block scales: a
//    32x32 block per instruction over 64 k.  A lane supplies 32 bytes of its row (A) or
//    of its column (B): lanes 0-31 k = 0..31, lanes 32-63 k = 32..63 of the step.  The
//    instruction sums over every (lane half, byte) pair, so any k order applied to both
//    operands alike gives the same sum; this one reads two 16-byte LDS chunks per lane.
//  - A step covers BK = 64 codes: a 64-byte row per operand row, the same byte geometry
//    as the bf16 kernel's A tile, so both operands use its direct-to-LDS loads and its
//    row swizzle (conflict-free reads: each 16-lane group reads one chunk column).
//  - 8 waves in the same ping-pong of memory and compute clusters; the per-tensor scale
//    is applied to the fp32 accumulators in the epilogue, before the one bf16 rounding.
//  - Every tile shape uses the same instruction and k order, so an output's bits depend
//    only on its A row and B row: chunking, offsets and tile choice never change a result.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <cstring>

#include "gemm_common.h"
#include "ub_internal.h"

namespace ubx {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

struct F8Params {
  const uint8_t* a;
  const uint8_t* b;
  uint16_t* c;
  int64_t lda, ldb, ldc;
  int64_t sa, sb, sc;                    // batch strides (bytes, bytes, elements)
  int32_t n, k;
  float scale;
  int32_t tiles_n;
  int32_t group;                         // row tiles per group (tile_of)
  int32_t tiles_total;                   // unit_tile0[n_units]: the launch's tiles
  int32_t n_units;
  int32_t unit_row0[kMaxGemmUnits];
  int32_t unit_rows[kMaxGemmUnits];
  int32_t unit_tile0[kMaxGemmUnits + 1];
};

// BNL: B rows in LDS.  A tile narrower than 256 columns keeps 256 B rows in its stage, so
// that its direct loads still split evenly over the waves; the loads of rows past BN fall
// outside B's resource (zeros in LDS, no memory access) and no fragment read uses them.
template <int BM_, int BN_, int S_, int WGM_, int WGN_, int BNL_ = BN_>
struct F8Cfg {
  static constexpr int BM = BM_, BN = BN_, BK = 64, S = S_, BNL = BNL_;
  static constexpr int WGM = WGM_, WGN = WGN_;
  static constexpr int NW = WGM * WGN;
  static constexpr int THREADS = 64 * NW;
  static constexpr int WM = BM / WGM, WN = BN / WGN;
  static constexpr int FM = WM / 32, FN = WN / 32;
  static constexpr int ROW = 64;            // bytes of one operand row in a stage
  static constexpr int CPR = 4;             // 16-byte chunks per row
  static constexpr int ROWS_PER_LOAD = 16;  // a 1 KiB direct load covers 16 rows
  static constexpr int A_BYTES = BM * ROW;
  static constexpr int B_BYTES = BNL * ROW;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int NA = A_BYTES / 1024 / NW;  // direct loads per wave per step
  static constexpr int NB = B_BYTES / 1024 / NW;
  static constexpr int L = NA + NB;
  static constexpr int LDC = BN + 8;
  static constexpr int EPI = BM * LDC * 2;
  static constexpr int LDS_BYTES = (S * STAGE > EPI) ? S * STAGE : EPI;
  static_assert(NW == 8, "ping-pong needs two waves per SIMD");
  static_assert(NA >= 1 && NB >= 1 && A_BYTES % (1024 * NW) == 0 && B_BYTES % (1024 * NW) == 0,
                "direct loads do not split over the waves");
  static_assert(WM % 32 == 0 && WN % 32 == 0 && FM >= 1 && FN >= 1, "32x32 blocks");
  static_assert(S * L <= 63, "vmcnt is a 6-bit count");
  static_assert(BN <= BNL, "the tile's B rows within the stage");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS is 160 KiB per CU");
};

template <class C>
struct F8Tile {
  int lane, wave, group, wm, wn, m0, m_end, n0;
  uint16_t* cg;
  i32x4 ra, rb;
  uint32_t a_off[C::NA], b_off[C::NB];
  uint32_t rd_a, rd_b;  // byte offset of this lane's first A / B fragment row in a stage
  int rd_c0, rd_c1;     // the two 16-byte chunk slots (swizzled) this lane reads

  // (a workgroup past the launch's last tile ends in tile_of_lanes, before any barrier)
  __device__ inline void init(const F8Params& p, int tid) {
    lane = tid & 63;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    group = wave >> 2;
    wm = wave / C::WGN;
    wn = wave % C::WGN;
    // every kernel argument the prologue needs, loaded before the first branch (args_here)
    const UnitLanes ul = unit_lanes(p);
    const auto pa = p.a;
    const auto pb = p.b;
    const auto pc = p.c;
    const int64_t lda = p.lda, sa = p.sa, ldb = p.ldb, sb = p.sb, sc = p.sc;
    const int nn = p.n;
    lanes_here(ul);
    const int nu = p.n_units, tc = p.tiles_n, tg = p.group, tt = p.tiles_total;
    args_here(pa, pb, pc, lda, sa, ldb, sb, sc, nn, nu, tc, tg, tt);
    int tn;
    tile_of_lanes(ul, nu, tc, tg, tt, (int)blockIdx.x, C::BM, m0, m_end, tn);
    n0 = tn * C::BN;
    const int rows_a = min(C::BM, m_end - m0);
    const int rows_b = min(C::BN, nn - n0);
    // batch entry blockIdx.z: A and B start sa / sb bytes further (a K slice), C sc elements
    ra = make_rsrc(pa + blockIdx.z * sa + (int64_t)m0 * lda, (uint32_t)(rows_a * lda));
    rb = make_rsrc(pb + blockIdx.z * sb + (int64_t)n0 * ldb, (uint32_t)(rows_b * ldb));
    cg = pc + blockIdx.z * sc;
    // Direct load t of this wave covers operand rows 16 (wave * N + t) + lane / 4; lane
    // slot lane % 4 holds k-chunk slot ^ a_swz(row).  Rows past the operand's valid rows
    // are beyond the resource's size and read as zeros.
#pragma unroll
    for (int t = 0; t < C::NA; ++t) {
      const int row = C::ROWS_PER_LOAD * (wave * C::NA + t) + lane / C::CPR;
      a_off[t] = (uint32_t)(row * lda + ((lane % C::CPR) ^ a_swz<C::CPR>(row)) * 16);
    }
#pragma unroll
    for (int t = 0; t < C::NB; ++t) {
      const int row = C::ROWS_PER_LOAD * (wave * C::NB + t) + lane / C::CPR;
      b_off[t] = (uint32_t)(row * ldb + ((lane % C::CPR) ^ a_swz<C::CPR>(row)) * 16);
    }
    // Fragments: A row wm*WM + i*32 + (lane&31), B row wn*WN + j*32 + (lane&31); the
    // swizzle of a row depends only on its low bits, i.e. on lane & 31.
    rd_a = (uint32_t)((wm * C::WM + (lane & 31)) * C::ROW);
    rd_b = (uint32_t)(C::A_BYTES + (wn * C::WN + (lane & 31)) * C::ROW);
    const int x = a_swz<C::CPR>(lane & 31);
    rd_c0 = ((2 * (lane >> 5)) ^ x) * 16;
    rd_c1 = ((2 * (lane >> 5) + 1) ^ x) * 16;
  }

  // Steps past the end are issued with out-of-range offsets (zeros, no memory touched) so
  // that every wait counts a fixed number of newer loads.
  __device__ inline void issue_loads(unsigned char* smem, int ks, int nk) const {
    unsigned char* st = smem + (ks % C::S) * C::STAGE;
    const bool live = ks < nk;
    const uint32_t kk = (uint32_t)ks * C::BK;
#pragma unroll
    for (int t = 0; t < C::NA; ++t)
      dma16(ra, lds_addr(st + (wave * C::NA + t) * 1024), live ? a_off[t] + kk : OOB);
#pragma unroll
    for (int t = 0; t < C::NB; ++t)
      dma16(rb, lds_addr(st + C::A_BYTES + (wave * C::NB + t) * 1024), live ? b_off[t] + kk : OOB);
  }

  // Load slot j alone (A's NA slots, then B's), the same load issue_loads makes for it.
  __device__ inline void issue_load_slot(unsigned char* smem, int ks, int nk, int j) const {
    unsigned char* st = smem + (ks % C::S) * C::STAGE;
    const bool live = ks < nk;
    const uint32_t kk = (uint32_t)ks * C::BK;
    if (j < C::NA)
      dma16(ra, lds_addr(st + (wave * C::NA + j) * 1024), live ? a_off[j] + kk : OOB);
    else
      dma16(rb, lds_addr(st + C::A_BYTES + (wave * C::NB + j - C::NA) * 1024),
            live ? b_off[j - C::NA] + kk : OOB);
  }

  __device__ inline i32x8 frag(const unsigned char* row) const {
    const u32x4 lo = *LDS_PTR(const u32x4, row + rd_c0);
    const u32x4 hi = *LDS_PTR(const u32x4, row + rd_c1);
    return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }

  __device__ inline void read_frags(const unsigned char* smem, int ks, i32x8* af, i32x8* bf) const {
    const unsigned char* st = smem + (ks % C::S) * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::FM; ++i) af[i] = frag(st + rd_a + i * 32 * C::ROW);
#pragma unroll
    for (int j = 0; j < C::FN; ++j) bf[j] = frag(st + rd_b + j * 32 * C::ROW);
  }

  // scale, round to bf16, stage the tile in LDS and write it with 16-byte stores (rows
  // >= m_end and columns >= n masked).  32x32 accumulator layout: lane holds column
  // (lane & 31); element e holds row 8*(e/4) + 4*(lane/32) + (e%4).
  __device__ inline void store(unsigned char* smem, const F8Params& p, int tid,
                               const f32x16 (&acc)[C::FM][C::FN]) const {
    uint16_t* ct = reinterpret_cast<uint16_t*>(smem);
    const float s = p.scale;
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        const int col = wn * C::WN + j * 32 + (lane & 31);
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
          const int row = wm * C::WM + i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
          const uint32_t v = pack_bf16x2(acc[i][j][e] * s, acc[i][j][e + 1] * s);
          *LDS_PTR(uint16_t, ct + row * C::LDC + col) = (uint16_t)(v & 0xFFFF);
          *LDS_PTR(uint16_t, ct + (row + 1) * C::LDC + col) = (uint16_t)(v >> 16);
        }
      }
    __syncthreads();
    constexpr int VPR = C::BN / 8;
#pragma unroll
    for (int i = 0; i < C::BM * VPR / C::THREADS; ++i) {
      const int v = tid + i * C::THREADS;
      const int r = v / VPR, cc = (v % VPR) * 8;
      const int gr = m0 + r, gc = n0 + cc;
      if (gr < m_end && gc < p.n)
        *GLOBAL_PTR(u32x4, cg + (int64_t)gr * p.ldc + gc) = *LDS_PTR(const u32x4, ct + r * C::LDC + cc);
    }
  }
};

// The ping-pong of gemm_bf16_pingpong (same barriers, same landing argument) with one
// 64-deep MFMA step per stage.
// LIC: the loads of step ks + D issue between the MFMAs of step ks instead of in the memory
// cluster (as in the bf16 ping-pong: group 1's wait at the end of its memory cluster then
// allows (D - 2) steps in flight).
template <class C, int D, bool LIC = false>
__global__ __launch_bounds__(C::THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_fp8_pingpong(F8Params p) {
  static_assert(D >= 2 && D <= C::S - 1, "load distance");
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const int tid = threadIdx.x;
  F8Tile<C> t;
  t.init(p, tid);
  const int group = t.group;

  f32x16 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  i32x8 af[C::FM], bf[C::FN];
  const int nk = p.k / C::BK;

#pragma unroll
  for (int s = 0; s < D; ++s) t.issue_loads(smem, s, nk);
  __builtin_amdgcn_sched_barrier(0);
  wait_vmcnt_and_barrier<(D - 1) * C::L>();  // b0: step 0 landed everywhere
  __builtin_amdgcn_sched_barrier(0);
  if (group == 1) __asm__ volatile("s_barrier" ::: "memory");  // b1 for group 1
  __builtin_amdgcn_sched_barrier(0);

  for (int ks = 0; ks < nk; ++ks) {
    t.read_frags(smem, ks, af, bf);  // memory cluster
    if constexpr (!LIC) t.issue_loads(smem, ks + D, nk);
    __builtin_amdgcn_sched_barrier(0);
    if (group == 1) {
      __asm__ volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"((LIC ? D - 2 : D - 1) * C::L) : "memory");
    } else {
      __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    __builtin_amdgcn_sched_barrier(0);
    {
      constexpr int NM = C::FM * C::FN;
      int m = 0, jl = 0;
#pragma unroll
      for (int i = 0; i < C::FM; ++i)  // compute cluster
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc[i][j],
                                                                      0, 0, 0, 127, 0, 127);
          ++m;
          if (LIC && jl < C::L && m == (jl + 1) * NM / (C::L + 1)) {
            __builtin_amdgcn_sched_barrier(0);
            t.issue_load_slot(smem, ks + D, nk, jl);
            __builtin_amdgcn_sched_barrier(0);
            ++jl;
          }
        }
      if constexpr (LIC) {  // slots the MFMA count left over (NM <= L)
#pragma unroll
        for (; jl < C::L; ++jl) t.issue_load_slot(smem, ks + D, nk, jl);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    // Both groups take the same wait and barrier here: group 1 has issued no loads since
    // its own wait at the end of its memory cluster, so the wait costs it nothing.  With
    // this one unconditional statement the MFMAs stay in front of the barrier: behind a
    // branch on the group, the compiler sank them past it, so that both groups computed
    // at the same time and the clusters no longer alternated.
    __asm__ volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"((D - 1) * C::L) : "memory");
    __builtin_amdgcn_sched_barrier(0);
  }
  if (group == 0) __asm__ volatile("s_barrier" ::: "memory");  // matches group 1's b1
  wait_vmcnt_and_barrier<0>();
  t.store(smem, p, tid, acc);
}

using F8_256x256 = F8Cfg<256, 256, 4, 2, 4>;  // 8 waves of 128x64
using F8_128x256 = F8Cfg<128, 256, 4, 2, 4>;  // 8 waves of 64x64
using F8_256x192 = F8Cfg<256, 192, 4, 4, 2, 256>;  // 8 waves of 64x96 (B rows 256 deep in LDS)
constexpr int F8_D = 3;
// The narrow tile and 128x256 issue their loads between the MFMAs (their memory cluster is
// the longer one): on the qkv shape, forced tiles, bit-identical, 256x192 ran 1.5-1.8 PFLOP/s
// at T = 5536 ... 8192 with it and 1.46-1.86 without (256x256: 1.44-1.91), 128x256 +1-4%.
template <class C> constexpr bool kF8LoadsInCompute = C::BN < 256 || C::BM < 256;

template <class C>
hipError_t launch(const GemmF8Args& g, const GemmUnits& units, hipStream_t stream) {
  const GemmUnits u = tile_aligned_units(units, C::BM);
  F8Params p{};
  p.a = g.a;
  p.b = g.b;
  p.c = g.c;
  p.lda = g.lda;
  p.ldb = g.ldb;
  p.ldc = g.ldc;
  p.sa = g.a_batch_stride;
  p.sb = g.b_batch_stride;
  p.sc = g.c_batch_stride;
  p.n = g.n;
  p.k = g.k;
  p.scale = g.scale;
  p.tiles_n = (g.n + C::BN - 1) / C::BN;
  p.n_units = u.n;
  int64_t tiles = 0;
  for (int i = 0; i < u.n; ++i) {
    p.unit_row0[i] = u.row0[i];
    p.unit_rows[i] = u.rows[i];
    p.unit_tile0[i] = (int32_t)tiles;
    tiles += (int64_t)((u.rows[i] + C::BM - 1) / C::BM) * p.tiles_n;
  }
  p.unit_tile0[u.n] = (int32_t)tiles;
  p.tiles_total = (int32_t)tiles;
  if (tiles == 0) return hipSuccess;
  p.group = tile_group(tiles, p.tiles_n, 1, g.dbg ? g.dbg->tile_group : 0);
  const int64_t grid = tiles;
  if (grid > 0x7FFFFFFF || g.batch < 1 || g.batch > 65535) return hipErrorInvalidValue;
  auto kernel = &gemm_fp8_pingpong<C, F8_D, kF8LoadsInCompute<C>>;
  hipError_t e = ensure_lds_attr(reinterpret_cast<const void*>(kernel), C::LDS_BYTES);
  if (e != hipSuccess) return e;
  return launch_k(kernel, dim3((unsigned)grid, 1, g.batch), dim3(C::THREADS), C::LDS_BYTES, stream, p);
}

// Tile choice as for bf16 (rounds of a launch x tile area / efficiency); a handle's debug
// setting can force one of the two shapes.
// 0: 256x256, 1: 128x256, 2: 256x192.  Efficiencies against 256x256: 128x256 0.62; 256x192
// 0.82, the ratio of forced one-round launches on the qkv shape (0.77 at T = 8192 ... 0.86 at
// 4096), which takes it at every qkv pack (5536 ... 8176 rows, 2-11% faster than 256x256
// there) and leaves 128x256 at T = 4096, where it measured fastest.
int f8_tile(const GemmF8Args& g, const GemmUnits& u) {
  if (g.dbg && g.dbg->tile_m > 0) return g.dbg->tile_m == 128 ? 1 : g.dbg->tile_n == 192 ? 2 : 0;
  const int share = 256 / (g.concurrency > 1 ? g.concurrency : 1);
  auto cost = [&](int bm, int bn, double eff) {
    const int64_t tiles = row_tiles(u, bm) * ((g.n + bn - 1) / bn) * g.batch;
    const int64_t slots = share > 0 ? share : 1;
    return (double)((tiles + slots - 1) / slots) * bm * bn / eff;
  };
  const double c0 = cost(256, 256, 1.0), c1 = cost(128, 256, 0.62), c2 = cost(256, 192, 0.82);
  return c1 < c0 && c1 < c2 ? 1 : c2 < c0 ? 2 : 0;
}

}  // namespace

bool gemm_fp8_shape_supported(const GemmF8Args& g) {
  // 32-bit byte offsets inside one tile's rows of A and B
  return (int64_t)256 * g.lda < (int64_t)OOB && (int64_t)256 * g.ldb < (int64_t)OOB;
}

hipError_t launch_gemm_fp8_units(const GemmF8Args& g, const GemmUnits& u, hipStream_t stream) {
  if (g.n <= 0 || u.n <= 0 || g.batch <= 0) return hipSuccess;
  if (u.n > kMaxGemmUnits || g.k <= 0 || g.k % kGemmF8KStep != 0 || g.n % 8 != 0 ||
      g.lda % 16 != 0 || g.ldb % 16 != 0 || g.ldc % 8 != 0 || !gemm_fp8_shape_supported(g))
    return hipErrorInvalidValue;
  for (int i = 0; i < u.n; ++i)
    if (u.rows[i] < 0 || u.row0[i] < 0) return hipErrorInvalidValue;
  const int kind = f8_tile(g, u);
  if (g.plan_out) {
    const int32_t d = g.plan_out->dispatches;
    *g.plan_out = TilePlanRecord{};
    g.plan_out->dispatches = d + 1;
    g.plan_out->tile_m = kind == 1 ? 128 : 256;
    g.plan_out->tile_n = kind == 2 ? 192 : 256;
  }
  return kind == 1 ? launch<F8_128x256>(g, u, stream)
                   : kind == 2 ? launch<F8_256x192>(g, u, stream) : launch<F8_256x256>(g, u, stream);
}

bool gemm_fp8_tile_supported(int tile_m, int tile_n) {
  return (tile_n == 256 && (tile_m == 128 || tile_m == 256)) || (tile_m == 256 && tile_n == 192);
}

}  // namespace ubx
