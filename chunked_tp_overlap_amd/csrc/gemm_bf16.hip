// bf16 GEMM on gfx950 matrix cores: C = bf16(A * B), fp32 accumulation.
//
// This is the per-chunk GEMM of the overlap schedule ("How to setup TP Overlap configs",
// Transformer Engine issue 1344, "num_splits": the GEMM is cut into chunks, each a GEMM of
// its own).  A chunk's A operand is read in place from the capacity-sized UserBuffer at
// the chunk's row offset ("[Feature Request] Support dynamic token counts in TP
// communication/GEMM overlap", Transformer Engine issue 3564, "Implementation approach in
// the prototype": offsets from the active first dimension).
//
// All operands row-major: A [m, k] (lda), B [k, n] (ldb), C [m, n] (ldc).  blockIdx.z
// selects a batch entry at the given element strides (the reduce-scatter side's K slices).
//
// Design (CDNA4):
//  - A workgroup computes a BM x BN tile of C with v_mfma_f32_16x16x32_bf16 (fp32
//    accumulators): one 32-deep instruction per 16x16 block of a wave's tile per step.
//    K advances BK = 32 per step through S stages in LDS.  The 16x16x32 form moves fewer
//    register bytes per flop than the 32x32x16 form, and under the part's power limit
//    it holds a higher clock: measured +1-2% on the qkv launches, +3-5% on longer
//    full-chip launches (fc1, the GQA sweep, 8192^3), same LDS traffic.
//  - A fragment (16 rows x 32 k): lane l holds row l % 16, k 8 (l / 16) .. + 7.  B
//    fragment (32 k x 16 columns): lane l holds column l % 16, the same k.  Accumulator:
//    lane l holds column l % 16 of rows 4 (l / 16) .. + 3.
//  - Global -> LDS moves use buffer_load_dwordx4 ... lds: 16 bytes per lane straight into
//    LDS, no staging registers.  The buffer range check returns zeros for rows past m and
//    for columns past n (those lanes get an offset beyond the resource's size), so ragged
//    edges need no branches; every byte of the offset is in the per-lane VGPR offset, so
//    the range check covers all of it.  The loads are issued from inline asm: the
//    compiler cannot tell which stage an LDS read touches and would otherwise wait for
//    every in-flight load before each read, which serialises loads and MFMAs.  Their
//    completion is tracked by explicit vmcnt waits before the barriers instead.
//  - A direct load writes 64 lanes x 16 bytes contiguously, so bank conflicts are avoided
//    by XOR swizzles instead of padding (conflict-free whether the LDS serves 128 or 256
//    bytes per clock): A row R keeps its 16-byte k-chunk c in slot c ^ a_swz(R); B k-row
//    r keeps its 16-byte column chunk q in slot q ^ b_swz(r).
//  - A operands: one ds_read_b128 per lane (8 consecutive k of one row).  B operands: two
//    ds_read_b64_tr_b16 per lane: a 16-lane group reads 4 k-rows x 16 columns (lane j at
//    k-row j/4, columns 4*(j%4)..+3) and lane i receives the 4 k values of column i, so the
//    n-contiguous B tile feeds the MFMA without a transpose pass.
//  - Large tiles use 8 waves in a ping-pong: two groups of four waves, one wave of each
//    per SIMD, alternate memory clusters (fragment reads + their share of the direct
//    loads) and compute clusters (MFMAs), one group a cluster behind the other, so every
//    SIMD has one wave issuing MFMAs while its sibling waits on memory.  Small tiles use 4
//    waves, two workgroups per CU.
//  - Epilogue: accumulators are rounded to bf16 (RNE), staged through LDS as a row-major
//    tile and written with 16-byte coalesced stores; rows >= m and columns >= n are masked.
//  - Every tile shape uses the same instruction and the same ascending-K order, so an
//    output element's bits depend only on its own A row and B column: chunking, row offset
//    and tile choice never change a result.
//  - In the device-side chunk loop the plan's units are re-cut at tile boundaries (each
//    tile goes to the unit holding its last row), so a chunk that is not a multiple of the
//    tile height does not leave a partly empty tile behind.
//  - Workgroups are numbered so that consecutive tiles of a launch land on the same XCD
//    (the dispatcher deals workgroups round-robin over the 8 XCDs, each with its own L2),
//    and within an XCD tiles are walked in groups of rows that share B columns.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <vector>

#include "gemm_common.h"
#include "ub_internal.h"

namespace ubx {
namespace {

struct Params {
  const uint16_t* a;
  const uint16_t* b;
  uint16_t* c;
  int64_t lda, sa, ldb, sb, ldc, sc;
  int32_t n, k;
  int32_t tiles_n;                       // tile columns
  int32_t group;                         // row tiles per group (tile_of)
  int32_t tiles_total;                   // unit_tile0[n_units]: the launch's tiles
  int32_t n_units;                       // row units, in processing order
  int32_t unit_row0[kMaxGemmUnits];
  int32_t unit_rows[kMaxGemmUnits];
  int32_t unit_tile0[kMaxGemmUnits + 1];  // first workgroup of each unit (prefix sums)
  // arrival gating (GemmArgs): nullptr ready = none
  const uint32_t* ready;
  uint32_t* timeouts;
  uint64_t wait_ticks;
  uint32_t epoch;
  int32_t n_chunks;
  int32_t chunk_row0[kMaxGemmUnits + 1];
  // K segmentation (seg kernel): nseg segments of the k-steps; split: one workgroup per
  // (tile, segment), fp32 partials and per-tile counters in scratch
  int32_t nseg;
  int32_t split;
  float* parts;
  uint32_t* seg_counters;
  // fused reduction (GemmArgs): nslots == 0 = none
  uint16_t* out;
  int64_t ldo;
  uint32_t* counters;
  int64_t row0, shard_rows;
  int32_t nslots;
  int32_t ring;
};

// Arrival flags (see ub_internal.h).  Host code takes the array's device address from
// hipGetSymbolAddress (ready_flags_base), never its name.
static __device__ __align__(256) uint32_t g_ready[kReadySlots * kReadyWords];

constexpr uint64_t kReadyTimeoutTicks = 50000000ull;  // 0.5 s of the 100 MHz s_memrealtime clock

// Arrival gating: wait until every chunk holding a row of [r0, r1) has been delivered
// (its flag equals the call's epoch; the copy stream writes it after the chunk's copy),
// then acquire at system scope so that the A loads see the delivered rows rather than
// lines cached before they arrived.  The wait is bounded in time, so every wave ends.
// Returns, to every wave of the workgroup alike, whether some wave ran past the bound; the
// workgroup then counts one timeout and stores NaN instead of computing its tile.
// The workgroup's OR of v, through the first words of the kernel's LDS (called before any
// load writes there; the kernels then need no LDS of their own, which leaves all 160 KiB to
// the stages).
__device__ inline int workgroup_or(unsigned char* smem, int v) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, waves = blockDim.x >> 6;
  const bool any = __ballot(v != 0) != 0;
  if (lane == 0) *LDS_PTR(uint32_t, smem + 4 * wave) = any ? 1u : 0u;
  __syncthreads();
  uint32_t r = 0;
  for (int i = 0; i < waves; ++i) r |= *LDS_PTR(const uint32_t, smem + 4 * i);
  __syncthreads();  // every wave has read the words before LDS is reused
  return (int)r;
}

__device__ inline bool wait_ready(const Params& p, unsigned char* smem, int r0, int r1,
                                  bool count = true) {
  int c = 0;
  while (c + 1 < p.n_chunks && p.chunk_row0[c + 1] <= r0) ++c;
  const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
  int late = 0;
  for (; !late && c < p.n_chunks && p.chunk_row0[c] < r1; ++c) {
    while (__hip_atomic_load(p.ready + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM) != p.epoch) {
      if (__builtin_amdgcn_s_memrealtime() - t0 > p.wait_ticks) {
        late = 1;
        break;
      }
      __builtin_amdgcn_s_sleep(8);
    }
  }
  late = workgroup_or(smem, late);
  if (late && count && threadIdx.x == 0)
    __hip_atomic_fetch_add(p.timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "");
  return late != 0;
}

// ---- fused reduction arithmetic (the same operations as the separate reduction kernel) --
__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ inline float round_to_bf16(float x) {  // RNE, as an fp32 value
  return __uint_as_float((uint32_t)__builtin_bit_cast(uint16_t, static_cast<__bf16>(x)) << 16);
}

// Hop h of the sum of 8 elements.  Ascending order: fp32 adds from a zero start, one
// rounding at the end.  Ring order: start from the first partial, round to bf16 after
// every later hop.
__device__ inline void add_hop(float (&acc)[8], u32x4 x, int h, bool ring) {
  const float v[8] = {bf16_lo(x[0]), bf16_hi(x[0]), bf16_lo(x[1]), bf16_hi(x[1]),
                      bf16_lo(x[2]), bf16_hi(x[2]), bf16_lo(x[3]), bf16_hi(x[3])};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (h == 0)
      acc[i] = ring ? v[i] : 0.0f + v[i];
    else
      acc[i] = ring ? round_to_bf16(acc[i] + v[i]) : acc[i] + v[i];
  }
}

template <int NL>
__device__ inline void sum_slots(float (&acc)[8], const u32x4 (&x)[NL], bool ring) {
#pragma unroll
  for (int h = 0; h < NL; ++h) add_hop(acc, x[h], h, ring);
}

__device__ inline u32x4 pack8(const float (&acc)[8]) {
  return u32x4{pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
               pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
}

// BNL: columns of a B k-row in LDS.  A tile narrower than 256 columns (BN 192 or 160) keeps
// the 256-column row, so that the direct loads still cover whole rows and the B swizzle
// stays a permutation of the row; its loads of chunks past BN are out of range (zeros in
// LDS, no memory access) and no read uses them.
template <int BM_, int BN_, int BK_, int S_, int WGM_, int WGN_, int BNL_ = BN_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, S = S_, BNL = BNL_;
  static constexpr int WGM = WGM_, WGN = WGN_;      // wave grid
  static constexpr int NW = WGM * WGN;              // waves per workgroup
  static constexpr int THREADS = 64 * NW;
  static constexpr int WM = BM / WGM;               // wave tile rows
  static constexpr int WN = BN / WGN;               // wave tile cols
  static constexpr int FM = WM / 16;                // 16x16 blocks per wave, along m
  static constexpr int FN = WN / 16;                // along n
  static constexpr int SUBS = BK / 32;              // 32-deep k sub-steps per step
  static constexpr int A_ROW = BK * 2;              // bytes per A row in a stage
  static constexpr int A_CPR = BK / 8;              // 16-byte chunks per A row
  static constexpr int A_BYTES = BM * A_ROW;
  static constexpr int B_ROW = BNL * 2;             // bytes per B k-row in LDS
  static constexpr int B_CPR = BNL / 8;
  static constexpr int B_BYTES = BK * B_ROW;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int NA_ALL = A_BYTES / 1024;     // 1 KB direct loads per step, A
  static constexpr int NB_ALL = B_BYTES / 1024;     // and B
  // The step's NL loads, B's first, are dealt round-robin over the waves: wave w issues
  // loads w, w + NW, w + 2 NW, ...  B's loads fill whole rounds of NW, so every wave's
  // load slot j is of the same operand.  The first NFULL waves issue LMAX loads per step,
  // the others LMAX - 1 (the last slot, an A load); each wave waits on its own count.
  static constexpr int NL = NA_ALL + NB_ALL;
  static constexpr int LMAX = (NL + NW - 1) / NW;
  static constexpr int NFULL = NL % NW == 0 ? NW : NL % NW;
  static constexpr int A_ROWS_PER_LOAD = 1024 / A_ROW;
  static constexpr int B_ROWS_PER_LOAD = 1024 / B_ROW;
  static constexpr int LDC = BN + 8;                // epilogue tile row (elements)
  // The epilogue stages the bf16 tile in LDS: in one pass, or, when the whole tile does not
  // fit in 160 KiB, one pass per wave row.
  static constexpr int EPI_PASSES = BM * LDC * 2 <= 160 * 1024 ? 1 : WGM;
  static constexpr int EPI = (BM / EPI_PASSES) * LDC * 2;
  static constexpr int LDS_BYTES = (S * STAGE > EPI) ? S * STAGE : EPI;
  static_assert(NW == 8 || NL % NW == 0, "four-wave tiles split the loads evenly");
  static_assert(NB_ALL % NW == 0, "B loads fill whole rounds of the waves");
  static_assert(FM >= 1 && FN >= 1 && SUBS >= 1, "wave tile below one 16x16 block");
  static_assert(WM % 16 == 0 && WN % 16 == 0 && BK % 32 == 0, "whole 16x16x32 blocks");
  static_assert(A_BYTES % 1024 == 0 && B_BYTES % 1024 == 0, "whole 1 KB loads");
  static_assert(1024 % A_ROW == 0 && 1024 % B_ROW == 0, "a load covers whole rows");
  static_assert(BN <= BNL && BN % 16 == 0, "the tile's columns within the LDS row");
  static_assert(S * LMAX <= 63, "vmcnt is a 6-bit count");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS is 160 KiB per CU");
};

// Per-workgroup state shared by both kernels: tile position, buffer resources, and the
// per-lane offsets of the direct loads and of the fragment reads.
template <class C>
struct Tile {
  int lane, wave, group, wm, wn, m0, m_end, n0;
  int tile, z;                           // tile of the launch and batch entry
  int nl;                                // direct loads this wave issues per step
  uint16_t* cg;
  i32x4 ra, rb;
  // Load slot j of this wave is load w + NW j of the step: B load w + NW j for the first
  // NB_ALL / NW slots, then A load w + NW j - NB_ALL (a compile-time kind per slot keeps
  // the issue code free of branches and selects).
  static constexpr bool slot_is_a(int j) { return j * C::NW >= C::NB_ALL; }
  uint32_t lds_off[C::LMAX];             // byte offset in a stage
  uint32_t off[C::LMAX];                 // per-lane byte offset of step 0 (OOB: none)
  uint32_t tail_mask[C::LMAX];           // OOB for A chunks past k in the last step, else 0
  uint32_t a_kstep, b_kstep;
  int k_tail_step;                       // the step whose A chunks past k are masked, or -1
  int a_rd_row, a_rd_c, a_rd_x, b_krow, b_col_chunk, b_x, b_in;
  const uint32_t* ready;                 // the launch's arrival flags (nullptr: none)
  int nslots;                            // fused reduction's slices (0: none)

  // (a workgroup past the launch's last tile ends in tile_of_lanes, before any barrier)
  __device__ inline void init(const Params& p, int tid, int tile_index = -1) {
    lane = tid & 63;
    wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    group = wave >> 2;
    wm = wave / C::WGN;
    wn = wave % C::WGN;
    z = blockIdx.z;
    tile = tile_index >= 0 ? tile_index : (int)blockIdx.x;
    // every kernel argument the prologue needs, loaded before the first branch (args_here)
    const UnitLanes ul = unit_lanes(p);
    const uint16_t* const pa = p.a;
    const uint16_t* const pb = p.b;
    uint16_t* const pc = p.c;
    const int64_t lda = p.lda, sa = p.sa, ldb = p.ldb, sb = p.sb, sc = p.sc;
    const int kk = p.k, nn = p.n;
    ready = p.ready;
    nslots = p.nslots;
    lanes_here(ul);
    const int nu = p.n_units, tc = p.tiles_n, tg = p.group, tt = p.tiles_total;
    args_here(pa, pb, pc, lda, sa, ldb, sb, sc, kk, nn, ready, nslots, nu, tc, tg, tt);
    int tn;
    tile_of_lanes(ul, nu, tc, tg, tt, tile, C::BM, m0, m_end, tn);
    n0 = tn * C::BN;
    const uint16_t* A = pa + z * sa + (int64_t)m0 * lda;
    const uint16_t* B = pb + z * sb + n0;
    cg = pc + z * sc;
    // A from this tile's first row, valid rows only; B from column n0 of the batch entry,
    // k rows only (rows past k read zeros)
    const int rows_valid = min(C::BM, m_end - m0);
    ra = make_rsrc(A, (uint32_t)(rows_valid * lda * 2));
    rb = make_rsrc(B, (uint32_t)(((int64_t)kk * ldb - n0) * 2));
    // Direct loads: A load i covers rows A_ROWS_PER_LOAD*i + lane/A_CPR, slot lane%A_CPR
    // holding k-chunk slot ^ a_swz(row); B load i covers k-rows B_ROWS_PER_LOAD*i +
    // lane/B_CPR, slot lane%B_CPR holding column chunk slot ^ b_swz(krow).  Load i of an
    // operand lands at byte 1024*i of that operand's part of the stage.
    nl = wave < C::NFULL ? C::LMAX : C::LMAX - 1;
    k_tail_step = kk % C::BK ? kk / C::BK : -1;
    const int k_tail = kk - (kk / C::BK) * C::BK;  // valid k of the last step (if partial)
#pragma unroll
    for (int j = 0; j < C::LMAX; ++j) {
      const int li = wave + C::NW * j;
      const int idx = slot_is_a(j) ? li - C::NB_ALL : li;
      tail_mask[j] = 0;
      if (slot_is_a(j)) {
        const int row = C::A_ROWS_PER_LOAD * idx + lane / C::A_CPR;
        const int chunk = (lane % C::A_CPR) ^ a_swz<C::A_CPR>(row);
        lds_off[j] = (uint32_t)idx * 1024;
        off[j] = (uint32_t)((row * lda + chunk * 8) * 2);
        if (k_tail_step >= 0 && chunk * 8 >= k_tail) tail_mask[j] = OOB;
      } else {
        const int krow = C::B_ROWS_PER_LOAD * idx + lane / C::B_CPR;
        const int chunk = (lane % C::B_CPR) ^ b_swz(krow);
        lds_off[j] = (uint32_t)(C::A_BYTES + idx * 1024);
        off[j] = chunk * 8 < C::BN && n0 + chunk * 8 < nn
                     ? (uint32_t)((krow * ldb + chunk * 8) * 2) : OOB;
      }
      if (j >= nl) off[j] = OOB;
    }
    a_kstep = C::BK * 2;
    b_kstep = (uint32_t)(C::BK * ldb * 2);
    // Fragment reads.  A: row R = wm*WM + i*16 + (lane&15), k-chunk (kk/8 + lane/16) in
    // slot ^ a_swz(R) (a function of lane&15 only).  B: k-row kk + (lane/16)*8 + (lane>>2)&3
    // (+4 for the second read), column wn*WN + j*16 + (lane&3)*4.
    a_rd_row = (wm * C::WM + (lane & 15)) * C::A_ROW;
    a_rd_c = lane >> 4;
    a_rd_x = a_swz<C::A_CPR>(lane & 15);
    b_krow = (lane >> 4) * 8 + ((lane >> 2) & 3);
    b_col_chunk = (wn * C::WN + (lane & 3) * 4) >> 3;
    b_x = b_swz(b_krow);  // bits 0, 1 and 3 of the k-row; the second read's +4 leaves them
    b_in = (lane & 1) * 8;
  }

  // This wave's direct loads of step ks into stage ks % S.  Steps past the end are issued
  // with out-of-range offsets (they write zeros and touch no memory) so that every wait
  // can count a fixed number of newer loads; so are B chunks past column n, and, in the
  // last step of a k that is not a multiple of BK, A chunks past k (B rows past k are past
  // the B resource).  An offset is made out of range by setting its top bit: every
  // in-range offset is below 2^31 - 64 (gemm_shape_supported), so the result stays out of
  // range without wrapping.  No branches and no selects on the wave: the memory cluster
  // is the kernel's critical path.
  __device__ inline void issue_loads(unsigned char* smem, int ks, int nk) const {
    const uint32_t st = lds_addr(smem) + (uint32_t)((ks % C::S) * C::STAGE);
    const uint32_t dead = ks < nk ? 0u : OOB;
    const uint32_t tail = ks == k_tail_step ? ~0u : 0u;
    const uint32_t ak = (uint32_t)ks * a_kstep, bk = (uint32_t)ks * b_kstep;
#pragma unroll
    for (int j = 0; j < C::LMAX; ++j) {
      if (j + 1 == C::LMAX && C::LMAX * C::NW != C::NL && j >= nl) break;
      if (slot_is_a(j))
        dma16(ra, st + lds_off[j], ((off[j] + ak) | dead) | (tail_mask[j] & tail));
      else
        dma16(rb, st + lds_off[j], (off[j] + bk) | dead);
    }
  }

  // Load slot j alone (the same load issue_loads makes for it).
  __device__ inline void issue_load_slot(unsigned char* smem, int ks, int nk, int j) const {
    if (j + 1 == C::LMAX && C::LMAX * C::NW != C::NL && j >= nl) return;
    const uint32_t st = lds_addr(smem) + (uint32_t)((ks % C::S) * C::STAGE);
    const uint32_t dead = ks < nk ? 0u : OOB;
    if (slot_is_a(j)) {
      const uint32_t tail = ks == k_tail_step ? ~0u : 0u;
      dma16(ra, st + lds_off[j], ((off[j] + (uint32_t)ks * a_kstep) | dead) | (tail_mask[j] & tail));
    } else {
      dma16(rb, st + lds_off[j], (off[j] + (uint32_t)ks * b_kstep) | dead);
    }
  }

  __device__ inline void read_frags(const unsigned char* smem, int ks, int kk, bf16x8* af,
                                    bf16x8* bf) const {
    const unsigned char* sa = smem + (ks % C::S) * C::STAGE;
    const unsigned char* sb = sa + C::A_BYTES;
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
      af[i] = *LDS_PTR(const bf16x8,
                       sa + a_rd_row + i * 16 * C::A_ROW + (((kk >> 3) + a_rd_c) ^ a_rd_x) * 16);
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      const unsigned char* q =
          sb + (kk + b_krow) * C::B_ROW + (((b_col_chunk + j * 2) ^ b_x) * 16) + b_in;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, q));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, q + 4 * C::B_ROW));
      bf[j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  }

  // bf16 tile in LDS (the caller guarantees no wave still reads or loads into LDS), then
  // 16-byte coalesced stores; in EPI_PASSES passes of BM / EPI_PASSES rows (one per wave
  // row when the whole tile does not fit in LDS).  16x16 accumulator layout: lane holds
  // column (lane & 15); element e holds row 4*(lane/16) + e.
  __device__ inline void store(unsigned char* smem, const Params& p, int tid,
                               const f32x4 (&acc)[C::FM][C::FN]) const {
    uint16_t* ct = reinterpret_cast<uint16_t*>(smem);
    constexpr int PR = C::BM / C::EPI_PASSES;  // rows per pass
#pragma unroll
    for (int pass = 0; pass < C::EPI_PASSES; ++pass) {
      if (pass > 0) __syncthreads();  // the previous pass's reads of the LDS tile are done
      if (C::EPI_PASSES == 1 || wm == pass) {
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
          for (int j = 0; j < C::FN; ++j) {
            const int col = wn * C::WN + j * 16 + (lane & 15);
            const int row = (C::EPI_PASSES == 1 ? wm * C::WM : 0) + i * 16 + (lane >> 4) * 4;
#pragma unroll
            for (int e = 0; e < 4; e += 2) {
              const uint32_t v = pack_bf16x2(acc[i][j][e], acc[i][j][e + 1]);
              *LDS_PTR(uint16_t, ct + (row + e) * C::LDC + col) = (uint16_t)(v & 0xFFFF);
              *LDS_PTR(uint16_t, ct + (row + e + 1) * C::LDC + col) = (uint16_t)(v >> 16);
            }
          }
      }
      __syncthreads();
      constexpr int VPR = C::BN / 8;  // 16-byte vectors per tile row
      static_assert(PR * VPR % C::THREADS == 0, "whole vectors per lane");
#pragma unroll
      for (int i = 0; i < PR * VPR / C::THREADS; ++i) {
        const int v = tid + i * C::THREADS;
        const int r = v / VPR, cc = (v % VPR) * 8;
        const int gr = m0 + pass * PR + r, gc = n0 + cc;
        if (gr < m_end && gc < p.n)
          *GLOBAL_PTR(u32x4, cg + (int64_t)gr * p.ldc + gc) =
              *LDS_PTR(const u32x4, ct + r * C::LDC + cc);
      }
    }
  }

  // The tile's output as bf16 quiet NaNs (0x7FC0): what a tile stores when its arrival wait
  // ran out, so that rows computed from data that may not have arrived cannot pass for
  // results.
  __device__ inline void store_nan(const Params& p, int tid) const {
    constexpr int VPR = C::BN / 8;
    const u32x4 nan4 = {0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u};
    for (int v = tid; v < C::BM * VPR; v += C::THREADS) {
      const int r = v / VPR, cc = (v % VPR) * 8;
      const int gr = m0 + r, gc = n0 + cc;
      if (gr < m_end && gc < p.n) *GLOBAL_PTR(u32x4, cg + (int64_t)gr * p.ldc + gc) = nan4;
    }
  }

  // Fused reduction, after store().  The batch entries' tiles of one output tile (the
  // slices) may run on different XCDs, each with its own L2: every wave makes its partial
  // stores visible at agent scope, then one lane counts the tile's arrival.  The slice
  // that arrives last resets the counter, acquires, and sums every slice's partial in the
  // order launch_reduce_partials uses, so the result is bit-identical to the separate
  // reduction.  The arrival count goes through row 0's padding of the LDS tile, which the
  // store loop never reads.
  __device__ inline void fused_reduce(unsigned char* smem, const Params& p, int tid) const {
    switch (p.nslots) {
      case 2: reduce_tile<2>(smem, p, tid); break;
      case 4: reduce_tile<4>(smem, p, tid); break;
      case 8: reduce_tile<8>(smem, p, tid); break;
      default: reduce_tile<0>(smem, p, tid); break;
    }
  }

  template <int NS>
  __device__ inline void reduce_tile(unsigned char* smem, const Params& p, int tid) const {
    uint32_t* arrived = reinterpret_cast<uint32_t*>(smem + C::BN * 2);
    const int ns = NS > 0 ? NS : p.nslots;
    uint32_t* counter = p.counters + tile;
    // Each wave's partial stores complete (reach the L2) before the barrier; after it one
    // release RMW (an L2 write-back, then the count) publishes the whole tile.
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) {
      const uint32_t before =
          __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      // the last slice acquires every other slice's release before anyone reads
      if (before == (uint32_t)(ns - 1)) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      *LDS_PTR(uint32_t, arrived) = before;
    }
    __syncthreads();
    if (*LDS_PTR(const uint32_t, arrived) != (uint32_t)(ns - 1)) return;
    if (tid == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    constexpr int VPR = C::BN / 8;
    constexpr int NV = C::BM * VPR / C::THREADS;  // 16-byte vectors per lane
    // G vectors per round with all their slices' loads in flight (16 loads per lane)
    constexpr int G0 = NS > 0 && NS <= 16 ? 16 / (NS > 0 ? NS : 1) : 1;
    constexpr int G = NV % G0 == 0 ? G0 : (NV % 4 == 0 ? 4 : (NV % 2 == 0 ? 2 : 1));
    static_assert(NV % G == 0, "vectors per lane split into rounds");
    constexpr int NL = NS > 0 ? NS : 1;
    for (int i0 = 0; i0 < NV; i0 += G) {
      int64_t off[G], oo[G];
      int first[G];
      bool ok[G];
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const int v = tid + (i0 + j) * C::THREADS;
        const int r = v / VPR, cc = (v % VPR) * 8;
        const int gr = m0 + r, gc = n0 + cc;
        ok[j] = gr < m_end && gc < p.n;
        off[j] = ok[j] ? (int64_t)gr * p.ldc + gc : 0;
        oo[j] = ok[j] ? (int64_t)gr * p.ldo + gc : 0;
        first[j] = p.ring ? (int)(((p.row0 + gr) / p.shard_rows + 1) % ns) : 0;
      }
      if constexpr (NS > 0) {
        // hop h of vector j reads slot (first + h) mod NS: every partial of the vector, in
        // the order it is summed
        u32x4 x[G][NL];
#pragma unroll
        for (int j = 0; j < G; ++j)
#pragma unroll
          for (int h = 0; h < NL; ++h) {
            int s = first[j] + h;
            if (s >= NL) s -= NL;
            x[j][h] = ok[j] ? __builtin_nontemporal_load(
                                  GLOBAL_PTR(const u32x4, p.c + s * p.sc + off[j]))
                            : u32x4{0, 0, 0, 0};
          }
#pragma unroll
        for (int j = 0; j < G; ++j) {
          float acc[8];
          sum_slots<NL>(acc, x[j], p.ring != 0);
          if (ok[j])
            __builtin_nontemporal_store(pack8(acc), GLOBAL_PTR(u32x4, p.out + oo[j]));
        }
      } else {
#pragma unroll
        for (int j = 0; j < G; ++j) {
          float acc[8];
          for (int h = 0; h < ns; ++h) {
            int s = first[j] + h;
            if (s >= ns) s -= ns;
            const u32x4 x = ok[j] ? __builtin_nontemporal_load(
                                        GLOBAL_PTR(const u32x4, p.c + s * p.sc + off[j]))
                                  : u32x4{0, 0, 0, 0};
            add_hop(acc, x, h, p.ring != 0);
          }
          if (ok[j])
            __builtin_nontemporal_store(pack8(acc), GLOBAL_PTR(u32x4, p.out + oo[j]));
        }
      }
    }
  }
};

template <class C>
__device__ inline void mfma_block(f32x4 (&acc)[C::FM][C::FN], const bf16x8* af, const bf16x8* bf) {
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
}

// The MFMAs of one step with this wave's direct loads of step ks_load dealt between them:
// load slot j after MFMA (j + 1) NM / (LMAX + 1) of the NM.  The loads' issue leaves the
// memory cluster, which is the longer of the two clusters on the tiles that use this.
template <class C>
__device__ inline void mfma_block_loads(f32x4 (&acc)[C::FM][C::FN],
                                        const bf16x8 (&af)[C::SUBS][C::FM],
                                        const bf16x8 (&bf)[C::SUBS][C::FN], const Tile<C>& t,
                                        unsigned char* smem, int ks_load, int k1) {
  constexpr int NM = C::SUBS * C::FM * C::FN;
  int m = 0, j = 0;
#pragma unroll
  for (int sub = 0; sub < C::SUBS; ++sub)
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int n = 0; n < C::FN; ++n) {
        acc[i][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[sub][i], bf[sub][n], acc[i][n], 0, 0, 0);
        ++m;
        if (j < C::LMAX && m == (j + 1) * NM / (C::LMAX + 1)) {
          __builtin_amdgcn_sched_barrier(0);
          t.issue_load_slot(smem, ks_load, k1, j);
          __builtin_amdgcn_sched_barrier(0);
          ++j;
        }
      }
}

// ---- 8-wave ping-pong ------------------------------------------------------------------
// Waves 0-3 (group 0) and 4-7 (group 1) hold one SIMD each.  Each wave alternates a memory
// cluster (all fragments of step ks from LDS; its share of the direct loads of step ks+D)
// and a compute cluster (the MFMAs of step ks), with a barrier after each.  Group 1 starts
// one barrier late, so the groups' clusters interleave.  With barriers b0, b1, ... group 0
// runs memory clusters between b(2ks) and b(2ks+1), group 1 between b(2ks+1) and b(2ks+2).
//  - stage reuse: step ks+D goes into the stage of step ks+D-S, whose last reader finished
//    before b(2(ks+D-S)+2) <= b(2ks) because D <= S-1;
//  - landing: before b(2ks+2) each wave waits for its own loads of step ks+1 (issued D-1
//    memory clusters earlier, so (D-1)*L newer loads may stay in flight, L = this wave's
//    loads per step): group 1 at the end of its memory cluster, group 0 at the end of its
//    compute cluster;
//  - every wave executes the same number of barriers (2*nk + 4).
// LIC (loads in the compute cluster): a wave issues its loads of step ks+D between the MFMAs
// of step ks instead of in its memory cluster.  Those loads come after b(2ks+1), later than
// the stage-reuse bound needs; group 1's wait at the end of its memory cluster of step ks
// then has only steps ks+2 ... ks+D-1 issued after ks+1, so (D-2)*L may stay in flight,
// while group 0's wait, after its compute cluster, is unchanged.  Where the memory cluster
// is the longer one (the narrow tiles and 128x256, whose waves hold 16-24 MFMAs per step)
// this measured 2-11% faster; where the MFMA cluster is (256x256, 320x256: 32 and 40),
// 3-7% slower, and 10% slower with all loads at the cluster's start.

// s_waitcnt for this wave's loads: at most (D-1) steps' worth (LMAX or LMAX-1 per step) in
// flight, optionally with the LDS reads drained, then the workgroup barrier.
template <class C, int D, bool LGKM>
__device__ inline void wait_loads_barrier(bool full) {
  if (full) {
    if (LGKM)
      __asm__ volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"((D - 1) * C::LMAX) : "memory");
    else
      __asm__ volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"((D - 1) * C::LMAX) : "memory");
  } else {
    constexpr int L = C::LMAX > 1 ? C::LMAX - 1 : 1;
    if (LGKM)
      __asm__ volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"((D - 1) * L) : "memory");
    else
      __asm__ volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"((D - 1) * L) : "memory");
  }
}

// ---- split-K meeting point ----------------------------------------------------------------
// K-segmented rows: the nk k-steps of a tile form nseg segments, segment s holding steps
// [s nk / nseg, (s+1) nk / nseg); each segment's products are accumulated from zero (MFMAs
// in ascending k, as in every kernel here) into P_s, and the tile's result is
//   C = bf16( ((P_0 + P_1) + P_2) + ... + P_{nseg-1} )   (fp32 adds, in that order).
// Split: workgroup w computes segment w % nseg of tile w / nseg.  Here each segment writes
// P_s (fp32, [i][j][thread] f32x4, coalesced) to its scratch slot, makes it visible at agent
// scope (the tile's segments may run on different XCDs, each with its own L2) and counts
// itself on the tile's counter (low 16 bits: segments arrived; a segment whose arrival wait
// ran out adds 1 << 16 and writes nothing).  The last to arrive resets the counter, acquires
// and returns true with the ordered sum in acc; if some segment ran late it counts one
// timeout and stores NaN instead.  Every other workgroup returns false.
template <class C>
__device__ inline bool split_meet(unsigned char* smem, const Params& p, const Tile<C>& t,
                                  int tid, int tile, int seg, int nseg, bool late,
                                  f32x4 (&acc)[C::FM][C::FN]) {
  constexpr int TILE = C::BM * C::BN;
  if (!late) {
    float* mine = p.parts + ((int64_t)tile * nseg + seg) * TILE;
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j)
        *GLOBAL_PTR(f32x4, mine + ((i * C::FN + j) * C::THREADS + tid) * 4) = acc[i][j];
  }
  uint32_t* arrived = reinterpret_cast<uint32_t*>(smem);
  uint32_t* counter = p.seg_counters + tile;
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) {
    const uint32_t add = late ? 0x10001u : 1u;
    const uint32_t now =
        __hip_atomic_fetch_add(counter, add, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT) + add;
    if ((now & 0xFFFFu) == (uint32_t)nseg) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    *LDS_PTR(uint32_t, arrived) = now;
  }
  __syncthreads();
  const uint32_t now = *LDS_PTR(const uint32_t, arrived);
  if ((now & 0xFFFFu) != (uint32_t)nseg) return false;
  __syncthreads();  // every wave has read `arrived` before the epilogue reuses LDS
  if (tid == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (now >> 16) {
    if (tid == 0) __hip_atomic_fetch_add(p.timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    t.store_nan(p, tid);
    return false;
  }
  const float* base = p.parts + (int64_t)tile * nseg * TILE;
  for (int sg = 0; sg < nseg; ++sg) {
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
      for (int j = 0; j < C::FN; ++j) {
        const f32x4 v = __builtin_nontemporal_load(
            GLOBAL_PTR(const f32x4, base + (int64_t)sg * TILE + ((i * C::FN + j) * C::THREADS + tid) * 4));
        acc[i][j] = sg == 0 ? v : acc[i][j] + v;
      }
  }
  return true;
}

// The other split mode: every segment only writes P_s to its slot (a segment whose arrival
// wait ran out writes quiet NaNs instead, which make the tile's sum NaN), and a separate
// launch, gemm_bf16_split_reduce, sums the tile's partials in order over the whole chip.
template <class C>
__device__ inline void split_write(const Params& p, int tid, int tile, int seg, int nseg,
                                   bool late, const f32x4 (&acc)[C::FM][C::FN]) {
  float* mine = p.parts + ((int64_t)tile * nseg + seg) * (C::BM * C::BN);
  const f32x4 nan4 = {__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
      *GLOBAL_PTR(f32x4, mine + ((i * C::FN + j) * C::THREADS + tid) * 4) = late ? nan4 : acc[i][j];
}

// Sum of the split partials of tiles of C, in segment order, rounded to bf16 and stored:
// thread q of a tile's 256-thread group reads slot q (one f32x4: rows 4 (lane / 16) + e,
// e < 4, of column lane % 16 of a 16 x 16 block of the producing wave) of every partial.
template <class C>
__global__ __launch_bounds__(256) void gemm_bf16_split_reduce(Params p) {
  constexpr int TILE = C::BM * C::BN;
  constexpr int GROUPS = TILE / 4 / 256;  // 256-slot groups per tile
  const int tile = (int)blockIdx.x / GROUPS;
  const int q = ((int)blockIdx.x % GROUPS) * 256 + (int)threadIdx.x;
  int m0, m_end, tn;
  tile_of_wave(p, tile, C::BM, m0, m_end, tn);
  const float* src = p.parts + (int64_t)tile * p.nseg * TILE + q * 4;
  // four partials' loads in flight (past the last segment the last is read again, an L2
  // hit that no add uses), then their adds in segment order
  const int ns = p.nseg;
  f32x4 sum = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int s0 = 0; s0 < ns; s0 += 4) {
    f32x4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      v[i] = __builtin_nontemporal_load(
          GLOBAL_PTR(const f32x4, src + (int64_t)min(s0 + i, ns - 1) * TILE));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 t = s0 + i == 0 ? v[i] : sum + v[i];
      if (s0 + i < ns) sum = t;
    }
  }
  const int t = q % C::THREADS, ij = q / C::THREADS;
  const int i = ij / C::FN, j = ij % C::FN;
  const int wave = t >> 6, lane = t & 63;
  const int row = m0 + (wave / C::WGN) * C::WM + i * 16 + (lane >> 4) * 4;
  const int col = tn * C::BN + (wave % C::WGN) * C::WN + j * 16 + (lane & 15);
  if (col >= p.n) return;
  uint16_t* c = p.c + (int64_t)row * p.ldc + col;
#pragma unroll
  for (int e = 0; e < 4; e += 2) {
    const uint32_t v = pack_bf16x2(sum[e], sum[e + 1]);
    if (row + e < m_end) c[(int64_t)e * p.ldc] = (uint16_t)(v & 0xFFFF);
    if (row + e + 1 < m_end) c[(int64_t)(e + 1) * p.ldc] = (uint16_t)(v >> 16);
  }
}

// SPLIT 1 or 2: workgroup w runs segment w % nseg of tile w / nseg; 1 meets the tile's
// other segments in split_meet, 2 only writes its partial (split_write).
template <class C, int D, int SPLIT = 0, bool LIC = false>
__global__ __launch_bounds__(C::THREADS) __attribute__((amdgpu_waves_per_eu(2, 2)))
void gemm_bf16_pingpong(Params p) {
  static_assert(C::NW == 8, "ping-pong needs two waves per SIMD");
  static_assert(D >= 2 && D <= C::S - 1, "load distance");
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const int tid = threadIdx.x;
  const int nseg = SPLIT ? p.nseg : 1;
  const int tile = SPLIT ? (int)blockIdx.x / nseg : (int)blockIdx.x;
  const int seg = SPLIT ? (int)blockIdx.x % nseg : 0;
  Tile<C> t;
  t.init(p, tid, tile);
  bool late = false;
  if (t.ready) {
    late = wait_ready(p, smem, t.m0, min(t.m0 + C::BM, t.m_end), SPLIT != 1);
    if (!SPLIT && late) {
      t.store_nan(p, tid);
      return;
    }
  }
  const int group = t.group;
  const bool full = C::NFULL == C::NW || t.nl == C::LMAX;

  f32x4 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  bf16x8 af[C::SUBS][C::FM], bf[C::SUBS][C::FN];
  const int nk = (p.k + C::BK - 1) / C::BK;
  // steps [k0, k1) of this workgroup (all of them unless split; none for a late segment)
  const int k0 = SPLIT ? (int)((int64_t)seg * nk / nseg) : 0;
  const int k1 = !SPLIT ? nk : late ? k0 : (int)((int64_t)(seg + 1) * nk / nseg);

#pragma unroll
  for (int s = 0; s < D; ++s) t.issue_loads(smem, k0 + s, k1);
  __builtin_amdgcn_sched_barrier(0);
  wait_loads_barrier<C, D, true>(full);  // b0: step k0 landed everywhere
  __builtin_amdgcn_sched_barrier(0);
  if (group == 1) __asm__ volatile("s_barrier" ::: "memory");  // b1 for group 1
  __builtin_amdgcn_sched_barrier(0);

  for (int ks = k0; ks < k1; ++ks) {
    // memory cluster
#pragma unroll
    for (int sub = 0; sub < C::SUBS; ++sub) t.read_frags(smem, ks, sub * 32, af[sub], bf[sub]);
    if constexpr (!LIC) t.issue_loads(smem, ks + D, k1);
    __builtin_amdgcn_sched_barrier(0);
    if (group == 1) {
      wait_loads_barrier<C, LIC ? D - 1 : D, true>(full);
    } else {
      __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    __builtin_amdgcn_sched_barrier(0);
    // compute cluster
    if constexpr (LIC) {
      mfma_block_loads<C>(acc, af, bf, t, smem, ks + D, k1);
    } else {
#pragma unroll
      for (int sub = 0; sub < C::SUBS; ++sub) mfma_block<C>(acc, af[sub], bf[sub]);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (group == 0) {
      wait_loads_barrier<C, D, false>(full);
    } else {
      __asm__ volatile("s_barrier" ::: "memory");
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if (group == 0) __asm__ volatile("s_barrier" ::: "memory");  // matches group 1's b1
  wait_vmcnt_and_barrier<0>();  // trailing out-of-range loads landed before LDS is reused
  if constexpr (SPLIT == 2) {
    split_write<C>(p, tid, tile, seg, nseg, late, acc);
    return;
  }
  if constexpr (SPLIT == 1) {
    if (!split_meet(smem, p, t, tid, tile, seg, nseg, late, acc)) return;
  }
  t.store(smem, p, tid, acc);
  if (!SPLIT && t.nslots) t.fused_reduce(smem, p, tid);
}

// ---- 4-wave, S-stage pipeline -----------------------------------------------------------
// One barrier per step, before its last 32-deep sub-step: step ks+1 has landed (the S-2 newer
// steps may still be in flight), every wave is done reading stage ks % S, which then takes
// step ks + S; the first fragments of step ks+1 load while the last MFMAs of step ks run.
template <class C>
__global__ __launch_bounds__(C::THREADS) __attribute__((amdgpu_waves_per_eu(1, 2)))
void gemm_bf16_pipelined(Params p) {
  static_assert(C::S >= 2, "at least two stages");
  static_assert(C::NW == 4 && C::NL % C::NW == 0, "one group of four waves, even load split");
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const int tid = threadIdx.x;
  Tile<C> t;
  t.init(p, tid);
  if (t.ready && wait_ready(p, smem, t.m0, min(t.m0 + C::BM, t.m_end))) {
    t.store_nan(p, tid);
    return;
  }

  f32x4 acc[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  bf16x8 af[2][C::FM], bf[2][C::FN];
  const int nk = (p.k + C::BK - 1) / C::BK;

#pragma unroll
  for (int s = 0; s < C::S; ++s) t.issue_loads(smem, s, nk);
  wait_vmcnt_and_barrier<(C::S - 1) * C::LMAX>();
  t.read_frags(smem, 0, 0, af[0], bf[0]);

  // The two fragment buffers alternate per sub-step; with one sub-step per k-step an
  // iteration takes two k-steps, so that each iteration starts on buffer 0.  With an odd
  // step count the last iteration's second step is past the end: its loads were issued out
  // of range, and its MFMAs are skipped, so every tile shape runs exactly nk steps.
  constexpr int PAIR = C::SUBS == 1 ? 2 : 1;
  static_assert((PAIR * C::SUBS) % 2 == 0, "an even number of sub-steps per iteration");
  for (int ks0 = 0; ks0 < nk; ks0 += PAIR) {
#pragma unroll
    for (int u = 0; u < PAIR * C::SUBS; ++u) {
      const int ks = ks0 + u / C::SUBS, sub = u % C::SUBS, b = u & 1;
      if (sub + 1 < C::SUBS) {
        t.read_frags(smem, ks, (sub + 1) * 32, af[b ^ 1], bf[b ^ 1]);
      } else {
        wait_vmcnt_and_barrier<(C::S - 2) * C::LMAX>();
        t.issue_loads(smem, ks + C::S, nk);
        // at the last step this reads a stage of zeros that is never used
        t.read_frags(smem, ks + 1, 0, af[b ^ 1], bf[b ^ 1]);
      }
      if (PAIR == 1 || ks < nk) mfma_block<C>(acc, af[b], bf[b]);
    }
  }
  wait_vmcnt_and_barrier<0>();  // trailing out-of-range loads landed before LDS is reused
  t.store(smem, p, tid, acc);
  if (t.nslots) t.fused_reduce(smem, p, tid);
}

// ---- K-segmented 4-wave kernel -----------------------------------------------------------
// The segments of split_meet on 128 x 128 tiles.  SPLIT 1 or 2: one segment per workgroup,
// as in the ping-pong kernel.  SPLIT 0: one workgroup per tile runs all steps and folds each
// finished segment into the sum at the segment boundary, which gives the same bits without
// scratch (the fallback when none is registered or it is too small).
template <class C, int SPLIT>
__global__ __launch_bounds__(C::THREADS) __attribute__((amdgpu_waves_per_eu(1, 2)))
void gemm_bf16_seg(Params p) {
  static_assert(C::S >= 2, "at least two stages");
  static_assert(C::NW == 4 && C::NL % C::NW == 0, "one group of four waves, even load split");
  extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
  const int tid = threadIdx.x;
  const int nseg = p.nseg;
  const int tile = SPLIT ? (int)blockIdx.x / nseg : (int)blockIdx.x;
  const int seg = SPLIT ? (int)blockIdx.x % nseg : 0;
  Tile<C> t;
  t.init(p, tid, tile);
  bool late = false;
  if (t.ready) {
    late = wait_ready(p, smem, t.m0, min(t.m0 + C::BM, t.m_end), SPLIT != 1);
    if (!SPLIT && late) {
      t.store_nan(p, tid);
      return;
    }
  }

  f32x4 acc[C::FM][C::FN], sum[C::FM][C::FN];
#pragma unroll
  for (int i = 0; i < C::FM; ++i)
#pragma unroll
    for (int j = 0; j < C::FN; ++j) {
      acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      sum[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  bf16x8 af[2][C::FM], bf[2][C::FN];
  const int nk = (p.k + C::BK - 1) / C::BK;
  const int k0 = SPLIT ? (int)((int64_t)seg * nk / nseg) : 0;
  const int k1 = !SPLIT ? nk : late ? k0 : (int)((int64_t)(seg + 1) * nk / nseg);
  int done = 0;                                  // segments folded into sum
  int boundary = (int)((int64_t)1 * nk / nseg);  // end of the current segment

#pragma unroll
  for (int s = 0; s < C::S; ++s) t.issue_loads(smem, k0 + s, k1);
  wait_vmcnt_and_barrier<(C::S - 1) * C::LMAX>();
  t.read_frags(smem, k0, 0, af[0], bf[0]);

  for (int ks0 = k0; ks0 < k1; ks0 += 2) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int ks = ks0 + u, b = u;
      wait_vmcnt_and_barrier<(C::S - 2) * C::LMAX>();
      t.issue_loads(smem, ks + C::S, k1);
      t.read_frags(smem, ks + 1, 0, af[b ^ 1], bf[b ^ 1]);
      if (ks < k1) {
        mfma_block<C>(acc, af[b], bf[b]);
        if (!SPLIT && ks + 1 == boundary) {  // a segment ends: fold it into the sum
#pragma unroll
          for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j) {
              sum[i][j] = done == 0 ? acc[i][j] : sum[i][j] + acc[i][j];
              acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            }
          ++done;
          boundary = (int)((int64_t)(done + 1) * nk / nseg);
        }
      }
    }
  }
  wait_vmcnt_and_barrier<0>();  // trailing out-of-range loads landed before LDS is reused
  if constexpr (SPLIT == 2) {
    split_write<C>(p, tid, tile, seg, nseg, late, acc);
  } else if constexpr (SPLIT == 1) {
    if (!split_meet(smem, p, t, tid, tile, seg, nseg, late, acc)) return;
    t.store(smem, p, tid, acc);
  } else {
    t.store(smem, p, tid, sum);
  }
}

// seg_mode: 0 plain; 1 K-segmented in one workgroup per tile; 2 split, met in the kernel;
// 3 split, summed by a gemm_bf16_split_reduce launch after it.
template <class C, class K>
hipError_t launch(K kernel, const GemmArgs& g, const GemmUnits& units, hipStream_t stream,
                  int seg_mode = 0, int nseg = 1) {
  const GemmUnits u = tile_aligned_units(units, C::BM);
  Params p{};
  p.a = g.a;
  p.b = g.b;
  p.c = g.c;
  p.lda = g.lda;
  p.sa = g.a_batch_stride;
  p.ldb = g.ldb;
  p.sb = g.b_batch_stride;
  p.ldc = g.ldc;
  p.sc = g.c_batch_stride;
  p.n = g.n;
  p.k = g.k;
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
  p.group = tile_group(tiles, p.tiles_n, C::NW == 8 ? 1 : 2, g.dbg ? g.dbg->tile_group : 0);
  p.ready = g.ready;
  p.timeouts = g.timeouts;
  p.wait_ticks = g.wait_ticks ? g.wait_ticks : kReadyTimeoutTicks;
  p.epoch = g.epoch;
  p.n_chunks = g.ready ? g.n_chunks : 0;
  for (int c = 0; c <= p.n_chunks && c <= kMaxGemmUnits; ++c) p.chunk_row0[c] = g.chunk_row0[c];
  p.nslots = g.fuse_nslots;
  if (p.nslots > 0) {
    if (tiles > g.counters_n) return hipErrorInvalidValue;
    p.out = g.fuse_out;
    p.ldo = g.fuse_ldo;
    p.counters = g.counters;
    p.ring = g.fuse_ring;
    p.row0 = g.fuse_row0;
    p.shard_rows = g.fuse_shard_rows;
  }
  int64_t grid = tiles;
  if (seg_mode != 0) {  // K-segmented launch (batch 1, no fused sum)
    if (g.batch != 1 || p.nslots) return hipErrorInvalidValue;
    p.nseg = nseg;
    p.split = seg_mode >= 2;
    if (p.split) {
      if ((seg_mode == 2 && tiles > g.split_counters_n) ||
          tiles * nseg * C::BM * C::BN > g.split_parts_n)
        return hipErrorInvalidValue;
      p.parts = g.split_parts;
      p.seg_counters = g.split_counters;
      grid = tiles * nseg;
    }
  }
  if (grid > 0x7FFFFFFF || g.batch > 65535) return hipErrorInvalidValue;
  hipError_t e = ensure_lds_attr(reinterpret_cast<const void*>(kernel), C::LDS_BYTES);
  if (e != hipSuccess) return e;
  e = launch_k(kernel, dim3((unsigned)grid, 1, g.batch), dim3(C::THREADS), C::LDS_BYTES, stream, p);
  if (e != hipSuccess || seg_mode != 3) return e;
  constexpr int GROUPS = C::BM * C::BN / 4 / 256;
  if (tiles * GROUPS > 0x7FFFFFFF) return hipErrorInvalidValue;
  return launch_k(&gemm_bf16_split_reduce<C>, dim3((unsigned)(tiles * GROUPS)), dim3(256), 0, stream, p);
}

using PP320x256 = Cfg<320, 256, 32, 4, 2, 4>;   // 8 waves of 160x64
using PP256x256 = Cfg<256, 256, 32, 4, 2, 4>;   // 8 waves of 128x64
using PP128x256 = Cfg<128, 256, 32, 4, 2, 4>;   // 8 waves of 64x64
using PP256x192 = Cfg<256, 192, 32, 4, 4, 2, 256>;  // 8 waves of 64x96 (B rows 256 wide in LDS)
using PP256x160 = Cfg<256, 160, 32, 4, 4, 2, 256>;  // 8 waves of 64x80
using PL128x128 = Cfg<128, 128, 32, 4, 2, 2>;   // 4 waves of 64x64, 2 workgroups per CU
constexpr int PP_D = 3;
// load distance of a ping-pong tile: one step less than its stages
template <class C> constexpr int kDist = C::S - 1;
// Tiles whose direct loads issue between the MFMAs (see the ping-pong kernel): the narrow
// tiles and 128x256.  At load distance 3 they measured 2-11% faster than with the loads in
// the memory cluster at distance 2 (the narrow tiles' best before) on the GQA, qkv and fc1
// points where the plans take them; at distance 2 the gain was a third of that.
template <class C> constexpr bool kLoadsInCompute = C::BN < 256 || C::BM < 256;

// Tile choice by a cost model fitted to measurements.  A launch of `tiles` workgroups on
// the CUs left to it (share = 256 / concurrency; the 128 x 128 kernel holds two workgroups
// per CU) runs in rounds; a round's time is one tile's work over the tile's speed and the
// clock that the round's busy CUs allow:
//   time(round) = BM * BN * K / (speed(tile) * boost(busy CUs)),
//   boost(b) = min(1.476, (256 / b)^0.2245)
// (the part runs into its power limit under MFMA load, so a launch that leaves CUs idle
// runs the busy ones faster: counters of the GEMM show 2.25 GHz with ~145 busy CUs and 2.0
// with ~217).  Tile speeds, relative to the 256x256 ping-pong at full occupancy: 320x256
// 1.03, 128x256 0.75, 128x128 0.49 alone on a CU and 0.37 when two share one.  The five
// constants are a least-squares fit of log time ratios to a forced-tile sweep on MI355X
// over the workloads' own shapes (GQA 1280 x 8192 at 33 T, qkv 1536 x 4096, fc1 3584 x
// 4096, fc2 4096 x 1792 in 8 slices; device-side loop and host loop; 78 points, including
// forced cuts): the model's plan is within 2% of the best measured plan at 67 of them, at
// 0.989 of the best on average.  The narrow tiles 256x192 and 256x160 (eight and ten
// column tiles on N = 1536, eight on N = 1280) fill one round where 256x256 leaves a third
// of the CUs idle; their speeds, 0.883 and 0.835 (with their loads between the MFMAs), are
// the same ratio fitted to forced one-round launches of the three shapes at 19 and 15 T
// against 256x256 (within 10% at each; the fit overrates them a little next to full
// occupancy, where the clock falls faster than the boost curve has it).  With these the
// plans moved to 256x192 at GQA T = 9152, qkv 6656 ... 8192 and fc1 3072 and measured
// 2-10% faster there (in-process A/B against 0.80 and 0.76); raising 128x256 to the
// 0.78 its one-round points give as well lost 6-10% at GQA T = 2040 and qkv T = 2048,
// where it displaces split-K plans, so 128x256 keeps the joint fit's 0.749.
// A one-round launch's time barely follows the tile's area (a 128x256 or 256x160 tile
// takes 0.72 or 0.81 of a 256x256 tile's time): the narrow tiles pay only where they fill
// CUs that a wider tile leaves idle.
//
// Besides one tile shape for the whole launch, the model prices cuts: a launch that has the
// chip to itself runs the leading row bands that fill whole rounds of a large tile, then
// the remaining rows as a second launch on the same stream with the tile that finishes them
// soonest.  Rows are cut at a band boundary, so every row is still computed once, by one
// instruction sequence: the results do not change.  With several streams (the host loop)
// the other streams' launches fill the idle CUs, and no cut is taken.
struct TileOpt { int kind, bm, bn, per_cu; double speed, speed_alone; };
enum TileKind { kTile128x128 = 0, kTile128x256 = 1, kTile256x256 = 2, kTile320x256 = 3,
                kTile256x192 = 4, kTile256x160 = 5 };
const TileOpt kTileOpts[] = {{kTile320x256, 320, 256, 1, 1.030, 1.030},
                             {kTile256x256, 256, 256, 1, 1.000, 1.000},
                             {kTile128x256, 128, 256, 1, 0.749, 0.749},
                             {kTile128x128, 128, 128, 2, 0.373, 0.493},
                             {kTile256x192, 256, 192, 1, 0.883, 0.883},
                             {kTile256x160, 256, 160, 1, 0.835, 0.835}};
constexpr double kBoostMax = 1.476, kBoostExp = 0.2245;

const TileOpt* find_tile(int bm, int bn) {
  for (const TileOpt& o : kTileOpts)
    if (o.bm == bm && o.bn == bn) return &o;
  return nullptr;
}

struct TilePlan {
  int kind;           // tile of the (first) launch
  int64_t cut = -1;   // >= 0: rows from `cut` on go to a second launch
  int tail_kind = 0;  // tile of the second launch
};

// Rows [lo, hi) of the units, in the same order (empty pieces dropped).
GemmUnits clip_units(const GemmUnits& u, int64_t lo, int64_t hi) {
  GemmUnits out;
  out.n = 0;
  for (int i = 0; i < u.n; ++i) {
    const int64_t r0 = std::max<int64_t>(u.row0[i], lo);
    const int64_t r1 = std::min<int64_t>((int64_t)u.row0[i] + u.rows[i], hi);
    if (r1 <= r0) continue;
    out.row0[out.n] = (int32_t)r0;
    out.rows[out.n] = (int32_t)(r1 - r0);
    ++out.n;
  }
  return out;
}

// At short K the 320x256 tile gains on the others: its launch has a fifth fewer tiles, and
// each tile's fixed part (the loads before the first MFMA, the epilogue) weighs more.  Forced
// launches of the fc2 slices (K = 1792) give it 1.10 against 256x256 (the right choice at
// all six T from 2048 to 16384); K >= 4096 keeps the fitted 1.03.  Linear in between.
double short_k_gain(const TileOpt& o, int64_t k) {
  if (o.kind != kTile320x256 || k >= 4096) return 1.0;
  const double f = k <= 1792 ? 1.0 : (4096.0 - (double)k) / (4096.0 - 1792.0);
  return 1.0 + f * (1.10 / 1.03 - 1.0);
}

// Predicted time (in units of one 256x256 tile's k-work at full occupancy) of one launch of
// `row_tiles_` row tiles of `o` on `share` CUs.
// With nseg > 1, each tile is nseg split-K pieces of 1/nseg of its k-work.
double tile_cost(const TileOpt& o, int64_t row_tiles_, const GemmArgs& g, int share, int nseg = 1) {
  const int64_t tiles = row_tiles_ * ((g.n + o.bn - 1) / o.bn) * g.batch * nseg;
  const int64_t cus = share > 0 ? share : 1;
  const int64_t slots = cus * o.per_cu;
  const double area = (double)o.bm * o.bn / (256.0 * 256.0) / nseg;
  double t = 0.0;
  for (int64_t left = tiles; left > 0;) {
    const int64_t now = std::min(left, slots);
    const bool alone = o.per_cu == 1 || now <= cus;
    const int64_t busy_cus = alone ? now : cus;
    const double busy = std::min(256.0, (double)busy_cus * 256.0 / (double)cus);
    const double boost = std::min(kBoostMax, std::pow(256.0 / busy, kBoostExp));
    t += area / ((alone ? o.speed_alone : o.speed) * short_k_gain(o, g.k) * boost);
    left -= now;
  }
  return t;
}

// The cheapest single tile over the units; its cost in *cost.
const TileOpt& best_single(const GemmArgs& g, const GemmUnits& u, int share, double* cost) {
  const TileOpt* best = &kTileOpts[1];
  double best_cost = 1e300;
  for (const TileOpt& o : kTileOpts) {
    const double c = tile_cost(o, row_tiles(u, o.bm), g, share);
    if (c < best_cost) {
      best_cost = c;
      best = &o;
    }
  }
  *cost = best_cost;
  return *best;
}

TilePlan choose_plan(const GemmArgs& g, const GemmUnits& u) {
  if (g.dbg && (g.dbg->tile_m > 0 || g.dbg->cut_row > 0)) {
    // forced by the handle's debug settings (validated by the caller): the tile, and a cut
    // at cut_row when that row lies inside this launch group and on a band boundary
    const TileOpt* o = find_tile(g.dbg->tile_m, g.dbg->tile_n);
    if (!o) o = find_tile(256, 256);
    TilePlan plan{o->kind};
    int64_t lo = 0, hi = 0;
    const int64_t cut = g.dbg->cut_row;
    if (cut > 0 && contiguous_rows(u, &lo, &hi) && lo < cut && cut < hi && (cut - lo) % o->bm == 0) {
      const TileOpt* t = find_tile(g.dbg->tail_m, g.dbg->tail_n);
      plan.cut = cut;
      plan.tail_kind = t ? t->kind : kTile128x128;
    }
    return plan;
  }
  const int share = 256 / (g.concurrency > 1 ? g.concurrency : 1);
  double best_cost;
  const TileOpt& one = best_single(g, u, share, &best_cost);
  TilePlan plan{one.kind};
  int64_t lo = 0, hi = 0;
  if (g.concurrency > 1 || !contiguous_rows(u, &lo, &hi)) return plan;
  // cuts: for each large tile, the row bands that fill its whole rounds
  for (const TileOpt& o : kTileOpts) {
    if (o.per_cu != 1) continue;
    const int64_t bands = (hi - lo + o.bm - 1) / o.bm;
    const int64_t band_tiles = (int64_t)((g.n + o.bn - 1) / o.bn) * g.batch;
    const int64_t slots = share > 0 ? share : 1;
    const int64_t full = bands * band_tiles / slots;          // whole rounds
    const int64_t b1 = full * slots / band_tiles;             // bands inside them
    if (b1 <= 0 || b1 >= bands) continue;
    const int64_t cut = lo + b1 * o.bm;
    double tail_cost;
    const TileOpt& t = best_single(g, clip_units(u, cut, hi), share, &tail_cost);
    const double c = tile_cost(o, b1, g, share) + tail_cost;
    if (c < best_cost * 0.98) {  // a second launch costs a little: cut only for a clear gain
      best_cost = c;
      plan = {o.kind, cut, t.kind};
    }
  }
  return plan;
}

// The split-K launch of K-segmented rows on tiles of `kind`: reduce 1 meets the segments in
// the kernel (split_meet), 2 sums them in a gemm_bf16_split_reduce launch after it.
template <int R>
hipError_t launch_split_r(int kind, const GemmArgs& g, const GemmUnits& u, hipStream_t stream,
                          int nseg) {
  constexpr int mode = R == 1 ? 2 : 3;
  switch (kind) {
    case kTile320x256:
      return launch<PP320x256>(&gemm_bf16_pingpong<PP320x256, kDist<PP320x256>, R, kLoadsInCompute<PP320x256>>, g, u, stream, mode, nseg);
    case kTile256x256:
      return launch<PP256x256>(&gemm_bf16_pingpong<PP256x256, kDist<PP256x256>, R, kLoadsInCompute<PP256x256>>, g, u, stream, mode, nseg);
    case kTile128x256:
      return launch<PP128x256>(&gemm_bf16_pingpong<PP128x256, kDist<PP128x256>, R, kLoadsInCompute<PP128x256>>, g, u, stream, mode, nseg);
    case kTile256x192:
      return launch<PP256x192>(&gemm_bf16_pingpong<PP256x192, kDist<PP256x192>, R, kLoadsInCompute<PP256x192>>, g, u, stream, mode, nseg);
    case kTile256x160:
      return launch<PP256x160>(&gemm_bf16_pingpong<PP256x160, kDist<PP256x160>, R, kLoadsInCompute<PP256x160>>, g, u, stream, mode, nseg);
    default:
      return launch<PL128x128>(&gemm_bf16_seg<PL128x128, R>, g, u, stream, mode, nseg);
  }
}

hipError_t launch_split(int kind, const GemmArgs& g, const GemmUnits& u, hipStream_t stream,
                        int nseg, int reduce) {
  return reduce == 2 ? launch_split_r<2>(kind, g, u, stream, nseg)
                     : launch_split_r<1>(kind, g, u, stream, nseg);
}

hipError_t launch_kind(int kind, const GemmArgs& g, const GemmUnits& u, hipStream_t stream) {
  if (u.n <= 0) return hipSuccess;
  switch (kind) {
    case kTile320x256:
      return launch<PP320x256>(&gemm_bf16_pingpong<PP320x256, kDist<PP320x256>, 0, kLoadsInCompute<PP320x256>>, g, u, stream);
    case kTile256x256:
      return launch<PP256x256>(&gemm_bf16_pingpong<PP256x256, kDist<PP256x256>, 0, kLoadsInCompute<PP256x256>>, g, u, stream);
    case kTile128x256:
      return launch<PP128x256>(&gemm_bf16_pingpong<PP128x256, kDist<PP128x256>, 0, kLoadsInCompute<PP128x256>>, g, u, stream);
    case kTile256x192:
      return launch<PP256x192>(&gemm_bf16_pingpong<PP256x192, kDist<PP256x192>, 0, kLoadsInCompute<PP256x192>>, g, u, stream);
    case kTile256x160:
      return launch<PP256x160>(&gemm_bf16_pingpong<PP256x160, kDist<PP256x160>, 0, kLoadsInCompute<PP256x160>>, g, u, stream);
    default:
      return launch<PL128x128>(&gemm_bf16_pipelined<PL128x128>, g, u, stream);
  }
}

const TileOpt& opt_of(int kind) {
  for (const TileOpt& o : kTileOpts)
    if (o.kind == kind) return o;
  return kTileOpts[1];
}

}  // namespace

bool gemm_bf16_tile_supported(int tile_m, int tile_n) { return find_tile(tile_m, tile_n) != nullptr; }

uint32_t* ready_flags_base(hipError_t* err) {
  static std::mutex mu;
  static std::map<int, uint32_t*> by_device;
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
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(g_ready));
  if (e != hipSuccess || !ptr) {
    *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
    return nullptr;
  }
  by_device[dev] = static_cast<uint32_t*>(ptr);
  return by_device[dev];
}

bool gemm_shape_supported(const GemmArgs& g) {
  // Offsets into B are 32-bit byte offsets from column n0 of the batch entry (up to a
  // step past k), and one A tile spans at most 320 rows; both must stay below the
  // out-of-range marker with room for a 16-byte access.
  const int64_t lim = (int64_t)OOB - 64;
  return ((int64_t)g.k + 64) * g.ldb * 2 < lim && (int64_t)320 * g.lda * 2 < lim;
}

hipError_t launch_gemm_bf16_units(const GemmArgs& g, const GemmUnits& u, hipStream_t stream) {
  if (g.n <= 0 || g.batch <= 0 || u.n <= 0) return hipSuccess;
  if (u.n > kMaxGemmUnits || g.k <= 0 || g.k % kGemmKStep != 0 || g.n % 8 != 0 ||
      !gemm_shape_supported(g))
    return hipErrorInvalidValue;
  for (int i = 0; i < u.n; ++i)
    if (u.rows[i] < 0 || u.row0[i] < 0) return hipErrorInvalidValue;
  if (g.fuse_nslots != 0) {
    if (g.fuse_nslots != g.batch || !g.fuse_out || !g.counters || g.fuse_ldo < g.n ||
        g.fuse_ldo % 8 != 0)
      return hipErrorInvalidValue;
    if (g.fuse_ring) {  // every row's shard index must lie in [0, nslots)
      int64_t last = 0;
      for (int i = 0; i < u.n; ++i)
        if (u.rows[i] > 0) last = std::max<int64_t>(last, (int64_t)u.row0[i] + u.rows[i] - 1);
      if (g.fuse_shard_rows <= 0 || g.fuse_row0 < 0 ||
          (g.fuse_row0 + last) / g.fuse_shard_rows >= g.fuse_nslots)
        return hipErrorInvalidValue;
    }
  }
  // K segmentation: rows at or after seg_row go to the segmented kernel (clamped so that no
  // segment is empty); the rows before it follow the tile plan
  const int nk = (g.k + PL128x128::BK - 1) / PL128x128::BK;
  const int nseg = std::min(g.nseg, nk);
  const bool seg = nseg > 1 && g.batch == 1 && g.fuse_nslots == 0;
  const GemmUnits plain = seg ? clip_units(u, 0, g.seg_row) : u;
  const GemmUnits segu = seg ? clip_units(u, g.seg_row, INT64_MAX) : GemmUnits{0, {}, {}};
  if (g.plan_out) {  // this launch group's plan; the call's dispatch count carries on
    const int32_t d = g.plan_out->dispatches, pieces = g.plan_out->rs_pieces;
    *g.plan_out = TilePlanRecord{};
    g.plan_out->dispatches = d;
    g.plan_out->rs_pieces = pieces;
  }
  hipError_t e = hipSuccess;
  if (plain.n > 0) {
    const TilePlan plan = choose_plan(g, plain);
    if (g.plan_out) {
      const TileOpt& a = opt_of(plan.kind);
      g.plan_out->tile_m = a.bm;
      g.plan_out->tile_n = a.bn;
      g.plan_out->cut = plan.cut;
      const TileOpt& b = opt_of(plan.tail_kind);
      g.plan_out->tail_m = plan.cut >= 0 ? b.bm : 0;
      g.plan_out->tail_n = plan.cut >= 0 ? b.bn : 0;
    }
    if (g.plan_out) g.plan_out->dispatches += plan.cut < 0 ? 1 : 2;
    if (plan.cut < 0) {
      e = launch_kind(plan.kind, g, plain, stream);
    } else {
      // two launches on one stream: the leading whole-round bands, then the rest (the fused
      // reduction's counters are back at zero when the second starts)
      int64_t lo = 0, hi = 0;
      contiguous_rows(plain, &lo, &hi);
      e = launch_kind(plan.kind, g, clip_units(plain, lo, plan.cut), stream);
      if (e == hipSuccess) e = launch_kind(plan.tail_kind, g, clip_units(plain, plan.cut, hi), stream);
    }
    if (e != hipSuccess) return e;
  }
  if (segu.n > 0) {
    // split pieces on the plan's tile (256 x 256 unless given); when the scratch cannot
    // hold their partials, the 128 x 128 folding kernel (the same bits)
    const TileOpt* o = g.seg_m > 0 ? find_tile(g.seg_m, g.seg_n) : find_tile(256, 256);
    if (!o) return hipErrorInvalidValue;
    const int64_t tiles = row_tiles(segu, o->bm) * ((g.n + o->bn - 1) / o->bn);
    const int reduce = g.seg_reduce == 1 ? 1 : 2;
    const bool split = g.split_parts && (reduce == 2 || (g.split_counters && tiles <= g.split_counters_n)) &&
                       tiles * nseg * o->bm * o->bn <= g.split_parts_n;
    if (!split) o = find_tile(128, 128);
    if (g.plan_out) {
      if (plain.n == 0) {
        g.plan_out->tile_m = o->bm;
        g.plan_out->tile_n = o->bn;
      }
      int64_t lo = 0, hi = 0;
      g.plan_out->seg_row = contiguous_rows(segu, &lo, &hi) ? lo : segu.row0[0];
      g.plan_out->nseg = nseg;
      g.plan_out->split = split ? reduce : 0;
      g.plan_out->seg_m = o->bm;
      g.plan_out->seg_n = o->bn;
      g.plan_out->dispatches += split && reduce == 2 ? 2 : 1;
    }
    e = split ? launch_split(o->kind, g, segu, stream, nseg, reduce)
              : launch<PL128x128>(&gemm_bf16_seg<PL128x128, 0>, g, segu, stream, 1, nseg);
  }
  return e;
}

namespace {

// Predicted time of the split-K launch over `rows` rows on tiles `o`, nseg pieces per tile
// (a piece does 1/nseg of the tile's k-steps), in the units of tile_cost (one 256 x 256
// tile's k-work on a CU at full occupancy, ~0.0291 us per unit of k): the pieces' rounds
// with the tile speeds and clock boost of tile_cost, plus the separate sum's launch gap and
// the partials' round trip (each piece writes its fp32 tile, the sum reads it back).  The
// two constants, 7.3 us per launch and 0.179 us per MB of partials written and read, are a
// least-squares fit of log time ratios to a forced sweep on MI355X (tile x nseg x first
// segmented row over the GQA, qkv and fc1 shapes at small T and at the tails of larger T;
// 443 points): with them the choice below lands within 2% of the best measured
// configuration at all but 4 of 44 token counts.
constexpr double kUnitUsPerK = 0.0291, kSplitGapUs = 7.3, kSplitUsPerMB = 0.179;
constexpr int64_t kSplitPartsMax = int64_t(16) << 20;  // floats: 64 MiB of partials

double seg_cost(const TileOpt& o, int64_t rows, int64_t n, int64_t k, int nseg) {
  GemmArgs g{};
  g.n = (int32_t)n;
  g.k = (int32_t)k;
  g.batch = 1;
  const int64_t row_t = (rows + o.bm - 1) / o.bm;
  const int64_t pieces = row_t * ((n + o.bn - 1) / o.bn) * nseg;
  if (pieces * o.bm * o.bn > kSplitPartsMax) return 1e30;
  const double unit_us = kUnitUsPerK * (double)k;
  const double mb = (double)pieces * o.bm * o.bn * 8.0 / 1e6;
  return tile_cost(o, row_t, g, 256, nseg) + (kSplitGapUs + kSplitUsPerMB * mb) / unit_us;
}

}  // namespace

// K segmentation of a call of T rows (device-side loop, the chip to itself): the best of no
// segmentation (one tile, or whole rounds of a large tile and a tail launch, as choose_plan
// prices them), all rows split, and whole rounds of a large tile followed by the remaining
// rows split; each split option over the four tiles the split costs were fitted on (not the
// narrow 256x192 and 256x160) and nseg in {2, 3, 4, 6, 8, 12, 16}
// (at most one segment per k-step).  Segmentation is taken only for a predicted gain of 3%.
SegPlan choose_segmentation(int64_t T, int64_t n, int64_t k, int32_t batch) {
  SegPlan none;
  const int64_t nk = (k + PL128x128::BK - 1) / PL128x128::BK;
  if (batch != 1 || T <= 0 || n <= 0 || nk < 4) return none;
  GemmArgs g{};
  g.n = (int32_t)n;
  g.k = (int32_t)k;
  g.batch = 1;
  g.concurrency = 1;
  GemmUnits u;
  u.n = 1;
  u.row0[0] = 0;
  u.rows[0] = (int32_t)T;
  double base;
  best_single(g, u, 256, &base);
  // leading whole rounds of each one-per-CU tile: (rows, cost), rows 0 for none
  std::vector<std::pair<int64_t, double>> leads = {{0, 0.0}};
  for (const TileOpt& o : kTileOpts) {
    if (o.per_cu != 1) continue;
    const int64_t bands = (T + o.bm - 1) / o.bm;
    const int64_t band_tiles = (n + o.bn - 1) / o.bn;
    const int64_t b1 = bands * band_tiles / 256 * 256 / band_tiles;
    if (b1 <= 0 || b1 >= bands) continue;
    const double lead = tile_cost(o, b1, g, 256);
    double tail;
    best_single(g, clip_units(u, b1 * o.bm, T), 256, &tail);
    base = std::min(base, (lead + tail) / 0.98);
    leads.push_back({b1 * o.bm, lead});
  }
  SegPlan best = none;
  double best_cost = base * 0.97;
  const int counts[] = {2, 3, 4, 6, 8, 12, 16};
  for (const auto& lead : leads)
    for (const TileOpt& o : kTileOpts) {
      if (o.kind == kTile256x192 || o.kind == kTile256x160) continue;  // split cost not fitted
      for (int nseg : counts) {
        if (nseg > nk) break;
        const double c = lead.second + seg_cost(o, T - lead.first, n, k, nseg);
        if (c < best_cost) {
          best_cost = c;
          best = {lead.first, nseg, o.bm, o.bn, 2};
        }
      }
    }
  return best;
}

hipError_t launch_gemm_bf16(const GemmArgs& g, hipStream_t stream) {
  if (g.m <= 0) return hipSuccess;
  GemmUnits u;
  u.n = 1;
  u.row0[0] = 0;
  u.rows[0] = g.m;
  return launch_gemm_bf16_units(g, u, stream);
}

}  // namespace ubx
