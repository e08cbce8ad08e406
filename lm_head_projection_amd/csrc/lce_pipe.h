// bf16 MFMA GEMM pipeline for gfx950 built on direct-to-LDS buffer loads.
//
// One workgroup (8 wave64, two per SIMD) computes a sequence of 256 x 256
// output tiles; each wave owns a 128 x 64 part (4 x 2 blocks of
// v_mfma_f32_32x32x16_bf16).  Operand tiles travel
// global -> LDS with `buffer_load_dwordx4 ... lds` (no staging registers) in
// stages of BK = 64, through two LDS slots: while the MFMAs consume stage g
// from registers, stage g+1 sits in LDS and stage g+2 is in flight.  A stage
// is read into registers in four 16-wide k-substeps, double-buffered: the
// fragments of substep j+1 are read while the MFMAs of substep j run.  One
// workgroup barrier per stage publishes the next stage and frees the slot the
// following load overwrites; the loads of the next tile's first stages
// overlap the current tile's epilogue.
//
// LDS layouts (per operand and stage, 32 KB):
//  * K-contiguous operand: [r][k], 128-byte rows of eight 16-byte chunks;
//    chunk c of row r sits in slot c ^ ((r >> 1) & 7), so the 16 rows one
//    ds_read_b128 phase touches fall in 16 distinct 16-byte bank groups.
//    Each row is one full 128-byte line of the source per stage.
//  * K-outer operand (element (r, k) at base[k*ld + r]): [k][r], 512-byte
//    rows; 32-byte pairs permuted by XOR with 2*(k & 3).  MFMA fragments come
//    from ds_read_b64_tr_b16: within each 16-lane group, lane i receives
//    element i%4 of lane (4j + i/4)'s 8-byte chunk for j = 0..3, i.e. four
//    consecutive k of one r.
#pragma once

#include <type_traits>

#include "lce_device.h"

namespace lce {
namespace pipe {

constexpr int BM = 256, BN = 256, BK = 64, NSLOT = 2;
constexpr int NWAVES = 8, THREADS = 64 * NWAVES;
constexpr int OPND_BYTES = 256 * BK * 2;          // one operand, one stage: 32 KB
constexpr int STAGE_BYTES = 2 * OPND_BYTES;       // A then B
constexpr int RING_BYTES = NSLOT * STAGE_BYTES;   // 128 KB
constexpr int SCRATCH_BYTES = 4096;               // epilogue scratch after the ring
constexpr int BIAS_SLOTS = 4, BIAS_SLOT_BYTES = 1024;  // per-tile bias slices after the scratch
constexpr int BIAS_OFFSET = RING_BYTES + SCRATCH_BYTES;
constexpr int LDS_BYTES = BIAS_OFFSET + BIAS_SLOTS * BIAS_SLOT_BYTES;

// LDS copy of the bias slice of tile t (element j = bias[m0(t) + j], 0 past V).
__device__ __forceinline__ const uint16_t* bias_slice(const char* lds, int t) {
  return reinterpret_cast<const uint16_t*>(lds + BIAS_OFFSET + (t & (BIAS_SLOTS - 1)) * BIAS_SLOT_BYTES);
}
constexpr int WGM = 2, WGN = NWAVES / 2, WTM = BM / WGM, WTN = BN / WGN, TM = WTM / 32, TN = WTN / 32;
constexpr int DMA_PER_OPND = OPND_BYTES / 1024 / NWAVES;  // 1 KB DMA instructions per wave and operand: 4
constexpr int DMA_PER_STAGE = 2 * DMA_PER_OPND;           // 8 per wave per stage

typedef __attribute__((address_space(3))) void lds_void;
typedef short v4i16 __attribute__((ext_vector_type(4)));

// One operand of one output tile.
//   K-contiguous: element (r, k) at base[r*ld + (k/32)*32*kstep + k%32]
//     (kstep = 1: plain row-major; kstep = 256: the blocked G layout, whose
//     256 x 32 blocks follow each other along k).
//   K-outer: element (r, k) at base[k*ld + r], or, with bstride > 0 (blocked
//     G read transposed), at base[(k/256)*bstride + (k%256)*32 + (r/32)*8192 + r%32].
struct Opnd {
  const uint16_t* base;  // operand origin
  int64_t elems;         // elements from base to the end of the operand
  int64_t ld;            // leading dimension (elements)
  int r0;                // first row (M or N index) of the tile
  int64_t kstep = 1;     // K-contiguous only (see above)
  int64_t bstride = 0;   // K-outer only: > 0 selects the blocked layout
};

// Blocked G: 256 rows (c) x 32 columns (v) per 16 KB block; blocks of one row
// block follow each other along v, row blocks are `nvb` blocks apart.
constexpr int GB_ROWS = 256, GB_COLS = 32, GB_ELEMS = GB_ROWS * GB_COLS;
__host__ __device__ __forceinline__ int64_t gblock_offset(int64_t c, int64_t v, int64_t nvb) {
  return ((c / GB_ROWS) * nvb + v / GB_COLS) * GB_ELEMS + (c % GB_ROWS) * GB_COLS + v % GB_COLS;
}

// s_waitcnt with only vmcnt constrained (expcnt and lgkmcnt left free).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (0 << 8) | (3 << 14)); }
// Workgroup barrier without a memory fence (a fence would drain every
// in-flight LDS load); callers wait for what they need explicitly.
__device__ __forceinline__ void raw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ------------------------------------------------------------------ loads
// Per-tile load plan of one operand: a buffer resource at the tile origin
// and the byte offset of each of this wave's DMA_PER_OPND chunks at k = k0.
// Chunk i of a lane sits at vb[i & 1] + ub + i * us: the lane-dependent part
// only alternates with the parity of i, the rest is uniform, so a plan costs
// 2 VGPRs per operand.  Offsets are whole byte offsets (never split into an
// SGPR part), so rows past the operand's end fall past num_records and load
// 0 in hardware.
struct Plan {
  __amdgpu_buffer_rsrc_t rs;
  uint32_t vb[2];      // lane part of the offsets of even / odd chunks
  int kc8[2];          // K-contiguous only: k offset of the lane's even / odd chunk
  uint32_t ub, us;     // uniform part: ub + i * us
  uint32_t kstride;    // bytes per unit of k (stages are 64-aligned)
  uint32_t bstride_b;  // K-outer blocked: bytes between 256-row blocks (0 = plain)
};

template <bool KC>
__device__ __forceinline__ void plan_opnd(Plan& p, const Opnd& o, int k0, int wave, int lane) {
  p.bstride_b = 0;
  if constexpr (KC) {
    const int64_t base = (int64_t)o.r0 * o.ld + (int64_t)k0 * o.kstep;
    p.rs = make_rsrc(o.base + base, (o.elems - base) * 2);
    p.kstride = (uint32_t)(o.kstep * 2);
  } else if (o.bstride > 0) {
    // k0 is a multiple of 256 here (it is 0 for the transposed-G operand).
    const int64_t base = (int64_t)(k0 / GB_ROWS) * o.bstride + (int64_t)(o.r0 / GB_COLS) * GB_ELEMS;
    p.rs = make_rsrc(o.base + base, (o.elems - base) * 2);
    p.kstride = GB_COLS * 2;
    p.bstride_b = (uint32_t)(o.bstride * 2);
  } else {
    const int64_t base = (int64_t)k0 * o.ld + o.r0;
    p.rs = make_rsrc(o.base + base, (o.elems - base) * 2);
    p.kstride = (uint32_t)(o.ld * 2);
  }
  // Chunk q = (wave*DMA_PER_OPND + i)*64 + lane of the 32 KB stage tile.
  if constexpr (KC) {
    // row = q >> 3 = 8*(wave*DMA_PER_OPND + i) + (lane >> 3); slot = lane & 7;
    // the chunk brings k chunk kc = slot ^ ((row >> 1) & 7), and
    // (row >> 1) & 7 = (4*i + (lane >> 4)) & 7 depends on i only by parity.
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int kc = (lane & 7) ^ ((4 * par + (lane >> 4)) & 7);
      p.vb[par] = (uint32_t)(((int64_t)(lane >> 3) * o.ld + (int64_t)(kc >> 2) * 32 * o.kstep + (kc & 3) * 8) * 2);
      p.kc8[par] = kc * 8;
    }
    p.us = (uint32_t)(8 * o.ld * 2);
    p.ub = (uint32_t)(wave * DMA_PER_OPND) * p.us;
  } else {
    // kr = q >> 5 = 2*(wave*DMA_PER_OPND + i) + (lane >> 5); c = lane & 31;
    // the 32-byte pair swizzle 2*(kr & 3) depends on i only by parity.
#pragma unroll
    for (int par = 0; par < 2; ++par) {
      const int krl = lane >> 5, c = lane & 31;
      const int gp = (c >> 1) ^ (2 * ((2 * par + krl) & 3));
      const int gv = 8 * (2 * gp + (c & 1));  // first r of the lane's 16-byte chunk
      if (o.bstride > 0)
        p.vb[par] = (uint32_t)(((int64_t)krl * GB_COLS + (gv / GB_COLS) * GB_ELEMS + gv % GB_COLS) * 2);
      else
        p.vb[par] = (uint32_t)(((int64_t)krl * o.ld + gv) * 2);
      p.kc8[par] = 0;
    }
    p.us = o.bstride > 0 ? (uint32_t)(2 * GB_COLS * 2) : (uint32_t)(2 * o.ld * 2);
    p.ub = (uint32_t)(wave * DMA_PER_OPND) * p.us;
  }
}

// Issues this wave's share (DMA_PER_OPND x 1 KB) of one stage; krel = k of
// the stage relative to the tile's k0.  K-contiguous chunks at or past krel_end
// load 0 (only checked when the stage straddles it).  With `live` false every
// chunk takes an offset past the operand, so the hardware writes zeros into
// the slot: the issue has no branch and its loads can be scheduled among MFMAs.
template <bool KC>
__device__ __forceinline__ void issue_plan(const Plan& p, int krel, int krel_end, char* lds_opnd, int wave,
                                           bool live = true) {
  // Blocked K-outer: a stage stays inside one 256-row block (stages are 64
  // rows, blocks 256), so the stage offset is block base + row offset.
  uint32_t add = (uint32_t)krel * p.kstride;
  if constexpr (!KC)
    if (p.bstride_b) add = (uint32_t)(krel / GB_ROWS) * p.bstride_b + (uint32_t)(krel % GB_ROWS) * p.kstride;
  const bool tail = KC && (krel + BK > krel_end);
#pragma unroll
  for (int i = 0; i < DMA_PER_OPND; ++i) {
    // readfirstlane keeps the uniform sum in an SGPR computed here (not 8
    // precomputed per-lane offsets held across the loop).
    const uint32_t u = __builtin_amdgcn_readfirstlane(p.ub + (uint32_t)i * p.us + add);
    uint32_t off = p.vb[i & 1] + u;
    off = (tail && krel + p.kc8[i & 1] >= krel_end) ? kOobOffset : off;
    off = live ? off : kOobOffset;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(p.rs, (lds_void*)(lds_opnd + (wave * DMA_PER_OPND + i) * 1024), 16,
                                             off, 0, 0, 0);
  }
}

// ------------------------------------------------------------------ fragments
// 8 bf16 along k for MFMA lane `lane`: row/col r_base + (lane & 31),
// k = 16*kk + 8*(lane >> 5) + 0..7 (kk = 0..3 within the stage).
template <bool KC>
__device__ __forceinline__ u32x4 load_frag(const char* lds_opnd, int r_base, int kk, int lane) {
  if constexpr (KC) {
    const int R = r_base + (lane & 31);
    const int kc = 2 * kk + (lane >> 5);
    return *reinterpret_cast<const u32x4*>(lds_opnd + R * 128 + ((kc ^ ((R >> 1) & 7)) << 4));
  } else {
    const int a = lane & 15;
    const int n = r_base + 16 * ((lane >> 4) & 1) + 4 * (a & 3);
    const int k = 16 * kk + 8 * (lane >> 5) + (a >> 2);
    const char* p = lds_opnd + k * 512 + ((((n >> 4) ^ (2 * (k & 3)))) << 5) + ((n & 15) << 1);
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)p);
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p + 4 * 512));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return u32x4{l2[0], l2[1], h2[0], h2[1]};
  }
}

// A operand layout: 0 = K-contiguous, 1 = K-outer, 2 = chosen at run time by
// a wave-uniform flag (one pipeline serves both layouts).
template <int A_MODE>
__device__ __forceinline__ u32x4 load_frag_a(const char* sa, int r_base, int kk, int lane, bool a_kc) {
  if constexpr (A_MODE == 0) return load_frag<true>(sa, r_base, kk, lane);
  else if constexpr (A_MODE == 1) return load_frag<false>(sa, r_base, kk, lane);
  else return a_kc ? load_frag<true>(sa, r_base, kk, lane) : load_frag<false>(sa, r_base, kk, lane);
}
// Operand fragments of one k-substep (16 k) of one stage.  (Used for
// K-contiguous operands; a K-outer fragment takes two transposing reads.)
template <int A_MODE, bool B_KC>
struct Frags {
  u32x4 a[TM], b[TN];
  __device__ __forceinline__ void load(const char* st, int kk, int wm, int wn, int lane, bool a_kc) {
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) a[tm] = load_frag_a<A_MODE>(st, wm * WTM + tm * 32, kk, lane, a_kc);
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) b[tn] = load_frag<B_KC>(st + OPND_BYTES, wn * WTN + tn * 32, kk, lane);
  }
  __device__ __forceinline__ void mma(f32x16_t (&acc)[TM][TN]) const {
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
        acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[tm]),
                                                              __builtin_bit_cast(bf16x8_t, b[tn]),
                                                              acc[tm][tn], 0, 0, 0);
  }
  // First substep of a tile: the sums start from zero in the MFMA.
  __device__ __forceinline__ void mma0(f32x16_t (&acc)[TM][TN]) const {
    const f32x16_t z = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
        acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[tm]),
                                                              __builtin_bit_cast(bf16x8_t, b[tn]), z, 0, 0, 0);
  }
  // LDS read instructions per substep (a transposed fragment takes two).
  static constexpr int kReads = TM * (A_MODE == 0 ? 1 : 2) + TN * (B_KC ? 1 : 2);
};

// Schedule of one substep's M MFMAs and the R fragment reads (of the next
// substep) issued among them: the reads go out between the first MFMAs, so
// they have the remaining MFMAs' time to land (R > M puts several reads
// after one MFMA).
template <int R, int M>
__device__ __forceinline__ void front_reads() {
  if constexpr (R > 0 && M > 0) {
    constexpr int r = (R + M - 1) / M;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, r, 0);
    front_reads<R - r, M - 1>();
  } else if constexpr (M > 0) {
    __builtin_amdgcn_sched_group_barrier(0x008, M, 0);
  }
}
// The substep that follows a stage barrier: the DMA instructions of a later
// stage (Q) and the next substep's fragment reads (R) among its M MFMAs.
template <int Q, int R, int M>
__device__ __forceinline__ void front_dma_reads() {
  if constexpr (M > 0 && (Q > 0 || R > 0)) {
    constexpr int q = (Q + M - 1) / M, r = (R + M - 1) / M;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (q > 0) __builtin_amdgcn_sched_group_barrier(0x020, q, 0);
    if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);
    front_dma_reads<Q - q, R - r, M - 1>();
  } else if constexpr (M > 0) {
    __builtin_amdgcn_sched_group_barrier(0x008, M, 0);
  }
}

__device__ __forceinline__ void zero(f32x16_t (&acc)[TM][TN]) {
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[tm][tn][i] = 0.f;
}

// Runs ntiles output tiles back to back through one continuous pipeline.
//   origin(t, A, B, k0): operands of tile t and its first k;
//   nsteps: BK-stages per tile (all tiles alike); kend: K-contiguous k bound
//   (relative to the same origin as k0 + s*BK);
//   epi(t, acc): consumes tile t's accumulator (registers; may use the LDS
//   scratch after the ring, with raw_barrier + wait_lgkm0 for its own sync).
// On return no load is in flight and every wave has passed a final barrier.
// `acc` belongs to the caller; the first substep of every tile overwrites it
// (its MFMAs start from zero) and, after the call, it holds the last tile's
// sums (single-tile callers store it themselves after run()).
// EPI_STORES: vector memory operations every wave's epilogue certainly
// issues (an undercount is safe: the first stage wait after an epilogue then
// also drains some of them).  Vector memory operations retire in issue order
// on this target, so those younger stores need not be waited for.
// With HAS_BIAS and `bias` (A K-contiguous, A.r0 = the tile's first vocabulary row),
// wave 0 also loads each tile's 256 bias values into bias_slice(lds, t),
// right before that tile's first stage: the stage wait that publishes the
// stage publishes the slice too.  A slot is reloaded 4 tiles later, after
// the barriers that follow the last epilogue that read it.
//
// Schedule.  Per stage g (slot g & 1), substeps 0..2 each read the next
// substep's fragments among their first MFMAs; the compiler's own waits hold
// an MFMA until its fragments have landed, and a scheduling fence keeps each
// substep's MFMAs ahead of the next substep's.  After substep 2 every wave has
// its reads of slot g done (lgkm wait) and its loads of stage g+1 landed (vm
// wait); the barrier makes both true for the workgroup, so during substep 3
// slot g takes stage g+2 (DMA) and stage g+1's first fragments are read, both
// among substep 3's MFMAs.  Past the last stage these loads take an offset
// past the operand (zeros into a free slot) and the reads fetch values nobody
// uses, so no branch splits the substep.
template <int A_MODE, bool B_KC, int EPI_STORES = 0, bool HAS_BIAS = false, typename Origin, typename Epi>
__device__ __forceinline__ void run(int ntiles, int nsteps, int kend, char* lds, f32x16_t (&acc)[TM][TN],
                                    Origin origin, Epi epi, bool a_kc = true,
                                    const uint16_t* bias = nullptr, int V = 0) {
  static_assert(BK == 64, "four 16-wide k-substeps per stage");
  using F = Frags<A_MODE, B_KC>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave % WGM, wn = wave / WGM;
  const int total = ntiles * nsteps;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform: keeps LDS targets scalar
  // Issue state (the next global stage to load).
  int it = 0, is = 0;
  Plan pA, pB;
  int bias_m0 = 0;
  auto plan_tile = [&](int t) {
    Opnd A, B;
    int k0;
    origin(t, A, B, k0);
    bias_m0 = A.r0;
    if constexpr (A_MODE == 0) plan_opnd<true>(pA, A, k0, wave_s, lane);
    else if constexpr (A_MODE == 1) plan_opnd<false>(pA, A, k0, wave_s, lane);
    else if (a_kc) plan_opnd<true>(pA, A, k0, wave_s, lane);
    else plan_opnd<false>(pA, A, k0, wave_s, lane);
    plan_opnd<B_KC>(pB, B, k0, wave_s, lane);
  };
  plan_tile(0);
  auto issue = [&](int g, bool live) {
    char* st = lds + (g & 1) * STAGE_BYTES;
    if (HAS_BIAS && is == 0 && wave_s == 0 && live) {
      const __amdgpu_buffer_rsrc_t rb = make_rsrc(bias + bias_m0, (int64_t)(V - bias_m0) * 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(lds + BIAS_OFFSET + (it & (BIAS_SLOTS - 1)) * BIAS_SLOT_BYTES),
                                               16, (uint32_t)lane * 16, 0, 0, 0);
    }
    if constexpr (A_MODE == 0) issue_plan<true>(pA, is * BK, kend, st, wave_s, live);
    else if constexpr (A_MODE == 1) issue_plan<false>(pA, is * BK, kend, st, wave_s, live);
    else if (a_kc) issue_plan<true>(pA, is * BK, kend, st, wave_s, live);
    else issue_plan<false>(pA, is * BK, kend, st, wave_s, live);
    issue_plan<B_KC>(pB, is * BK, kend, st + OPND_BYTES, wave_s, live);
  };
  auto advance = [&]() {
    if (++is == nsteps) {
      is = 0;
      if (++it < ntiles) plan_tile(it);
    }
  };
  issue(0, true);
  advance();
  if (total > 1) {
    issue(1, true);
    advance();
  }
  // Stage 0 must have landed (stage 1 may stay in flight).
  if (total > 1) wait_vmcnt<DMA_PER_STAGE>();
  else wait_vmcnt<0>();
  raw_barrier();
  F x, y;
  x.load(lds, 0, wm, wn, lane, a_kc);

  // One stage; FIRST: the tile's first, whose first substep starts the sums
  // from zero (a separate copy, so no branch splits the substep schedule).
  auto stage = [&](int g, auto first) {
    const char* st = lds + (g & 1) * STAGE_BYTES;
    y.load(st, 1, wm, wn, lane, a_kc);
    if constexpr (decltype(first)::value) x.mma0(acc);
    else x.mma(acc);
    front_reads<F::kReads, TM * TN>();
    __builtin_amdgcn_sched_barrier(0);
    x.load(st, 2, wm, wn, lane, a_kc);
    y.mma(acc);
    front_reads<F::kReads, TM * TN>();
    __builtin_amdgcn_sched_barrier(0);
    y.load(st, 3, wm, wn, lane, a_kc);
    x.mma(acc);
    front_reads<F::kReads, TM * TN>();
    __builtin_amdgcn_sched_barrier(0);
    wait_lgkm0();
    if (g + 1 < total) {
      // Stage g+1 must have landed; the stores of an epilogue that ran
      // after its loads were issued may stay in flight.
      if (EPI_STORES > 0 && decltype(first)::value && g > 0) wait_vmcnt<EPI_STORES>();
      else wait_vmcnt<0>();
    }
    raw_barrier();
    const bool more2 = g + 2 < total;
    issue(g + 2, more2);
    x.load(lds + ((g + 1) & 1) * STAGE_BYTES, 0, wm, wn, lane, a_kc);
    y.mma(acc);
    front_dma_reads<DMA_PER_STAGE, F::kReads, TM * TN>();
    __builtin_amdgcn_sched_barrier(0);
    if (more2) advance();
  };
  for (int t = 0; t < ntiles; ++t) {
    stage(t * nsteps, std::true_type{});
    for (int s = 1; s < nsteps; ++s) stage(t * nsteps + s, std::false_type{});
    epi(t, acc);
  }
  // The last two stages issued loads past the operand: they must have
  // written their zeros before the workgroup's LDS can be reused.
  wait_vmcnt<0>();
  wait_lgkm0();
  raw_barrier();
}

// run_ko: run() re-framed for K-outer operands (same contract).
// Schedule.  One iteration runs from a stage barrier to the next.  After
// barrier g-1 (every wave done with slot g-1, stage g landed), iteration g
// issues stage g+1 into slot g-1 and reads stage g's first fragments among
// the MFMAs of stage g-1's last substep; at the first stage of a tile the
// previous tile's epilogue follows.  Substeps 0..2 of stage g then each read
// the next substep's fragments among their first MFMAs (the compiler's own
// waits hold an MFMA until its fragments have landed; a scheduling fence
// keeps each substep's MFMAs ahead of the next substep's).  Each wave then
// waits for its reads of slot g and its loads of stage g+1, and barrier g
// makes both true for the workgroup.  Past the last stage the loads take an
// offset past the operand (zeros into a free slot), so no branch splits the
// schedule.  An iteration reads only slot g and fills only slot g-1: it takes
// them as distinct restrict pointers, so that the compiler does not also
// drain every DMA in flight before a transposing LDS read (K-outer operands);
// the explicit vmcnt waits order each read after the DMA that fills its slot.
template <int A_MODE, bool B_KC, int EPI_STORES = 0, bool HAS_BIAS = false, typename Origin, typename Epi>
__device__ __forceinline__ void run_ko(int ntiles, int nsteps, int kend, char* lds, f32x16_t (&acc)[TM][TN],
                                       Origin origin, Epi epi, bool a_kc = true,
                                       const uint16_t* bias = nullptr, int V = 0) {
  static_assert(BK == 64, "four 16-wide k-substeps per stage");
  using F = Frags<A_MODE, B_KC>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave % WGM, wn = wave / WGM;
  const int total = ntiles * nsteps;
  if (total == 0) return;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform: keeps LDS targets scalar
  // Issue state (the next global stage to load).
  int it = 0, is = 0;
  Plan pA, pB;
  int bias_m0 = 0;
  auto plan_tile = [&](int t) {
    Opnd A, B;
    int k0;
    origin(t, A, B, k0);
    bias_m0 = A.r0;
    if constexpr (A_MODE == 0) plan_opnd<true>(pA, A, k0, wave_s, lane);
    else if constexpr (A_MODE == 1) plan_opnd<false>(pA, A, k0, wave_s, lane);
    else if (a_kc) plan_opnd<true>(pA, A, k0, wave_s, lane);
    else plan_opnd<false>(pA, A, k0, wave_s, lane);
    plan_opnd<B_KC>(pB, B, k0, wave_s, lane);
  };
  plan_tile(0);
  auto issue = [&](char* st, bool live) {
    if (HAS_BIAS && is == 0 && wave_s == 0 && live) {
      const __amdgpu_buffer_rsrc_t rb = make_rsrc(bias + bias_m0, (int64_t)(V - bias_m0) * 2);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void*)(lds + BIAS_OFFSET + (it & (BIAS_SLOTS - 1)) * BIAS_SLOT_BYTES),
                                               16, (uint32_t)lane * 16, 0, 0, 0);
    }
    if constexpr (A_MODE == 0) issue_plan<true>(pA, is * BK, kend, st, wave_s, live);
    else if constexpr (A_MODE == 1) issue_plan<false>(pA, is * BK, kend, st, wave_s, live);
    else if (a_kc) issue_plan<true>(pA, is * BK, kend, st, wave_s, live);
    else issue_plan<false>(pA, is * BK, kend, st, wave_s, live);
    issue_plan<B_KC>(pB, is * BK, kend, st + OPND_BYTES, wave_s, live);
  };
  auto advance = [&]() {
    if (++is == nsteps) {
      is = 0;
      if (++it < ntiles) plan_tile(it);
    }
  };
  issue(lds, true);
  advance();
  wait_vmcnt<0>();  // stage 0 landed
  raw_barrier();
  F x, y;
  // Iteration g: cur = slot g, dst = slot g+1 (= g-1).  FIRST: the tile's
  // first stage (its first substep starts the sums from zero; the previous
  // tile's epilogue runs first).  PREV: stage g-1's last substep is pending.
  auto iter = [&](const char* __restrict__ cur, char* __restrict__ dst, int g, int t, auto first, auto prev) {
    constexpr bool kFirst = decltype(first)::value, kPrev = decltype(prev)::value;
    const bool live = g + 1 < total;
    issue(dst, live);
    x.load(cur, 0, wm, wn, lane, a_kc);
    if constexpr (kPrev) {
      y.mma(acc);
      front_dma_reads<DMA_PER_STAGE, F::kReads, TM * TN>();
      __builtin_amdgcn_sched_barrier(0);
    }
    if (live) advance();
    if constexpr (kFirst && kPrev) epi(t - 1, acc);
    y.load(cur, 1, wm, wn, lane, a_kc);
    if constexpr (kFirst) x.mma0(acc);
    else x.mma(acc);
    front_reads<F::kReads, TM * TN>();
    __builtin_amdgcn_sched_barrier(0);
    x.load(cur, 2, wm, wn, lane, a_kc);
    y.mma(acc);
    front_reads<F::kReads, TM * TN>();
    __builtin_amdgcn_sched_barrier(0);
    y.load(cur, 3, wm, wn, lane, a_kc);
    x.mma(acc);
    front_reads<F::kReads, TM * TN>();
    __builtin_amdgcn_sched_barrier(0);
    wait_lgkm0();
    // Stage g+1 must have landed; the stores of an epilogue that ran after
    // its loads were issued may stay in flight.
    if (kFirst && kPrev && EPI_STORES > 0) wait_vmcnt<EPI_STORES>();
    else wait_vmcnt<0>();
    raw_barrier();
  };
  auto slot = [&](int g) { return lds + (g & 1) * STAGE_BYTES; };
  iter(slot(0), slot(1), 0, 0, std::true_type{}, std::false_type{});
  for (int s = 1; s < nsteps; ++s) iter(slot(s), slot(s + 1), s, 0, std::false_type{}, std::true_type{});
  for (int t = 1; t < ntiles; ++t) {
    const int g0 = t * nsteps;
    iter(slot(g0), slot(g0 + 1), g0, t, std::true_type{}, std::true_type{});
    for (int s = 1; s < nsteps; ++s) iter(slot(g0 + s), slot(g0 + s + 1), g0 + s, t, std::false_type{}, std::true_type{});
  }
  y.mma(acc);  // the last stage's last substep
  epi(ntiles - 1, acc);
  // The last stage issued loads past the operand: they must have written
  // their zeros before the workgroup's LDS can be reused.
  wait_vmcnt<0>();
  wait_lgkm0();
  raw_barrier();
}

}  // namespace pipe
}  // namespace lce
