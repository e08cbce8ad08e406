// bf16 MFMA GEMM pipeline with BK = 32 stages through a 4-deep LDS ring, for
// the gradient GEMMs, whose K-outer operands (rows of W, G or H_c read along
// k) come from many separate rows per stage: three stages in flight hide
// their latency better than the two-slot BK = 64 pipeline of lce_pipe.h.
// Same workgroup shape (8 wave64, 256 x 256 tiles, 128 x 64 per wave) and the
// same operand descriptions (pipe::Opnd) as lce_pipe.h.
//
// Operand tiles travel global -> LDS with `buffer_load_dwordx4 ... lds` (no
// staging registers) through a ring of NS = 4 LDS stages of BK = 32: while a
// stage is consumed the next one has landed and the one after it is in
// flight, and the slot freed at the previous barrier takes the stage after
// those.  Each wave waits only for its
// own loads (vmcnt) and one workgroup barrier per stage publishes the stage
// and frees the slot that the next load overwrites.
//
// LDS layouts (per operand and stage, 16 KB):
//  * K-contiguous operand (element (r, k) at base[r*ld + k]): [r][k], 64-byte
//    rows of four 16-byte chunks; chunk c of row r sits in slot
//    c ^ ((r >> 2) & 3), so the 16 rows that one ds_read_b128 phase touches
//    fall in 16 distinct bank groups.
//  * K-outer operand (element (r, k) at base[k*ld + r]): [k][r], exactly as in
//    global memory, 512-byte rows; 32-byte pairs permuted by XOR with
//    2*(k & 3).  MFMA fragments come from ds_read_b64_tr_b16: within each
//    16-lane group, lane i receives element i%4 of lane (4j + i/4)'s 8-byte
//    chunk for j = 0..3, i.e. four consecutive k of one r.
#pragma once

#include "lce_pipe.h"

namespace lce {
namespace pipe32 {

constexpr int BM = 256, BN = 256, BK = 32, NS = 4;
constexpr int OPND_BYTES = 256 * BK * 2;          // one operand, one stage: 16 KB
constexpr int STAGE_BYTES = 2 * OPND_BYTES;       // A then B
constexpr int RING_BYTES = NS * STAGE_BYTES;      // 128 KB
constexpr int SCRATCH_BYTES = 4096;               // epilogue scratch after the ring
constexpr int LDS_BYTES = RING_BYTES + SCRATCH_BYTES + 4096;  // the BK=64 pipeline's footprint

constexpr int WGM = 2, WGN = 4, WTM = 128, WTN = 64, TM = 4, TN = 2;
constexpr int DMA_PER_OPND = OPND_BYTES / 1024 / 8;  // 1 KB DMA instructions per wave: 2
constexpr int DMA_PER_STAGE = 2 * DMA_PER_OPND;      // 4 per wave per stage

using pipe::GB_COLS;
using pipe::GB_ELEMS;
using pipe::GB_ROWS;
using pipe::lds_void;
using pipe::Opnd;
using pipe::raw_barrier;
using pipe::v4i16;
using pipe::wait_lgkm0;
using pipe::wait_vmcnt;

// ------------------------------------------------------------------ loads
// Per-tile load plan of one operand: a buffer resource at the tile origin
// and each lane's byte offsets for its DMA_PER_OPND instructions; a stage
// only adds its k offset.  Rows past the operand's end fall past
// num_records and load 0 in hardware.
struct Plan {
  __amdgpu_buffer_rsrc_t rs;
  uint32_t voff[DMA_PER_OPND];  // byte offsets at k = k0 of the tile
  int kc8[DMA_PER_OPND];        // K-contiguous only: k offset of the lane's chunk
  uint32_t kstride;             // bytes per unit of k (stages are 32-aligned)
  uint32_t bstride_b;           // K-outer blocked: bytes between 256-row blocks (0 = plain)
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
#pragma unroll
  for (int i = 0; i < DMA_PER_OPND; ++i) {
    const int q = (wave * DMA_PER_OPND + i) * 64 + lane;  // 16-byte chunk in the 16 KB tile
    if constexpr (KC) {
      const int row = q >> 2, slot = q & 3;
      const int kc = slot ^ ((row >> 2) & 3);
      p.voff[i] = (uint32_t)(((int64_t)row * o.ld + kc * 8) * 2);
      p.kc8[i] = kc * 8;
    } else {
      const int kr = q >> 5, c = q & 31;
      const int gp = (c >> 1) ^ (2 * (kr & 3));
      const int gv = 8 * (2 * gp + (c & 1));  // first r of the lane's 16-byte chunk
      if (o.bstride > 0)
        p.voff[i] = (uint32_t)(((int64_t)kr * GB_COLS + (gv / GB_COLS) * GB_ELEMS + gv % GB_COLS) * 2);
      else
        p.voff[i] = (uint32_t)(((int64_t)kr * o.ld + gv) * 2);
      p.kc8[i] = 0;
    }
  }
}

// Issues this wave's share (DMA_PER_OPND x 1 KB) of one stage; krel = k of
// the stage relative to the tile's k0.  K-contiguous chunks at or past krel_end
// load 0 (only checked when the stage straddles it).
template <bool KC>
__device__ __forceinline__ void issue_plan(const Plan& p, int krel, int krel_end, char* lds_opnd, int wave,
                                           bool live = true) {
  // Blocked K-outer: a stage stays inside one 256-row block (stages are 32
  // rows, blocks 256), so the stage offset is block base + row offset.
  uint32_t add = (uint32_t)krel * p.kstride;
  if constexpr (!KC)
    if (p.bstride_b) add = (uint32_t)(krel / GB_ROWS) * p.bstride_b + (uint32_t)(krel % GB_ROWS) * p.kstride;
  const bool tail = KC && (krel + BK > krel_end);
#pragma unroll
  for (int i = 0; i < DMA_PER_OPND; ++i) {
    uint32_t off = p.voff[i] + add;
    off = (tail && krel + p.kc8[i] >= krel_end) ? kOobOffset : off;
    off = live ? off : kOobOffset;  // no branch: see pipe::issue_plan
    __builtin_amdgcn_raw_ptr_buffer_load_lds(p.rs, (lds_void*)(lds_opnd + (wave * DMA_PER_OPND + i) * 1024), 16,
                                             off, 0, 0, 0);
  }
}

// ------------------------------------------------------------------ fragments
// 8 bf16 along k for MFMA lane `lane`: row/col r_base + (lane & 31),
// k = 16*kk + 8*(lane >> 5) + 0..7.
template <bool KC>
__device__ __forceinline__ u32x4 load_frag(const char* lds_opnd, int r_base, int kk, int lane) {
  if constexpr (KC) {
    const int R = r_base + (lane & 31);
    const int kc = 2 * kk + (lane >> 5);
    return *reinterpret_cast<const u32x4*>(lds_opnd + R * 64 + ((kc ^ ((R >> 2) & 3)) << 4));
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
// Operand fragments of one k-substep (16 k) of one stage.
template <int A_MODE, bool B_KC>
struct Frags {
  u32x4 a[TM], b[TN];
  __device__ __forceinline__ void load(const char* st, int kk, int wm, int wn, int lane, bool a_kc) {
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) b[tn] = load_frag<B_KC>(st + OPND_BYTES, wn * WTN + tn * 32, kk, lane);
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) a[tm] = load_frag_a<A_MODE>(st, wm * WTM + tm * 32, kk, lane, a_kc);
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
  __device__ __forceinline__ void mma0(f32x16_t (&acc)[TM][TN]) const {
    const f32x16_t z = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
        acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[tm]),
                                                              __builtin_bit_cast(bf16x8_t, b[tn]), z, 0, 0, 0);
  }
  static constexpr int kReads = (TM * (A_MODE == 0 ? 1 : 2)) + TN * (B_KC ? 1 : 2);
};

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
//   Stores an epilogue issues inside the walk only make later stage waits
//   drain more (the waits count every vector memory operation in order).
// On return no load is in flight and every wave has passed a final barrier.
// `acc` belongs to the caller: the first substep of every tile overwrites it
// (its MFMAs start from zero); after the call it holds the last tile's sums
// (single-tile callers store it themselves after run()).  With nsteps = 0 it
// is left untouched.
// kmap (optional, LDS, single-tile runs): the stages to run, as indices of
// BK-wide k steps from k0; stage s loads k = k0 + kmap[s]*BK (the other
// steps are skipped, as if their operand tiles were zero).
//
// Schedule.  Stage g sits in slot g % NS.  While stage g is consumed, stage
// g+1 has landed and stage g+2 is in flight.  Per stage: substep 0 reads
// substep 1's fragments among its first MFMAs; then each wave waits for its
// reads of slot g and its loads of stage g+1, and the barrier makes both true
// for the workgroup; substep 1 then issues stage g+3 into slot g-1 (free
// since the previous barrier) and reads stage g+1's first fragments, both
// among its MFMAs.  Stages past the end load zeros (constant counts, no
// branch).
// The explicit vmcnt waits order every LDS read after the DMA that fills its
// slot.  A stage's body takes its three slots (read now, read next, filled)
// as distinct restrict pointers, which they are, so that the compiler does
// not also drain every DMA in flight before each transposing LDS read.
template <int A_MODE, bool B_KC, typename Origin, typename Epi>
__device__ __forceinline__ void run(int ntiles, int nsteps, int kend, char* lds, f32x16_t (&acc)[TM][TN],
                                    Origin origin, Epi epi, bool a_kc = true, const int* kmap = nullptr) {
  static_assert(BK == 32 && NS == 4, "two 16-wide k-substeps per stage, four slots");
  using F = Frags<A_MODE, B_KC>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave % WGM, wn = wave / WGM;
  const int total = ntiles * nsteps;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform: keeps LDS targets scalar
  // Issue state (the next global step to load).
  int it = 0, is = 0;
  Plan pA, pB;
  auto plan_tile = [&](int t) {
    Opnd A, B;
    int k0;
    origin(t, A, B, k0);
    if constexpr (A_MODE == 0) plan_opnd<true>(pA, A, k0, wave_s, lane);
    else if constexpr (A_MODE == 1) plan_opnd<false>(pA, A, k0, wave_s, lane);
    else if (a_kc) plan_opnd<true>(pA, A, k0, wave_s, lane);
    else plan_opnd<false>(pA, A, k0, wave_s, lane);
    plan_opnd<B_KC>(pB, B, k0, wave_s, lane);
  };
  plan_tile(0);
  auto issue = [&](char* st, const int* km, bool live) {
    const int kr = live ? (km ? __builtin_amdgcn_readfirstlane(km[is]) : is) * BK : 0;
    if constexpr (A_MODE == 0) issue_plan<true>(pA, kr, kend, st, wave_s, live);
    else if constexpr (A_MODE == 1) issue_plan<false>(pA, kr, kend, st, wave_s, live);
    else if (a_kc) issue_plan<true>(pA, kr, kend, st, wave_s, live);
    else issue_plan<false>(pA, kr, kend, st, wave_s, live);
    issue_plan<B_KC>(pB, kr, kend, st + OPND_BYTES, wave_s, live);
  };
  auto advance = [&]() {
    if (++is == nsteps) {
      is = 0;
      if (++it < ntiles) plan_tile(it);
    }
  };
#pragma unroll
  for (int g = 0; g < NS - 1; ++g) {
    const bool live = g < total;
    issue(lds + g * STAGE_BYTES, kmap, live);
    if (live) advance();
  }
  // Stage 0 must have landed (stages 1 and 2 may stay in flight).
  wait_vmcnt<(NS - 2) * DMA_PER_STAGE>();
  raw_barrier();
  F x, y;
  x.load(lds, 0, wm, wn, lane, a_kc);

  // One stage: cur = slot g, nxt = slot g+1, dst = slot g+3 (= g-1).
  auto stage = [&](const char* __restrict__ cur, const char* __restrict__ nxt, char* __restrict__ dst,
                   const int* __restrict__ km, int g, auto first) {
    y.load(cur, 1, wm, wn, lane, a_kc);
    if constexpr (decltype(first)::value) x.mma0(acc);
    else x.mma(acc);
    pipe::front_reads<F::kReads, TM * TN>();
    __builtin_amdgcn_sched_barrier(0);
    wait_lgkm0();
    wait_vmcnt<DMA_PER_STAGE>();  // stage g+1 landed (stage g+2 may stay in flight)
    raw_barrier();
    const bool more = g + NS - 1 < total;
    issue(dst, km, more);
    x.load(nxt, 0, wm, wn, lane, a_kc);
    y.mma(acc);
    pipe::front_dma_reads<DMA_PER_STAGE, F::kReads, TM * TN>();
    __builtin_amdgcn_sched_barrier(0);
    if (more) advance();
  };
  // The tile's first stage is a separate copy (its first substep starts the
  // sums from zero), so no branch splits the substep schedule.
  auto run_stage = [&](int g, auto first) {
    stage(lds + (g & (NS - 1)) * STAGE_BYTES, lds + ((g + 1) & (NS - 1)) * STAGE_BYTES,
          lds + ((g + NS - 1) & (NS - 1)) * STAGE_BYTES, kmap, g, first);
  };
  for (int t = 0; t < ntiles && nsteps > 0; ++t) {
    run_stage(t * nsteps, std::true_type{});
    for (int s = 1; s < nsteps; ++s) run_stage(t * nsteps + s, std::false_type{});
    epi(t, acc);
  }
  // Loads past the end wrote zeros into free slots: done before the LDS is reused.
  wait_vmcnt<0>();
  wait_lgkm0();
  raw_barrier();
}

}  // namespace pipe32
}  // namespace lce
