// Kernels of the fused linear-cross-entropy path (gfx950).
//
//   K0  k_cmp_one, or k_cmp_count / k_cmp_scan /   valid-token compaction
//       k_cmp_scatter above 65536 positions
//   K1  k_gather                                   supervised rows H[idx] -> Hc
//                                                  (and per-position fills)
//   K2  k_fwd                                      score tiles + running (m, s)
//   K3  k_merge / k_loss_sum                       split merge, per-row CE, mean
//   K4  replay_body                                score tiles -> G = p - onehot
//   K5  grad_body                                  dH (+= G W) and dW (= G^T Hc)
//       launched as k_replay (K4 of the first chunk), k_grad_replay (K5 of
//       chunk c with K4 of chunk c+1, bf16) and k_grad (K5 of the last chunk;
//       fp32: K4 and K5 of every chunk apart)
//   K6  k_dh_finalize / k_db_finalize              ordered sums, cast
//   k_row_scale                                    per-row factor r_c of G,
//                                                  inverse row map
//
// Page references are to "分块交叉熵：从输出投影开始省保存量" (glenzli.com):
// section 01 (objective, tile steps), section 02 (running LSE), section 04
// (replay and the three gradient accumulations).
#pragma once

#include "lce_device.h"
#include "lce_pipe.h"
#include "lce_pipe32.h"

namespace lce {

static_assert(Geo<uint16_t>::TM == pipe::TM && Geo<uint16_t>::TN == pipe::TN && Geo<uint16_t>::WGM == pipe::WGM &&
                  Geo<uint16_t>::WGN == pipe::WGN && pipe::THREADS == kThreads && Cfg<uint16_t>::BM == pipe::BM &&
                  Cfg<uint16_t>::BN == pipe::BN,
              "the bf16 kernels and the BK=64 pipeline agree on the tile geometry");
static_assert(Geo<uint16_t>::TM == pipe32::TM && Geo<uint16_t>::TN == pipe32::TN && Geo<uint16_t>::WGM == pipe32::WGM &&
                  Geo<uint16_t>::WGN == pipe32::WGN && Cfg<uint16_t>::BK == pipe32::BK &&
                  pipe::LDS_BYTES == pipe32::LDS_BYTES,
              "the gradient kernel and the BK=32 pipeline agree on the tile geometry");

// ============================================================== K0 compaction
// a_i = 1[mask_i] 1[y_i != ignore] (section 01).  Three passes: per-block
// counts, one-block exclusive scan of the counts, ordered scatter.  No atomics.
constexpr int kCmpBlock = 256;
// Row blocks per L2 group in the score-tile kernels (see grouped_index): each
// item walks its W tiles with a fixed block of rows, and 4 row blocks keep an
// XCD's share of H_c at 2 MB of its 4 MB L2.
constexpr int kGroupRows = 4;

__device__ __forceinline__ bool is_supervised(const int64_t* labels, const uint8_t* mask, int64_t i,
                                              int64_t ignore) {
  return labels[i] != ignore && (mask == nullptr || mask[i] != 0);
}

__global__ __launch_bounds__(kCmpBlock) void k_cmp_count(const int64_t* __restrict__ labels,
                                                         const uint8_t* __restrict__ mask, int64_t N,
                                                         int64_t V, int64_t ignore, int* counts,
                                                         int* bad) {
  __shared__ int s_cnt[kCmpBlock / kWarp];
  __shared__ int s_bad[kCmpBlock / kWarp];
  const int64_t i = (int64_t)blockIdx.x * kCmpBlock + threadIdx.x;
  bool sup = false, oob = false;
  if (i < N) {
    sup = is_supervised(labels, mask, i, ignore);
    const int64_t y = labels[i];
    oob = sup && (y < 0 || y >= V);
  }
  const uint64_t bal = __ballot(sup);
  const int anybad = __any(oob);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
    s_cnt[wave] = __popcll(bal);
    s_bad[wave] = anybad;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int c = 0, b = 0;
    for (int w = 0; w < kCmpBlock / kWarp; ++w) {
      c += s_cnt[w];
      b |= s_bad[w];
    }
    counts[blockIdx.x] = c;
    bad[blockIdx.x] = b;
  }
}

// Block-wide exclusive scan helper for 1024 threads.
__device__ __forceinline__ int block_excl_scan_1024(int v, int* s_w, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) s_w[wave] = x;
  __syncthreads();
  if (wave == 0) {
    int w = lane < 16 ? s_w[lane] : 0;
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) {
      const int y = __shfl_up(w, off);
      if (lane >= off) w += y;
    }
    if (lane < 16) s_w[lane] = w;
  }
  __syncthreads();
  const int excl = x - v + (wave > 0 ? s_w[wave - 1] : 0);
  total = s_w[15];
  __syncthreads();
  return excl;
}

// stat[0] = C, stat[1] = 1 if any supervised label is out of range.
__global__ __launch_bounds__(1024) void k_cmp_scan(const int* __restrict__ counts,
                                                   const int* __restrict__ bad, int nblk,
                                                   int* offsets, int* stat) {
  __shared__ int s_w[16];
  int carry = 0, anybad = 0;
  for (int base = 0; base < nblk; base += 1024) {
    const int j = base + threadIdx.x;
    const int v = j < nblk ? counts[j] : 0;
    const int b = j < nblk ? bad[j] : 0;
    int total;
    const int excl = block_excl_scan_1024(v, s_w, total);
    if (j < nblk) offsets[j] = carry + excl;
    carry += total;
    anybad |= __syncthreads_or(b);
  }
  if (threadIdx.x == 0) {
    stat[0] = carry;
    stat[1] = anybad;
  }
}

// The same compaction in one workgroup, for N <= kCmpOneMax: the block walks
// the positions in rounds of 1024 x kCmpPer (each thread a run of kCmpPer
// consecutive positions), scans the per-thread counts across the block and
// writes each round's supervised positions after the previous rounds'.  One
// launch instead of three, for the sizes where launches dominate.
constexpr int kCmpPer = 8;
constexpr int64_t kCmpOneMax = 65536;
__global__ __launch_bounds__(1024) void k_cmp_one(const int64_t* __restrict__ labels,
                                                  const uint8_t* __restrict__ mask, int64_t N, int64_t V,
                                                  int64_t ignore, int32_t* __restrict__ idx, int* stat) {
  __shared__ int s_w[16];
  int carry = 0, anybad = 0;
  for (int64_t base = 0; base < N; base += 1024 * kCmpPer) {
    const int64_t i0 = base + (int64_t)threadIdx.x * kCmpPer;
    uint32_t bits = 0;
    int cnt = 0;
    bool oob = false;
#pragma unroll
    for (int k = 0; k < kCmpPer; ++k) {
      const int64_t i = i0 + k;
      if (i < N && is_supervised(labels, mask, i, ignore)) {
        bits |= 1u << k;
        ++cnt;
        const int64_t y = labels[i];
        oob = oob || y < 0 || y >= V;
      }
    }
    int total;
    int o = carry + block_excl_scan_1024(cnt, s_w, total);
#pragma unroll
    for (int k = 0; k < kCmpPer; ++k)
      if ((bits >> k) & 1u) idx[o++] = (int32_t)(i0 + k);
    carry += total;
    anybad |= __syncthreads_or(oob);
  }
  if (threadIdx.x == 0) {
    stat[0] = carry;
    stat[1] = anybad;
  }
}

__global__ __launch_bounds__(kCmpBlock) void k_cmp_scatter(const int64_t* __restrict__ labels,
                                                           const uint8_t* __restrict__ mask,
                                                           int64_t N, int64_t ignore,
                                                           const int* __restrict__ offsets,
                                                           int32_t* __restrict__ idx) {
  __shared__ int s_cnt[kCmpBlock / kWarp];
  const int64_t i = (int64_t)blockIdx.x * kCmpBlock + threadIdx.x;
  const bool sup = i < N && is_supervised(labels, mask, i, ignore);
  const uint64_t bal = __ballot(sup);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) s_cnt[wave] = __popcll(bal);
  __syncthreads();
  int off = offsets[blockIdx.x];
  for (int w = 0; w < wave; ++w) off += s_cnt[w];
  const uint64_t below = lane == 0 ? 0ull : (bal & ((~0ull) >> (64 - lane)));
  if (sup) idx[off + __popcll(below)] = (int32_t)i;
}

// ============================================================== K1 gather
// Hc[c] = H[idx[c]] for c < C, 0 for C <= c < Cpad; yc[c] = y[idx[c]] (-1 for
// padding).  With m/logs given (backward), mc/lsc hold them per compact row;
// padding rows get m = +inf so their replayed p is 0.
// The same launch fills the per-position arrays that later kernels write at
// the supervised positions only (each optional, N entries): the forward's
// m = log s = -inf (the recurrence's initial state) and l = 0, the
// backward's inverse map inv = -1.
struct PosFill {
  float* m = nullptr;
  float* logs = nullptr;
  float* row_loss = nullptr;
  int* inv = nullptr;
  int64_t N = 0;
};
template <typename T>
__global__ __launch_bounds__(256) void k_gather(const T* __restrict__ H,
                                                const int64_t* __restrict__ labels,
                                                const int32_t* __restrict__ idx, int C, int Cpad,
                                                int D, int64_t label_off, T* __restrict__ Hc, int* __restrict__ yc,
                                                const float* __restrict__ m,
                                                const float* __restrict__ logs, float* mc,
                                                float* lsc, PosFill fill) {
  for (int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; n < fill.N;
       n += (int64_t)gridDim.x * blockDim.x) {
    if (fill.m) fill.m[n] = -INFINITY;
    if (fill.logs) fill.logs[n] = -INFINITY;
    if (fill.row_loss) fill.row_loss[n] = 0.f;
    if (fill.inv) fill.inv[n] = -1;
  }
  constexpr int VEC = 16 / sizeof(T);
  const int vpr = D / VEC;
  const int64_t total = (int64_t)Cpad * vpr;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total;
       q += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(q / vpr), kv = (int)(q % vpr);
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    int src = -1;
    if (c < C) {
      src = idx[c];
      v = *reinterpret_cast<const u32x4*>(H + (int64_t)src * D + kv * VEC);
    }
    *reinterpret_cast<u32x4*>(Hc + (int64_t)c * D + kv * VEC) = v;
    if (kv == 0) {
      // Labels relative to the first vocabulary row of W (a vocabulary shard
      // starts at label_off); a label outside [0, V) of that W matches no column.
      yc[c] = -1;
      if (c < C) {
        const int64_t yl = labels[src] - label_off;
        yc[c] = (yl >= 0 && yl < INT32_MAX) ? (int)yl : -1;
      }
      if (mc) {
        mc[c] = c < C ? m[src] : INFINITY;
        lsc[c] = c < C ? logs[src] : 0.f;
      }
    }
  }
}

// ============================================================== K2 forward
// Work item = (row block rb, vocabulary split).  The workgroup walks the
// split's vocabulary tiles in order; for each tile it forms the score tile
// Z^T = W_B . Hc_T^T (+ b) with MFMA (FORWARD/PROJECT, section 01), then
// updates each row's running max and exp-sum (REDUCE/CAPTURE, section 02
// recurrence) and captures Z_{i,y_i} from the tile holding y_i by global
// column id.  The vocabulary is the MFMA M axis, so a lane's 64 scores of a
// row lie in its own registers and the tile needs no cross-lane reduction;
// lanes merge once per split.  Output: partial (m, s) per (split, row).
// The LDS bias slice arrives in whole dwords, so where V ends inside one the
// last values are zero: the ragged last tile rewrites its slice element by
// element (all waves reach this for the same tile).
__device__ __noinline__ void refill_bias_slice(const uint16_t* slice, const uint16_t* __restrict__ bias, int m0,
                                               int V) {
  uint16_t* s = const_cast<uint16_t*>(slice);
  if (threadIdx.x < 256) s[threadIdx.x] = (m0 + (int)threadIdx.x < V) ? bias[m0 + threadIdx.x] : (uint16_t)0;
  pipe::wait_lgkm0();
  pipe::raw_barrier();
}

// Adds b_v from the tile's LDS bias slice (bf16 pipeline).
__device__ __forceinline__ void add_bias_lds(f32x16_t (&acc)[Geo<uint16_t>::TM][Geo<uint16_t>::TN],
                                             const uint16_t* slice, int vloc0, int lane) {
  using G = Geo<uint16_t>;
#pragma unroll
  for (int tm = 0; tm < G::TM; ++tm)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int j = vloc0 + tm * 32 + 8 * i4 + 4 * (lane >> 5);
      const u32x2 w = *reinterpret_cast<const u32x2*>(slice + j);
      const float bv[4] = {to_f32((uint16_t)(w[0] & 0xFFFFu)), to_f32((uint16_t)(w[0] >> 16)),
                           to_f32((uint16_t)(w[1] & 0xFFFFu)), to_f32((uint16_t)(w[1] >> 16))};
#pragma unroll
      for (int tn = 0; tn < G::TN; ++tn)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[tm][tn][i4 * 4 + r] += bv[r];
    }
}

// Adds b_v to every score of the tile after the K loop (one rounding, so a
// large bias does not coarsen the fp32 partial sums of H.W).
template <typename T>
__device__ __forceinline__ void add_bias(f32x16_t (&acc)[Geo<T>::TM][Geo<T>::TN],
                                         const T* __restrict__ bias, int vbase, int V, int lane) {
  using G = Geo<T>;
#pragma unroll
  for (int tm = 0; tm < G::TM; ++tm)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int v = vbase + tm * 32 + 8 * i4 + 4 * (lane >> 5);
      float bv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) bv[r] = (v + r < V) ? to_f32(bias[v + r]) : 0.f;
#pragma unroll
      for (int tn = 0; tn < G::TN; ++tn)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[tm][tn][i4 * 4 + r] += bv[r];
    }
}

// Per-tile forward epilogue: bias, ragged-column mask, running (m, s) update
// and target capture for the TN rows a lane holds.
template <typename T>
__device__ __forceinline__ void fwd_epilogue(f32x16_t (&acc)[Geo<T>::TM][Geo<T>::TN],
                                             const T* __restrict__ bias, int m0, int V, const int (&row)[Geo<T>::TN],
                                             const int (&y)[Geo<T>::TN], float (&mrun)[Geo<T>::TN],
                                             float (&srun)[Geo<T>::TN], float* __restrict__ tgt,
                                             int wm, int lane, const uint16_t* bias_slice = nullptr) {
  using C = Cfg<T>;
  using G = Geo<T>;
  const int vbase = m0 + wm * G::WTM;
  if constexpr (sizeof(T) == 2) {
    if (bias) {
      if (m0 + C::BM > V) refill_bias_slice(bias_slice, reinterpret_cast<const uint16_t*>(bias), m0, V);
      add_bias_lds(acc, bias_slice, wm * G::WTM, lane);
    }
  } else {
    if (bias) add_bias<T>(acc, bias, vbase, V, lane);
  }
  if (m0 + C::BM > V) {  // ragged last tile: columns past V do not exist
#pragma unroll
    for (int tm = 0; tm < G::TM; ++tm)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (vbase + acc_row(tm, i, lane) >= V)
#pragma unroll
          for (int tn = 0; tn < G::TN; ++tn) acc[tm][tn][i] = -INFINITY;
  }
#pragma unroll
  for (int tn = 0; tn < G::TN; ++tn) {
    float mloc = -INFINITY;
#pragma unroll
    for (int tm = 0; tm < G::TM; ++tm)
#pragma unroll
      for (int i = 0; i < 16; ++i) mloc = fmaxf(mloc, acc[tm][tn][i]);
    const float mnew = fmaxf(mrun[tn], mloc);
    const float mref = (mnew == -INFINITY) ? 0.f : mnew;
    float ssum = 0.f;
    if constexpr (sizeof(T) == 4) {
      // fp32: Z - m is exact for nearby values, so a large common shift
      // costs no precision (section 02: compute relative to m).
#pragma unroll
      for (int tm = 0; tm < G::TM; ++tm)
#pragma unroll
        for (int i = 0; i < 16; ++i) ssum += __builtin_amdgcn_exp2f((acc[tm][tn][i] - mref) * kLog2e);
    } else {
      const float mneg = -mref * kLog2e;
#pragma unroll
      for (int tm = 0; tm < G::TM; ++tm)
#pragma unroll
        for (int i = 0; i < 16; ++i) ssum += __builtin_amdgcn_exp2f(fmaf(acc[tm][tn][i], kLog2e, mneg));
    }
    // First tile: the rescale factor of the (empty) old sum is 0.
    const float alpha = (mnew == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f((mrun[tn] - mnew) * kLog2e);
    srun[tn] = srun[tn] * alpha + ssum;
    mrun[tn] = mnew;
    // Target capture by global column id.
    const int d = y[tn] - vbase;
    if ((unsigned)d < (unsigned)G::WTM) {
#pragma unroll
      for (int tm = 0; tm < G::TM; ++tm)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (acc_row(tm, i, lane) == d) tgt[row[tn]] = acc[tm][tn][i];
    }
  }
}

template <typename T, bool HAS_BIAS>
__global__ __launch_bounds__(kThreads) void k_fwd(const T* __restrict__ W, const T* __restrict__ bias_arg,
                                                  const T* __restrict__ Hc,
                                                  const int* __restrict__ yc, int Cpad, int D, int V,
                                                  int n_rb, int n_split, int n_vt, int n_work,
                                                  int per_xcd, float* __restrict__ pm,
                                                  float* __restrict__ ps, float* __restrict__ tgt) {
  using C = Cfg<T>;
  using G = Geo<T>;
  extern __shared__ __align__(16) char smem_raw[];
  // Without a bias the instantiation carries no bias state through the tile loop.
  const T* __restrict__ bias = HAS_BIAS ? bias_arg : nullptr;
  const int w = xcd_remap(blockIdx.x, per_xcd);
  if (w >= n_work) return;
  int rb, split;
  grouped_index<kGroupRows>(w, n_rb, n_split, rb, split);
  const int t0 = (int)((int64_t)split * n_vt / n_split);
  const int t1 = (int)((int64_t)(split + 1) * n_vt / n_split);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave % G::WGM, wn = wave / G::WGM;
  const int n0 = rb * C::BN;

  int row[G::TN], y[G::TN];
  float mrun[G::TN], srun[G::TN];
#pragma unroll
  for (int tn = 0; tn < G::TN; ++tn) {
    row[tn] = n0 + wn * G::WTN + tn * 32 + (lane & 31);
    y[tn] = yc[row[tn]];
    mrun[tn] = -INFINITY;
    srun[tn] = 0.f;
  }
  // Stages per tile: BK = 64 in the bf16 pipeline, Cfg<T>::BK in the fp32 loop.
  const int nsteps = sizeof(T) == 2 ? (D + pipe::BK - 1) / pipe::BK : (D + C::BK - 1) / C::BK;
  float* red;
  if constexpr (sizeof(T) == 2) {
    f32x16_t acc[G::TM][G::TN];
    pipe::run<0, true, 0, HAS_BIAS>(
        t1 - t0, nsteps, D, smem_raw, acc,
        [&](int t, pipe::Opnd& A, pipe::Opnd& B, int& k0) {
          A = pipe::Opnd{W, (int64_t)V * D, D, (t0 + t) * C::BM};
          B = pipe::Opnd{Hc, (int64_t)Cpad * D, D, n0};
          k0 = 0;
        },
        [&](int t, f32x16_t (&acc)[G::TM][G::TN]) {
          fwd_epilogue<T>(acc, bias, (t0 + t) * C::BM, V, row, y, mrun, srun, tgt, wm, lane,
                          pipe::bias_slice(smem_raw, t));
        },
        true, reinterpret_cast<const uint16_t*>(bias), V);
    red = reinterpret_cast<float*>(smem_raw + pipe::RING_BYTES);
  } else {
    T* smem = reinterpret_cast<T*>(smem_raw);
    for (int t = t0; t < t1; ++t) {
      f32x16_t acc[G::TM][G::TN];
      zero_acc<T>(acc);
      gemm_tile<T, true, true>(W, (int64_t)V * D, D, t * C::BM, Hc, (int64_t)Cpad * D, D, n0, 0, D,
                               nsteps, acc, smem);
      fwd_epilogue<T>(acc, bias, t * C::BM, V, row, y, mrun, srun, tgt, wm, lane);
    }
    red = reinterpret_cast<float*>(smem_raw);  // free: gemm_tile ends on a barrier
  }

  // Lanes l and l^32 hold the same rows (different vocabulary entries).
#pragma unroll
  for (int tn = 0; tn < G::TN; ++tn) {
    const float mo = __shfl_xor(mrun[tn], 32);
    const float so = __shfl_xor(srun[tn], 32);
    lse_merge(mrun[tn], srun[tn], mo, so);
  }
  // Waves with the same wn and different wm hold the same rows.
  static_assert(G::WGM == 2, "merge below assumes two waves per row range");
  if (wm == 1 && lane < 32) {
#pragma unroll
    for (int tn = 0; tn < G::TN; ++tn) {
      red[((wn * G::TN + tn) * 32 + lane) * 2 + 0] = mrun[tn];
      red[((wn * G::TN + tn) * 32 + lane) * 2 + 1] = srun[tn];
    }
  }
  __syncthreads();
  if (wm == 0 && lane < 32) {
#pragma unroll
    for (int tn = 0; tn < G::TN; ++tn) {
      const float mo = red[((wn * G::TN + tn) * 32 + lane) * 2 + 0];
      const float so = red[((wn * G::TN + tn) * 32 + lane) * 2 + 1];
      lse_merge(mrun[tn], srun[tn], mo, so);
      pm[(int64_t)split * Cpad + row[tn]] = mrun[tn];
      ps[(int64_t)split * Cpad + row[tn]] = srun[tn];
    }
  }
}

// Dynamic LDS bytes of the GEMM kernels for element type T.
template <typename T> constexpr int gemm_lds_bytes() {
  return sizeof(T) == 2 ? pipe::LDS_BYTES : Geo<T>::LDS_BYTES;
}
// The bf16 replay keeps its rows' constants after the pipeline's bytes
// (16 B per row), and the filtered replay one vote word per wave after them.
constexpr int kRowStatOffset = pipe::LDS_BYTES, kRowStatBytes = 256 * 16;
constexpr int kVoteOffset = kRowStatOffset + kRowStatBytes, kVoteBytes = pipe::NWAVES * 4;
template <typename T, bool FILTER> constexpr int replay_lds_bytes() {
  return sizeof(T) == 2 ? kVoteOffset + (FILTER ? kVoteBytes : 0) : gemm_lds_bytes<T>();
}
static_assert(kVoteOffset + kVoteBytes <= 160 * 1024, "LDS of one workgroup per CU");

// ============================================================== K3 merge + loss
// Per supervised row: merge the split partials in split order (online-softmax
// merge), log s, l_i = (m - Z_{i,y_i}) + log s (section 02), scatter m, log s
// (and the row CE) to the row's position.
__global__ __launch_bounds__(256) void k_merge(const float* __restrict__ pm, const float* __restrict__ ps,
                                               const float* __restrict__ tgt, int n_split, int Cpad,
                                               int C, const int32_t* __restrict__ idx,
                                               float* __restrict__ m_out, float* __restrict__ logs_out,
                                               float* __restrict__ row_loss, float* __restrict__ lrow) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= C) return;
  float m = -INFINITY, s = 0.f;
  for (int k = 0; k < n_split; ++k) lse_merge(m, s, pm[(int64_t)k * Cpad + c], ps[(int64_t)k * Cpad + c]);
  const float ls = logf(s);
  const float l = (m - tgt[c]) + ls;
  const int n = idx[c];
  if (m_out) m_out[n] = m;
  if (logs_out) logs_out[n] = ls;
  if (row_loss) row_loss[n] = l;
  lrow[c] = l;
}

// Vocabulary shard (the partials one tensor-parallel rank would send): per
// supervised row, the split partials of this shard merged in split order
// into (m, s), and the target score when the row's label falls in the shard
// (0 otherwise; the cross-shard merge reads it only from the owning shard).
__global__ __launch_bounds__(256) void k_shard_partial(const float* __restrict__ pm, const float* __restrict__ ps,
                                                       const float* __restrict__ tgt, int n_split, int Cpad, int C,
                                                       const int* __restrict__ yc, int Vs, float* __restrict__ out_m,
                                                       float* __restrict__ out_s, float* __restrict__ out_t) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= C) return;
  float m = -INFINITY, s = 0.f;
  for (int k = 0; k < n_split; ++k) lse_merge(m, s, pm[(int64_t)k * Cpad + c], ps[(int64_t)k * Cpad + c]);
  out_m[c] = m;
  out_s[c] = s;
  out_t[c] = ((unsigned)yc[c] < (unsigned)Vs) ? tgt[c] : 0.f;
}

// Shard boundaries (vocabulary starts of P shards, then V): a kernel argument.
constexpr int kMaxShards = 64;
struct ShardBounds {
  int64_t b[kMaxShards + 1];
};

// Cross-shard merge (the exchange step of vocabulary sharding): per supervised
// row, the P shard partials merged in shard order (section 02 recurrence),
// the target score taken from the shard holding y_i, l_i = (m - z_y) + log s;
// m, log s and l scattered to the row's position as in k_merge.
__global__ __launch_bounds__(256) void k_merge_shards(const float* __restrict__ part_m,
                                                      const float* __restrict__ part_s,
                                                      const float* __restrict__ part_t, int P, int64_t ld,
                                                      ShardBounds bounds, const int64_t* __restrict__ labels,
                                                      const int32_t* __restrict__ idx, int C,
                                                      float* __restrict__ m_out, float* __restrict__ logs_out,
                                                      float* __restrict__ row_loss, float* __restrict__ lrow) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= C) return;
  float m = -INFINITY, s = 0.f;
  for (int p = 0; p < P; ++p) lse_merge(m, s, part_m[(int64_t)p * ld + c], part_s[(int64_t)p * ld + c]);
  const int n = idx[c];
  const int64_t y = labels[n];
  int owner = 0;
  for (int p = 0; p < P; ++p)
    if (y >= bounds.b[p] && y < bounds.b[p + 1]) owner = p;
  const float ls = logf(s);
  const float l = (m - part_t[(int64_t)owner * ld + c]) + ls;
  if (m_out) m_out[n] = m;
  if (logs_out) logs_out[n] = ls;
  if (row_loss) row_loss[n] = l;
  lrow[c] = l;
}

// Reductions of the per-row CE (NeMo chunked_ce page, ChunkedCrossEntropy.forward:
// mean over the supervised rows, or a sum with optional per-position weights
// divided by an external token count), summed in float64 in a fixed order:
//   mean: loss = (1/C) sum_c l_c
//   sum:  loss = (sum_c w_{idx_c} l_c) / div     (w = 1 without weights)
constexpr int kReduceMean = 0, kReduceSum = 1, kReduceNone = 2;

__global__ __launch_bounds__(1024) void k_loss_sum(const float* __restrict__ lrow, int C,
                                                   int reduction, const float* __restrict__ weights,
                                                   const int32_t* __restrict__ idx, double div,
                                                   float* __restrict__ loss) {
  __shared__ double s[1024];
  double acc = 0.0;
  for (int c = threadIdx.x; c < C; c += 1024)
    acc += weights ? (double)weights[idx[c]] * (double)lrow[c] : (double)lrow[c];
  s[threadIdx.x] = acc;
  __syncthreads();
  for (int off = 512; off > 0; off >>= 1) {
    if (threadIdx.x < off) s[threadIdx.x] += s[threadIdx.x + off];
    __syncthreads();
  }
  if (threadIdx.x == 0) loss[0] = (float)(reduction == kReduceMean ? s[0] / (double)C : s[0] / div);
}

// r_c, the factor of row c's (p - onehot) in G (section 04: lambda a_i / C for
// the mean; the derivative of the chosen reduction otherwise):
//   mean: lambda / C;  sum: lambda w_{idx_c} / div;  none: g_{idx_c} (per-row
//   upstream gradient).  lambda = grad[0] (1 without grad).  Padding rows: 0.
// The same launch completes the inverse map, inv[idx[c]] = c (the gather
// set every entry to -1 before).
__global__ void k_row_scale(const int32_t* __restrict__ idx, int C, int Cpad, int reduction,
                            const float* __restrict__ weights, float div, const float* __restrict__ grad,
                            float* __restrict__ rsc, int* __restrict__ inv) {
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (c >= Cpad) return;
  float r = 0.f;
  if (c < C) {
    const int n = idx[c];
    inv[n] = c;
    if (reduction == kReduceNone) {
      r = grad ? grad[n] : 1.f;
    } else {
      const float lam = grad ? grad[0] : 1.f;
      r = reduction == kReduceMean ? lam / (float)C : lam * (weights ? weights[n] : 1.f) / div;
    }
  }
  rsc[c] = r;
}

// m = log s = -inf and l = 0 at every position (each array optional).
__global__ void k_fill_stats(float* __restrict__ m, float* __restrict__ logs, float* __restrict__ row_loss,
                             int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    if (m) m[i] = -INFINITY;
    if (logs) logs[i] = -INFINITY;
    if (row_loss) row_loss[i] = 0.f;
  }
}
// Zero n16 16-byte words (plus a byte tail).
__global__ void k_zero(u32x4* __restrict__ p, int64_t n16, uint8_t* __restrict__ tail, int ntail) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = u32x4{0u, 0u, 0u, 0u};
  if (blockIdx.x == 0 && (int)threadIdx.x < ntail) tail[threadIdx.x] = 0;
}
__global__ void k_store_scalar(float* __restrict__ p, float v) { p[0] = v; }

// ============================================================== K4 replay
// Work item = (row block, run of `tpw` vocabulary tiles of this chunk).  For
// each tile: recompute the score tile, p = exp((Z - m) - log s) from the
// saved statistics, subtract 1 at the target column (global id), scale row c
// by its factor r_c (k_row_scale), write G = r_c (p - onehot) into the chunk
// buffer, and, with a bias, the per-row-block column sums of G (db partials)
// in a fixed order.
// FILTER: also mark, per block of 256 rows x 32 vocabulary entries of G, whether
// the block is live for the gradient GEMMs (see grad_body): some entry with
// |r| p >= eps |r| (r != 0), or the block holds a row's target column.
template <typename T, bool FILTER = false>
__device__ __forceinline__ void replay_epilogue(f32x16_t (&acc)[Geo<T>::TM][Geo<T>::TN],
                                                const T* __restrict__ bias, int m0, int n0, int V, int v0,
                                                const int* __restrict__ yc, const float* __restrict__ mc,
                                                const float* __restrict__ lsc, const float* __restrict__ rsc,
                                                T* __restrict__ Gc,
                                                int64_t ldg, float* __restrict__ dbp, int64_t lddb,
                                                int rb, float* red, bool raw_sync,
                                                const uint16_t* bias_slice = nullptr,
                                                uint8_t* __restrict__ flags = nullptr, int64_t fstride = 0,
                                                float eps = 0.f, uint32_t* votes = nullptr,
                                                int zero_dead = 0, const float4* rowstat = nullptr) {
  using C = Cfg<T>;
  using G = Geo<T>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave % G::WGM, wn = wave / G::WGM;
  const int vbase = m0 + wm * G::WTM;
  if constexpr (sizeof(T) == 2) {
    if (bias) {
      if (m0 + C::BM > V) refill_bias_slice(bias_slice, reinterpret_cast<const uint16_t*>(bias), m0, V);
      add_bias_lds(acc, bias_slice, wm * G::WTM, lane);
    }
  } else {
    if (bias) add_bias<T>(acc, bias, vbase, V, lane);
  }
  // bf16: the sign of r_c is applied when G is packed (sign bits of a bf16
  // pair) and in the db sums; the exponent carries |r_c|.
  uint32_t smask[G::TN];
  float sgn[G::TN];
  float absr[G::TN];
  int yrow[G::TN];
#pragma unroll
  for (int tn = 0; tn < G::TN; ++tn) {
    const int r = n0 + wn * G::WTN + tn * 32 + (lane & 31);
    // p = exp((Z - m) - log s) from the saved statistics (section 04).
    float sub;  // r_c at the target column
    if constexpr (sizeof(T) == 4) {
      const float mr = mc[r], lr = lsc[r], rr = rsc[r];
      yrow[tn] = yc[r];
      absr[tn] = fabsf(rr);
#pragma unroll
      for (int tm = 0; tm < G::TM; ++tm)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          acc[tm][tn][i] = rr * __builtin_amdgcn_exp2f(((acc[tm][tn][i] - mr) - lr) * kLog2e);
      sub = rr;
      smask[tn] = 0u;
      sgn[tn] = 1.f;
    } else {
      // |r| p = exp2(Z log2e - c) with c = (m + log s) log2e - log2 |r| (one
      // constant per row, so one FMA per entry); r = 0 gives c = +inf and 0.
      // The row's constants come from LDS (written once per workgroup).
      const float4 st = rowstat[wn * G::WTN + tn * 32 + (lane & 31)];
      const float c = st.x, rr = st.z;
      const float ar = fabsf(rr);
      yrow[tn] = __float_as_int(st.w);
      absr[tn] = ar;
#pragma unroll
      for (int tm = 0; tm < G::TM; ++tm)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          acc[tm][tn][i] = __builtin_amdgcn_exp2f(fmaf(acc[tm][tn][i], kLog2e, -c));
      sub = ar;
      const bool neg = (__float_as_uint(rr) >> 31) != 0u;
      smask[tn] = neg ? 0x80008000u : 0u;
      sgn[tn] = neg ? -1.f : 1.f;
    }
    const int d = yrow[tn] - vbase;
    if ((unsigned)d < (unsigned)G::WTM) {
#pragma unroll
      for (int tm = 0; tm < G::TM; ++tm)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (acc_row(tm, i, lane) == d) acc[tm][tn][i] -= sub;
    }
  }
  if (m0 + C::BM > V) {
#pragma unroll
    for (int tm = 0; tm < G::TM; ++tm)
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (vbase + acc_row(tm, i, lane) >= V)
#pragma unroll
          for (int tn = 0; tn < G::TN; ++tn) acc[tm][tn][i] = 0.f;
  }
  // Filter blocks kept (bit tm: column block tm of this wave).  When dW is
  // filtered too (zero_dead), dead blocks are stored as exact zeros: a dW
  // k-step covers all 8 column blocks of a tile, and must sum the live ones
  // only.  (A dH k-step is exactly one block, so dH needs no zeros.)  The
  // db sums below use the unmasked values.
  uint32_t keep = ~0u;
  if constexpr (FILTER) {
    // Block (row block n0/256, chunk column block (vbase - v0)/32 + tm): its
    // 256 rows lie in the WGN waves with this wm.  Each wave votes on its
    // rows, the votes meet in LDS, and the wn == 0 wave writes the flag (one
    // writer per flag, 0 or 1).  Ragged columns are 0 here.
    float thr[G::TN];  // eps |r|, or +inf for rows with r = 0 (never live)
    int dd[G::TN];
#pragma unroll
    for (int tn = 0; tn < G::TN; ++tn) {
      thr[tn] = absr[tn] > 0.f ? eps * absr[tn] : INFINITY;
      dd[tn] = yrow[tn] - vbase;
    }
    uint32_t mine = 0;
#pragma unroll
    for (int tm = 0; tm < G::TM; ++tm) {
      bool live = false;
#pragma unroll
      for (int tn = 0; tn < G::TN; ++tn) {
        live = live || (unsigned)(dd[tn] - tm * 32) < 32u;
#pragma unroll
        for (int i = 0; i < 16; ++i) live = live || fabsf(acc[tm][tn][i]) >= thr[tn];
      }
      if (__ballot(live) != 0) mine |= 1u << tm;
    }
    if (lane == 0) votes[wave] = mine;
    pipe::wait_lgkm0();
    pipe::raw_barrier();
    uint32_t live = 0;
#pragma unroll
    for (int q = 0; q < G::WGN; ++q) live |= votes[q * G::WGM + wm];
    if (wn == 0 && lane < G::TM)
      flags[(int64_t)(n0 / C::BN) * fstride + (vbase - v0) / 32 + lane] = (uint8_t)((live >> lane) & 1u);
    if (zero_dead) keep = live;
  }
  if constexpr (sizeof(T) == 2) {
    // Store G in the blocked layout (256 x 32 blocks, see gblock_offset).  One
    // (tm, tn) accumulator block is 32 rows c x 32 entries v, i.e. 32 whole
    // 64-byte block rows.  Lane l (l < 32) holds entries {8j..8j+3} of row l,
    // lane l+32 entries {8j+4..8j+7}; one permlane32 swap per register pair
    // leaves lane l with entries 0..15 and lane l+32 with 16..31, each
    // written as 32 contiguous bytes.
    const int h = lane >> 5;
    const int64_t tile = ((int64_t)(n0 / pipe::GB_ROWS) * (ldg / pipe::GB_COLS) + (vbase - v0) / pipe::GB_COLS) *
                         pipe::GB_ELEMS;
    T* gb = Gc + tile + (wn * G::WTN + (lane & 31)) * pipe::GB_COLS + 16 * h;
#pragma unroll
    for (int tn = 0; tn < G::TN; ++tn)
#pragma unroll
      for (int tm = 0; tm < G::TM; ++tm) {
        uint32_t d[8];
        const uint32_t km = ((keep >> tm) & 1u) ? ~0u : 0u;
#pragma unroll
        for (int k = 0; k < 8; ++k)
          d[k] = (pack_bf16x2(acc[tm][tn][2 * k], acc[tm][tn][2 * k + 1]) ^ smask[tn]) & km;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          // lanes 32..63 of d[k] <-> lanes 0..31 of d[k + 4]
          const auto sw = __builtin_amdgcn_permlane32_swap(d[k], d[k + 4], false, false);
          d[k] = sw[0];
          d[k + 4] = sw[1];
        }
        T* dst = gb + tm * pipe::GB_ELEMS + tn * 32 * pipe::GB_COLS;
        *reinterpret_cast<u32x4*>(dst) = u32x4{d[0], d[1], d[4], d[5]};
        *reinterpret_cast<u32x4*>(dst + 8) = u32x4{d[2], d[3], d[6], d[7]};
      }

  } else {
    // Store G row-major (4 consecutive vocabulary entries of one row per lane and group).
#pragma unroll
    for (int tn = 0; tn < G::TN; ++tn) {
      const int r = n0 + wn * G::WTN + tn * 32 + (lane & 31);
      T* grow = Gc + (int64_t)r * ldg + (vbase - v0);
#pragma unroll
      for (int tm = 0; tm < G::TM; ++tm)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
          *reinterpret_cast<f32x4_t*>(grow + tm * 32 + 8 * i4 + 4 * (lane >> 5)) =
              f32x4_t{acc[tm][tn][i4 * 4 + 0], acc[tm][tn][i4 * 4 + 1], acc[tm][tn][i4 * 4 + 2],
                      acc[tm][tn][i4 * 4 + 3]};
    }
  }
  if (dbp == nullptr) return;
  // Column sums over this workgroup's rows: first the TN rows a lane holds,
  // then the 32 lanes of the half-wave (butterfly), then the WGN waves.
  constexpr int NV = G::TM * 16;
  float cs[NV];
#pragma unroll
  for (int tm = 0; tm < G::TM; ++tm)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float sum = 0.f;
#pragma unroll
      for (int tn = 0; tn < G::TN; ++tn) sum = fmaf(sgn[tn], acc[tm][tn][i], sum);
      cs[tm * 16 + i] = sum;
    }
  halfwave_reduce_scatter<NV>(cs, lane);
  constexpr int PER = NV / 32;
  // red[wn][wm][lane][PER]
#pragma unroll
  for (int j = 0; j < PER; ++j) red[((wn * G::WGM + wm) * 64 + lane) * PER + j] = cs[j];
  if (raw_sync) {
    pipe::wait_lgkm0();
    pipe::raw_barrier();
  } else {
    __syncthreads();
  }
  if (wn == 0) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      float sum = red[((0 * G::WGM + wm) * 64 + lane) * PER + j];
#pragma unroll
      for (int q = 1; q < G::WGN; ++q) sum += red[((q * G::WGM + wm) * 64 + lane) * PER + j];
      const int e = (lane & 31) * PER + j;
      const int v = vbase + acc_row(e >> 4, e & 15, lane);
      if (v < V) dbp[(int64_t)rb * lddb + v] = sum;
    }
  }
}

// Arguments of one replay launch over one vocabulary chunk (see replay_body).
template <typename T>
struct ReplayArgs {
  const T* W;
  const T* bias;
  const T* Hc;
  const int* yc;
  const float* mc;
  const float* lsc;
  const float* rsc;
  int Cpad, D, V, v0, vtiles, tpw, n_rb, n_work, per_xcd;
  T* Gc;
  int64_t ldg;
  float* dbp;
  int64_t lddb;
  uint8_t* flags;
  int64_t fstride;
  float eps;
  int zero_dead;
};

// One workgroup's share of a replay launch; bid = its block index within the launch.
template <typename T, bool FILTER, bool HAS_BIAS>
__device__ __forceinline__ void replay_body(
    int bid, const T* __restrict__ W, const T* __restrict__ bias_arg, const T* __restrict__ Hc,
    const int* __restrict__ yc, const float* __restrict__ mc, const float* __restrict__ lsc,
    const float* __restrict__ rsc, int Cpad,
    int D, int V, int v0, int vtiles, int tpw, int n_rb, int n_work, int per_xcd, T* __restrict__ Gc,
    int64_t ldg, float* __restrict__ dbp_arg, int64_t lddb, uint8_t* __restrict__ flags,
    int64_t fstride, float eps, int zero_dead) {
  using C = Cfg<T>;
  using G = Geo<T>;
  extern __shared__ __align__(16) char smem_raw[];
  // HAS_BIAS: a bias to add or db partials to form (either may still be
  // absent); without it the instantiation carries neither through the loop.
  const T* __restrict__ bias = HAS_BIAS ? bias_arg : nullptr;
  float* __restrict__ dbp = HAS_BIAS ? dbp_arg : nullptr;
  const int w = xcd_remap(bid, per_xcd);
  if (w >= n_work) return;
  int rb, vg;
  grouped_index<kGroupRows>(w, n_rb, n_work / n_rb, rb, vg);
  const int vt0 = vg * tpw;
  const int ntiles = min(tpw, vtiles - vt0);
  const int n0 = rb * C::BN;
  // Stages per tile: BK = 64 in the bf16 pipeline, Cfg<T>::BK in the fp32 loop.
  const int nsteps = sizeof(T) == 2 ? (D + pipe::BK - 1) / pipe::BK : (D + C::BK - 1) / C::BK;
  if constexpr (sizeof(T) == 2) {
    float* red = reinterpret_cast<float*>(smem_raw + pipe::RING_BYTES);
    // The workgroup's 256 rows are the same for every tile: their exponent
    // constants (m log2e, log s log2e - log2 |r|), r and label go to LDS once.
    // Loading them in each epilogue would wait on the in-order vector-memory
    // counter behind the next stage's loads.
    float4* rowstat = reinterpret_cast<float4*>(smem_raw + kRowStatOffset);
    if (threadIdx.x < C::BN) {
      const int r = n0 + threadIdx.x;
      const float rr = rsc[r];
      rowstat[threadIdx.x] = float4{fmaf(mc[r], kLog2e, lsc[r] * kLog2e) - log2f(fabsf(rr)), 0.f, rr,
                                    __int_as_float(yc[r])};
    }
    pipe::wait_lgkm0();  // published by the pipeline's first barrier
    f32x16_t acc[G::TM][G::TN];
    // Each wave's epilogue ends with TN*TM*2 G-tile stores (plus, with a
    // bias, the db stores of some waves and, with the filter, the flag stores
    // of some).
    pipe::run<0, true, G::TN * G::TM * 2, HAS_BIAS>(
        ntiles, nsteps, D, smem_raw, acc,
        [&](int t, pipe::Opnd& A, pipe::Opnd& B, int& k0) {
          A = pipe::Opnd{W, (int64_t)V * D, D, v0 + (vt0 + t) * C::BM};
          B = pipe::Opnd{Hc, (int64_t)Cpad * D, D, n0};
          k0 = 0;
        },
        [&](int t, f32x16_t (&acc)[G::TM][G::TN]) {
          replay_epilogue<T, FILTER>(acc, bias, v0 + (vt0 + t) * C::BM, n0, V, v0, yc, mc, lsc, rsc, Gc, ldg, dbp,
                                     lddb, rb, red, true, pipe::bias_slice(smem_raw, t), flags, fstride, eps,
                                     reinterpret_cast<uint32_t*>(smem_raw + kVoteOffset), zero_dead, rowstat);
        },
        true, reinterpret_cast<const uint16_t*>(bias), V);
  } else {
    T* smem = reinterpret_cast<T*>(smem_raw);
    for (int t = 0; t < ntiles; ++t) {
      const int m0 = v0 + (vt0 + t) * C::BM;
      f32x16_t acc[G::TM][G::TN];
      zero_acc<T>(acc);
      gemm_tile<T, true, true>(W, (int64_t)V * D, D, m0, Hc, (int64_t)Cpad * D, D, n0, 0, D, nsteps, acc,
                               smem);
      replay_epilogue<T>(acc, bias, m0, n0, V, v0, yc, mc, lsc, rsc, Gc, ldg, dbp, lddb, rb,
                         reinterpret_cast<float*>(smem_raw), false);
      __syncthreads();  // the next tile's loads reuse the LDS the db sums used
    }
  }
}

template <typename T, bool FILTER, bool HAS_BIAS>
__device__ __forceinline__ void replay_body(int bid, const ReplayArgs<T>& a) {
  replay_body<T, FILTER, HAS_BIAS>(bid, a.W, a.bias, a.Hc, a.yc, a.mc, a.lsc, a.rsc, a.Cpad, a.D, a.V, a.v0,
                                   a.vtiles, a.tpw, a.n_rb, a.n_work, a.per_xcd, a.Gc, a.ldg, a.dbp, a.lddb,
                                   a.flags, a.fstride, a.eps, a.zero_dead);
}

template <typename T, bool FILTER, bool HAS_BIAS>
__global__ __launch_bounds__(kThreads) void k_replay(ReplayArgs<T> a) {
  replay_body<T, FILTER, HAS_BIAS>((int)blockIdx.x, a);
}

// Stage lists of the gradient filter live in LDS after the pipeline's bytes.
constexpr int kFilterListCap = 3584;  // entries (14 KB) + 8 wave sums
constexpr int kFilterLdsBytes = (kFilterListCap + 8) * 4;
// The gradient items' dynamic LDS: the BK=32 ring (the BK=64 core fits in it),
// plus the filter's stage list (bf16).
template <typename T> constexpr int grad_lds_bytes() {
  return sizeof(T) == 2 ? pipe32::LDS_BYTES + kFilterLdsBytes : Geo<T>::LDS_BYTES;
}
static_assert(pipe32::LDS_BYTES + kFilterLdsBytes <= 160 * 1024, "LDS of one workgroup per CU");
static_assert(pipe::RING_BYTES <= pipe32::LDS_BYTES, "the BK=64 gradient core uses the same LDS");

// Compacts {i < n : live(i)} in ascending order into list, each i expanded
// to `expand` consecutive stages i*expand + 0..expand-1; returns the number
// of stages, or -1 (list untouched beyond capacity: run every stage) if they
// would not fit.  All threads of the workgroup call it (it synchronises).
template <typename Live>
__device__ int build_live_list(int n, Live live, int* list, int* wsum, int expand) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int total = 0;
  bool overflow = false;
  for (int base = 0; base < n; base += kThreads) {
    const int i = base + (int)threadIdx.x;
    const bool f = i < n && live(i);
    const unsigned long long mask = __ballot(f);
    const int rank = __popcll(mask & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[wave] = __popcll(mask);
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int q = 0; q < kThreads / 64; ++q) {
      off += q < wave ? wsum[q] : 0;
      tot += wsum[q];
    }
    if (f) {
      const int pos = (total + off + rank) * expand;
      if (pos + expand <= kFilterListCap)
        for (int e = 0; e < expand; ++e) list[pos + e] = i * expand + e;
    }
    total += tot;
    overflow = overflow || total * expand > kFilterListCap;
    __syncthreads();
  }
  return overflow ? -1 : total * expand;
}

// ============================================================== K5 gradients
// One launch per vocabulary chunk, two kinds of output tiles:
//  * dH tiles (first n_dh blocks): slot[ks][c][d] (+)= sum_{v in split ks}
//    G[c][v] W[v0+v][d]  (dH_T += G_{T,B} W_B, section 04).  The chunk's
//    vocabulary range is cut into S splits; slot ks accumulates split ks of
//    every chunk in chunk order (stream order), so the sum is deterministic.
//  * dW tiles: dW[v0+v][d] = sum_c G[c][v] Hc[c][d]
//    (dW_B += G^T H_T summed over every row block inside one tile, so each dW
//    row is written exactly once).  G already carries the row factors r_c.
// Operands: G is K-contiguous for dH (k = v) and K-outer for dW (k = c); W
// (k = v) and Hc (k = c) are K-outer (read with transposing LDS reads).
template <typename T>
__device__ __forceinline__ void grad_store(const f32x16_t (&acc)[Geo<T>::TM][Geo<T>::TN], bool dh, int m0,
                                           int n0, int D, int vc, int v0, float* slot, int accumulate,
                                           T* __restrict__ dW) {
  using G = Geo<T>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave % G::WGM, wn = wave / G::WGM;
#pragma unroll
  for (int tn = 0; tn < G::TN; ++tn) {
    const int n = n0 + wn * G::WTN + tn * 32 + (lane & 31);
    if (n >= D) continue;
#pragma unroll
    for (int tm = 0; tm < G::TM; ++tm) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = m0 + wm * G::WTM + acc_row(tm, i, lane);
        const float a = acc[tm][tn][i];
        if (dh) {
          // A slot element has one owner per launch and launches run in
          // chunk order, so the L2 atomic add (no return) sums exactly what a
          // load-add-store would, without the wave waiting for the load.
          float* p = slot + (int64_t)r * D + n;
          if (accumulate) (void)__hip_atomic_fetch_add(p, a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          else *p = a;
        } else if (r < vc) {
          dW[(int64_t)(v0 + r) * D + n] = from_f32<T>(a);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// Arguments of one gradient launch over one vocabulary chunk (see grad_body).
template <typename T>
struct GradArgs {
  const T* Gc;
  int64_t ldg;
  int kpad_g;
  const T* Hc;
  const T* W;
  int Cpad, D, v0, vc, w_rows, n_nt, n_dh_mt, ks_len, n_dh, n_dw_mt, dh_first;
  float* slots;
  int64_t slot_stride;
  int accumulate;
  T* dW;
  const uint8_t* flags;
  int64_t fstride;
  int fmask;
};

// One workgroup's share of a gradient launch; bid = its block index within
// the launch (its low 3 bits name the XCD the block runs on).
template <typename T>
__device__ __forceinline__ void grad_body(
    int bid, const T* __restrict__ Gc, int64_t ldg, int kpad_g, const T* __restrict__ Hc,
    const T* __restrict__ W, int Cpad, int D, int v0, int vc, int w_rows, int n_nt, int n_dh_mt, int ks_len,
    int n_dh, int n_dw_mt, int dh_first, float* __restrict__ slots, int64_t slot_stride,
    int accumulate, T* __restrict__ dW, const uint8_t* __restrict__ flags, int64_t fstride, int fmask) {
  using C = Cfg<T>;
  using G = Geo<T>;
  extern __shared__ __align__(16) char smem_raw[];
  // Workgroups go to the 8 XCDs round-robin.  Each XCD takes an equal share of
  // the dH items and of the dW items (their K differ), the longer kind first,
  // so that every XCD finishes at about the same time.  Within a share the
  // n_nt column tiles that share an A block are consecutive, so they run
  // together and read that block through the XCD's L2.
  const int n_dw = n_dw_mt * n_nt;
  int b;
  {
    const int x = bid & 7, j = bid >> 3;
    const int dh_lo = (int)((int64_t)x * n_dh / 8), dh_cnt = (int)((int64_t)(x + 1) * n_dh / 8) - dh_lo;
    const int dw_lo = (int)((int64_t)x * n_dw / 8), dw_cnt = (int)((int64_t)(x + 1) * n_dw / 8) - dw_lo;
    if (dh_first)
      b = j < dh_cnt ? dh_lo + j : (j - dh_cnt < dw_cnt ? n_dh + dw_lo + (j - dh_cnt) : -1);
    else
      b = j < dw_cnt ? n_dh + dw_lo + j : (j - dw_cnt < dh_cnt ? dh_lo + (j - dw_cnt) : -1);
  }
  if (b < 0) return;
  const bool dh = b < n_dh;
  int m0, n0, kb, nsteps;
  float* slot = nullptr;
  if (dh) {
    const int nt = b % n_nt;
    const int q = b / n_nt;
    const int mt = q % n_dh_mt, ks = q / n_dh_mt;
    m0 = mt * C::BM;
    n0 = nt * C::BN;
    kb = ks * ks_len;
    const int ke = min(kb + ks_len, kpad_g);
    nsteps = (ke - kb + C::BK - 1) / C::BK;
    slot = slots + (int64_t)ks * slot_stride;
  } else {
    const int q = b - n_dh;
    const int nt = q % n_nt, mt = q / n_nt;
    m0 = mt * C::BM;
    n0 = nt * C::BN;
    kb = 0;
    nsteps = Cpad / C::BK;
  }
  if constexpr (sizeof(T) == 2) {
    // dH_T += G_T,B W_B: A = G (k = v contiguous), B = W rows (k-outer).
    // dW_B = G^T Hc: A = G (k = c outer), B = Hc (k-outer).
    f32x16_t acc[G::TM][G::TN];
    // G is stored blocked (gblock_offset with ldg/32 blocks per row block).
    const int64_t nvb = ldg / pipe::GB_COLS;
    auto origin = [&](int, pipe::Opnd& A, pipe::Opnd& B, int& k0) {
      if (dh)  // rows c of one 256-row block, k = v: 32 x 256 blocks along k
        A = pipe::Opnd{Gc + (int64_t)(m0 / pipe::GB_ROWS) * nvb * pipe::GB_ELEMS,
                       (int64_t)Cpad * ldg - (int64_t)(m0 / pipe::GB_ROWS) * nvb * pipe::GB_ELEMS, pipe::GB_COLS, 0,
                       pipe::GB_ELEMS / pipe::GB_COLS, 0};
      else     // rows v, k = c: the blocked layout read transposed
        A = pipe::Opnd{Gc, (int64_t)Cpad * ldg, ldg, m0, 1, nvb * pipe::GB_ELEMS};
      B = dh ? pipe::Opnd{W + (int64_t)v0 * D, (int64_t)w_rows * D, D, n0}
             : pipe::Opnd{Hc, (int64_t)Cpad * D, D, n0};
      k0 = kb;
    };
    auto no_epi = [](int, f32x16_t (&)[G::TM][G::TN]) {};
    const int kend = nsteps * C::BK;
    const int* kmap = nullptr;
    if (flags != nullptr && (fmask & (dh ? 1 : 2)) != 0) {
      // Gradient filtering (fmask bit 0: dH items, bit 1: dW items): run only
      // the stages whose G blocks are live.
      // dH tile: stage s is G block (row block m0/256, column block kb/32 + s).
      // dW tile: the 8 stages of row block q cover G blocks (q, m0/32 + 0..7).
      int* list = reinterpret_cast<int*>(smem_raw + pipe32::LDS_BYTES);
      int* wsum = list + kFilterListCap;
      const uint8_t* frow = flags + (int64_t)(m0 / C::BM) * fstride;
      int n_live;
      if (dh)
        n_live = build_live_list(nsteps, [&](int st) { return frow[kb / C::BK + st] != 0; }, list, wsum, 1);
      else
        n_live = build_live_list(Cpad / C::BN, [&](int q) {
          const uint32_t* f = reinterpret_cast<const uint32_t*>(flags + (int64_t)q * fstride + m0 / C::BK);
          return (f[0] | f[1]) != 0u;
        }, list, wsum, C::BN / C::BK);
      if (n_live >= 0) {
        nsteps = n_live;
        kmap = list;
      }
      if (nsteps == 0) pipe32::zero(acc);
    }
    if (kmap != nullptr) {
      // Filtered: the stage lists skip single 32-wide k steps.
      if (dh)
        pipe32::run<0, false>(1, nsteps, kend, smem_raw, acc, origin, no_epi, true, kmap);
      else
        pipe32::run<1, false>(1, nsteps, kend, smem_raw, acc, origin, no_epi, true, kmap);
    } else {
      // BK = 64 stages (half the barriers); a split whose length is an odd
      // multiple of 32 ends in a half stage whose K-contiguous G part reads
      // zeros past kend, so its other half contributes nothing.
      const int nsteps64 = (nsteps + 1) / 2;
      if (dh)
        pipe::run_ko<0, false>(1, nsteps64, kend, smem_raw, acc, origin, no_epi);
      else
        pipe::run_ko<1, false>(1, nsteps64, kend, smem_raw, acc, origin, no_epi);
    }
    grad_store<T>(acc, dh, m0, n0, D, vc, v0, slot, accumulate, dW);
  } else {
    T* smem = reinterpret_cast<T*>(smem_raw);
    f32x16_t acc[G::TM][G::TN];
    zero_acc<T>(acc);
    if (dh) {
      if (nsteps > 0)
        gemm_tile<T, true, false>(Gc, (int64_t)Cpad * ldg, ldg, m0, W + (int64_t)v0 * D, (int64_t)w_rows * D,
                                  D, n0, kb, kb + nsteps * C::BK, nsteps, acc, smem);
    } else {
      gemm_tile<T, false, false>(Gc, (int64_t)Cpad * ldg, ldg, m0, Hc, (int64_t)Cpad * D, D, n0, 0, Cpad,
                                 nsteps, acc, smem);
    }
    grad_store<T>(acc, dh, m0, n0, D, vc, v0, slot, accumulate, dW);
  }
}

template <typename T>
__device__ __forceinline__ void grad_body(int bid, const GradArgs<T>& a) {
  grad_body<T>(bid, a.Gc, a.ldg, a.kpad_g, a.Hc, a.W, a.Cpad, a.D, a.v0, a.vc, a.w_rows, a.n_nt, a.n_dh_mt,
               a.ks_len, a.n_dh, a.n_dw_mt, a.dh_first, a.slots, a.slot_stride, a.accumulate, a.dW, a.flags,
               a.fstride, a.fmask);
}

template <typename T>
__global__ __launch_bounds__(kThreads) void k_grad(GradArgs<T> a) {
  grad_body<T>((int)blockIdx.x, a);
}

// K5 of chunk c and K4 of chunk c+1 in one launch: blocks [0, n_grad) run the
// gradient tiles of chunk c, which read one G buffer; the blocks after them
// replay chunk c+1 into the other buffer.  Blocks start in index order, so
// the replay tiles fill the CUs that the gradient tiles' last wave leaves
// free.  n_grad is a multiple of 8, so both parts keep their XCD mapping.
template <typename T, bool FILTER, bool HAS_BIAS>
__global__ __launch_bounds__(kThreads) void k_grad_replay(GradArgs<T> g, ReplayArgs<T> r, int n_grad) {
  if ((int)blockIdx.x < n_grad) grad_body<T>((int)blockIdx.x, g);
  else replay_body<T, FILTER, HAS_BIAS>((int)blockIdx.x - n_grad, r);
}
template <typename T, bool FILTER> constexpr int grad_replay_lds_bytes() {
  return grad_lds_bytes<T>() > replay_lds_bytes<T, FILTER>() ? grad_lds_bytes<T>() : replay_lds_bytes<T, FILTER>();
}

// ============================================================== K6 finalize
// dH[n] = sum_ks slot[ks][inv[n]] for supervised rows (G already carries the
// row factors), 0 otherwise.
template <typename T>
__global__ void k_dh_finalize(const float* __restrict__ slots, int S, int64_t slot_stride,
                              const int* __restrict__ inv, int64_t N, int D, T* __restrict__ dH) {
  const int vpr = D / 4;
  const int64_t total = N * vpr;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < total;
       q += (int64_t)gridDim.x * blockDim.x) {
    const int64_t n = q / vpr;
    const int d = (int)(q % vpr) * 4;
    const int c = inv[n];
    float o[4] = {0.f, 0.f, 0.f, 0.f};
    if (c >= 0) {
      for (int s = 0; s < S; ++s) {
        const f32x4_t v = *reinterpret_cast<const f32x4_t*>(slots + s * slot_stride + (int64_t)c * D + d);
        o[0] += v[0];
        o[1] += v[1];
        o[2] += v[2];
        o[3] += v[3];
      }
    }
    if constexpr (sizeof(T) == 2)
      *reinterpret_cast<uint2*>(dH + n * D + d) = uint2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    else
      *reinterpret_cast<f32x4_t*>(dH + n * D + d) = f32x4_t{o[0], o[1], o[2], o[3]};
  }
}

// db[v] = sum_rb dbp[rb][v] in row-block order.
template <typename T>
__global__ void k_db_finalize(const float* __restrict__ dbp, int n_rb, int64_t lddb, int V,
                              T* __restrict__ db) {
  for (int v = blockIdx.x * blockDim.x + threadIdx.x; v < V; v += gridDim.x * blockDim.x) {
    float s = 0.f;
    // Unrolled so that several row blocks' loads are in flight at once; the
    // sum keeps the ascending row-block order.
#pragma unroll 8
    for (int rb = 0; rb < n_rb; ++rb) s += dbp[(int64_t)rb * lddb + v];
    db[v] = from_f32<T>(s);
  }
}

}  // namespace lce
