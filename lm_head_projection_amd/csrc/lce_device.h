// Device-side building blocks for the gfx950 (CDNA4) kernels: element types,
// the tile configuration, global->LDS tile loaders and the MFMA stage.
//
// Every contraction on the path (forward projection, backward replay, dH and
// dW) is an LDS-tiled MFMA GEMM (AIInfraGuide chapter 2, section 3.1: stage a
// block of A and B on chip, reuse it for many outputs, accumulate along K).
// One workgroup of 8 wave64s owns a BM x BN output tile; each wave owns a
// (BM/2) x (BN/4) sub-tile made of 32x32 MFMA blocks.  LDS holds two stages
// of the A and B tiles, stored [row][k] with a 16-byte row pad so the 16-byte
// MFMA operand reads of 32 consecutive rows hit distinct banks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lce {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kThreads = 512;  // 8 wave64 per workgroup
constexpr int kWarp = 64;

// ---------------------------------------------------------------- element types
// bf16 values travel as their 16-bit patterns (uint16_t); fp32 as float.
__device__ __forceinline__ float to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }
__device__ __forceinline__ float to_f32(float x) { return x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ uint16_t from_f32<uint16_t>(float x) {
  // Round to nearest even (hardware conversion on gfx950).
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// Two floats to a bf16 pair (a in the low half), round to nearest even: one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// ---------------------------------------------------------------- tile config
template <typename T> struct Cfg;
template <> struct Cfg<uint16_t> {
  static constexpr int BM = 256, BN = 256, BK = 32;  // BK: k granularity of the dH splits
  static constexpr int VEC = 8;     // elements per 16-byte vector
  static constexpr int KG = 4;      // k rows per transposed block (K-outer loader)
  static constexpr int ESZ = 2;
  static constexpr int STRIDE = BK + 8;  // LDS row stride in elements (80 B)
};
template <> struct Cfg<float> {
  static constexpr int BM = 128, BN = 128, BK = 32;
  static constexpr int VEC = 4;
  static constexpr int KG = 2;
  static constexpr int ESZ = 4;
  static constexpr int STRIDE = BK + 4;  // 144 B
};

template <typename T> struct Geo {
  using C = Cfg<T>;
  static constexpr int WGM = 2, WGN = 4;               // wave grid
  static constexpr int WTM = C::BM / WGM, WTN = C::BN / WGN;
  static constexpr int TM = WTM / 32, TN = WTN / 32;   // 32x32 blocks per wave
  static constexpr int A_ELEMS = C::BM * C::STRIDE;    // one stage of A in LDS
  static constexpr int B_ELEMS = C::BN * C::STRIDE;
  static constexpr int STAGE_ELEMS = A_ELEMS + B_ELEMS;
  static constexpr int LDS_BYTES = 2 * STAGE_ELEMS * C::ESZ;
};

// MFMA output element (tm, tn, i) of lane l sits at
//   row (M index) = wm*WTM + tm*32 + 8*(i/4) + 4*(l/32) + (i%4)
//   col (N index) = wn*WTN + tn*32 + (l%32)
// (v_mfma_f32_32x32x16_bf16 / v_mfma_f32_32x32x2_f32 accumulator layout).
__device__ __forceinline__ int acc_row(int tm, int i, int lane) {
  return tm * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}

// ---------------------------------------------------------------- loaders
// Global loads go through buffer resources: the hardware returns 0 for any
// 16-byte vector at or past `num_records`, so tiles that hang over the end of
// an operand need no per-vector branches.  Resources are rebased at the tile
// (or stage) origin so every offset stays far below 2^32 bytes.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int64_t n = bytes < 0 ? 0 : (bytes > 0xFFFFFF00ll ? 0xFFFFFF00ll : bytes);
  // Third dword: 32-bit data format, as required for raw (untyped) loads on gfx9.
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)(uint32_t)n,
                                           0x00020000);
}
// An offset no resource range reaches (num_records <= 0xFFFFFF00 < off).
constexpr uint32_t kOobOffset = 0xFFFFFFF0u;
__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// K-contiguous operand: element (r, k) at base[r*ld + k], `elems` elements
// from base to the end of the operand.  The tile holds ROWS rows x BK
// k-values; each thread moves whole 16-byte vectors.
template <typename T, int ROWS, bool KC> struct Loader;

template <typename T, int ROWS> struct Loader<T, ROWS, true> {
  using C = Cfg<T>;
  static constexpr int VPR = C::BK / C::VEC;
  static constexpr int NV = ROWS * VPR / kThreads;
  static_assert(NV * kThreads == ROWS * VPR, "tile/thread mismatch");
  u32x4 r[NV];
  __amdgpu_buffer_rsrc_t rs;
  int64_t ld;
  __device__ __forceinline__ void init(const T* base, int64_t elems, int64_t ld_, int row0) {
    ld = ld_;
    rs = make_rsrc(base + (int64_t)row0 * ld_, (elems - (int64_t)row0 * ld_) * (int64_t)sizeof(T));
  }
  // k0: first k of the stage; k-vectors at or past kend load 0 (only checked
  // when the stage straddles kend).
  __device__ __forceinline__ void load(int k0, int kend) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int q = threadIdx.x + j * kThreads;
      const int rr = q / VPR, kv = q % VPR;
      uint32_t off = (uint32_t)(((int64_t)rr * ld + k0 + kv * C::VEC) * (int64_t)sizeof(T));
      // A k-vector past kend gets an offset past num_records: the hardware
      // returns 0 and no wait on the loaded value is needed.
      if (k0 + kv * C::VEC >= kend) off = kOobOffset;
      r[j] = buf_load16(rs, off);
    }
  }
  __device__ __forceinline__ void store(T* lds) const {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int q = threadIdx.x + j * kThreads;
      const int rr = q / VPR, kv = q % VPR;
      *reinterpret_cast<u32x4*>(lds + rr * C::STRIDE + kv * C::VEC) = r[j];
    }
  }
};

// K-outer operand: element (r, k) at base[k*ld + r]; k-rows past the end of
// the operand load 0.  Each thread loads KG consecutive k-rows of one 16-byte
// vector of r values and transposes the KG x VEC block in registers, so LDS
// still holds [r][k].
template <typename T, int ROWS> struct Loader<T, ROWS, false> {
  using C = Cfg<T>;
  static constexpr int KGRP = C::BK / C::KG;   // k-groups per stage
  static constexpr int NGRP = ROWS / C::VEC;   // r-vectors per row of the tile
  static constexpr int NB = KGRP * NGRP / kThreads;
  static_assert(NB * kThreads == KGRP * NGRP, "tile/thread mismatch");
  u32x4 r[NB][C::KG];
  const T* base;
  int64_t elems, ld;
  int mn0;
  __device__ __forceinline__ void init(const T* base_, int64_t elems_, int64_t ld_, int mn0_) {
    base = base_;
    elems = elems_;
    ld = ld_;
    mn0 = mn0_;
  }
  __device__ __forceinline__ void load(int k0, int /*kend*/) {
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(base + (int64_t)k0 * ld, (elems - (int64_t)k0 * ld) * (int64_t)sizeof(T));
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int q = threadIdx.x + b * kThreads;
      const int kg = q % KGRP, g = q / KGRP;
#pragma unroll
      for (int kr = 0; kr < C::KG; ++kr)
        r[b][kr] = buf_load16(
            rs, (uint32_t)(((int64_t)(kg * C::KG + kr) * ld + mn0 + g * C::VEC) * (int64_t)sizeof(T)));
    }
  }
  __device__ __forceinline__ void store(T* lds) const {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int q = threadIdx.x + b * kThreads;
      const int kg = q % KGRP, g = q / KGRP;
      if constexpr (sizeof(T) == 2) {
        // 4 k-rows x 8 bf16: output row j gets (k0..k3) of element j.
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int w = j >> 1;
          uint32_t d0, d1;
          if ((j & 1) == 0) {
            d0 = (r[b][0][w] & 0xFFFFu) | (r[b][1][w] << 16);
            d1 = (r[b][2][w] & 0xFFFFu) | (r[b][3][w] << 16);
          } else {
            d0 = (r[b][0][w] >> 16) | (r[b][1][w] & 0xFFFF0000u);
            d1 = (r[b][2][w] >> 16) | (r[b][3][w] & 0xFFFF0000u);
          }
          *reinterpret_cast<u32x2*>(lds + (g * 8 + j) * C::STRIDE + kg * 4) = u32x2{d0, d1};
        }
      } else {
        // 2 k-rows x 4 fp32.
#pragma unroll
        for (int j = 0; j < 4; ++j)
          *reinterpret_cast<u32x2*>(lds + (g * 4 + j) * C::STRIDE + kg * 2) =
              u32x2{r[b][0][j], r[b][1][j]};
      }
    }
  }
};

// ---------------------------------------------------------------- MFMA stage
template <typename T>
__device__ __forceinline__ void mma_stage(const T* __restrict__ As, const T* __restrict__ Bs,
                                          f32x16_t (&acc)[Geo<T>::TM][Geo<T>::TN], int wm, int wn,
                                          int lane) {
  using C = Cfg<T>;
  using G = Geo<T>;
  const int lr = lane & 31, lk = 8 * (lane >> 5);
  const T* a_base = As + (wm * G::WTM + lr) * C::STRIDE + lk;
  const T* b_base = Bs + (wn * G::WTN + lr) * C::STRIDE + lk;
  if constexpr (sizeof(T) == 2) {
    // Operand fragments are double-buffered across the k-substeps: the LDS
    // reads of substep kk+1 are in flight while substep kk's MFMAs run.
    constexpr int KK = C::BK / 16;
    u32x4 a[2][G::TM], b[2][G::TN];
#pragma unroll
    for (int tm = 0; tm < G::TM; ++tm)
      a[0][tm] = *reinterpret_cast<const u32x4*>(a_base + tm * 32 * C::STRIDE);
#pragma unroll
    for (int tn = 0; tn < G::TN; ++tn)
      b[0][tn] = *reinterpret_cast<const u32x4*>(b_base + tn * 32 * C::STRIDE);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int cb = kk & 1, nb = cb ^ 1;
      if (kk + 1 < KK) {
#pragma unroll
        for (int tm = 0; tm < G::TM; ++tm)
          a[nb][tm] = *reinterpret_cast<const u32x4*>(a_base + tm * 32 * C::STRIDE + (kk + 1) * 16);
#pragma unroll
        for (int tn = 0; tn < G::TN; ++tn)
          b[nb][tn] = *reinterpret_cast<const u32x4*>(b_base + tn * 32 * C::STRIDE + (kk + 1) * 16);
      }
#pragma unroll
      for (int tm = 0; tm < G::TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < G::TN; ++tn)
          acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8_t, a[cb][tm]), __builtin_bit_cast(bf16x8_t, b[cb][tn]),
              acc[tm][tn], 0, 0, 0);
    }
  } else {
    // fp32: lane l supplies k = kk*16 + 8*(l/32) + j to the j-th 32x32x2 MFMA;
    // A and B use the same k-slots, so the 8 MFMAs sum all 16 k-values.
#pragma unroll
    for (int kk = 0; kk < C::BK / 16; ++kk) {
      float a[G::TM][8], b[G::TN][8];
#pragma unroll
      for (int tm = 0; tm < G::TM; ++tm) {
        const float* p = a_base + tm * 32 * C::STRIDE + kk * 16;
        *reinterpret_cast<u32x4*>(&a[tm][0]) = *reinterpret_cast<const u32x4*>(p);
        *reinterpret_cast<u32x4*>(&a[tm][4]) = *reinterpret_cast<const u32x4*>(p + 4);
      }
#pragma unroll
      for (int tn = 0; tn < G::TN; ++tn) {
        const float* p = b_base + tn * 32 * C::STRIDE + kk * 16;
        *reinterpret_cast<u32x4*>(&b[tn][0]) = *reinterpret_cast<const u32x4*>(p);
        *reinterpret_cast<u32x4*>(&b[tn][4]) = *reinterpret_cast<const u32x4*>(p + 4);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int tm = 0; tm < G::TM; ++tm)
#pragma unroll
          for (int tn = 0; tn < G::TN; ++tn)
            acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[tm][j], b[tn][j], acc[tm][tn], 0, 0, 0);
    }
  }
}

// ---------------------------------------------------------------- main loop
// acc[BM x BN] += A_tile . B_tile^T over k in [k0, k0 + nsteps*BK).
// A: rows = M index, K-contiguous if A_KC (origin at row m0 = base + m0*lda)
// or K-outer (element (m, k) at base[k*lda + m]); `a_elems` = elements from
// `A` to the end of the operand.  B likewise for the N index.  K-contiguous
// k-vectors at or past `kend` load 0.  Caller guarantees no wave still reads
// `smem` from an earlier use.
template <typename T, bool A_KC, bool B_KC>
__device__ __forceinline__ void gemm_tile(const T* __restrict__ A, int64_t a_elems, int64_t lda, int m0,
                                          const T* __restrict__ B, int64_t b_elems, int64_t ldb, int n0,
                                          int k0, int kend, int nsteps,
                                          f32x16_t (&acc)[Geo<T>::TM][Geo<T>::TN], T* smem) {
  using C = Cfg<T>;
  using G = Geo<T>;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave % G::WGM, wn = wave / G::WGM;
  Loader<T, C::BM, A_KC> la;
  Loader<T, C::BN, B_KC> lb;
  la.init(A, a_elems, lda, m0);
  lb.init(B, b_elems, ldb, n0);
  la.load(k0, kend);
  lb.load(k0, kend);
  la.store(smem);
  lb.store(smem + G::A_ELEMS);
  __syncthreads();
  for (int s = 0; s < nsteps; ++s) {
    const bool more = s + 1 < nsteps;
    T* cur = smem + (s & 1) * G::STAGE_ELEMS;
    T* nxt = smem + ((s + 1) & 1) * G::STAGE_ELEMS;
    if (more) {
      la.load(k0 + (s + 1) * C::BK, kend);
      lb.load(k0 + (s + 1) * C::BK, kend);
    }
    mma_stage<T>(cur, cur + G::A_ELEMS, acc, wm, wn, lane);
    if (more) {
      la.store(nxt);
      lb.store(nxt + G::A_ELEMS);
    }
    __syncthreads();
  }
}

template <typename T>
__device__ __forceinline__ void zero_acc(f32x16_t (&acc)[Geo<T>::TM][Geo<T>::TN]) {
#pragma unroll
  for (int tm = 0; tm < Geo<T>::TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < Geo<T>::TN; ++tn)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[tm][tn][i] = 0.f;
}

// ---------------------------------------------------------------- LSE helpers
// Merge running state (m, s) with (m2, s2): the online-softmax merge
// (AIInfraGuide chapter 2, section 9.4) in base 2.  A state with m = -inf is
// empty (s = 0); its rescale factor is 0.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) {
    m = mn;
    return;
  }
  s = s * __builtin_amdgcn_exp2f((m - mn) * kLog2e) + s2 * __builtin_amdgcn_exp2f((m2 - mn) * kLog2e);
  m = mn;
}

// Butterfly reduce-scatter over the 32 lanes of each half-wave: afterwards
// lane l holds, in v[0..NV/32), the sums over lanes of entries
// (l%32)*(NV/32) + j.  The order of additions is fixed (deterministic).
template <int CNT, int MASK>
__device__ __forceinline__ void bfly_step(float* v, int lane) {
  const bool hi = (lane & MASK) != 0;
#pragma unroll
  for (int e = 0; e < CNT / 2; ++e) {
    const float keep = hi ? v[e + CNT / 2] : v[e];
    const float send = hi ? v[e] : v[e + CNT / 2];
    v[e] = keep + __shfl_xor(send, MASK);
  }
}
template <int NV>
__device__ __forceinline__ void halfwave_reduce_scatter(float (&v)[NV], int lane) {
  static_assert(NV >= 32 && (NV & (NV - 1)) == 0, "NV must be a power of two >= 32");
  bfly_step<NV, 16>(v, lane);
  bfly_step<NV / 2, 8>(v, lane);
  bfly_step<NV / 4, 4>(v, lane);
  bfly_step<NV / 8, 2>(v, lane);
  bfly_step<NV / 16, 1>(v, lane);
}

// Workgroup -> work item remap: the 8 XCDs take workgroups round-robin, so
// workgroup b runs on XCD b%8.  Giving each XCD a contiguous range of work
// items keeps the items that share operand tiles on one L2.
__device__ __forceinline__ int xcd_remap(int b, int per_xcd) { return (b & 7) * per_xcd + (b >> 3); }

// Grouped order over an (n_a x n_b) grid of work items: consecutive items
// walk GA values of `a` before advancing `b`, so the ~32 workgroups that run
// together on one XCD touch GA row blocks and 32/GA column blocks (their
// operand tiles then stay in that XCD's L2).  The last group may be short.
template <int GA>
__device__ __forceinline__ void grouped_index(int w, int n_a, int n_b, int& a, int& b) {
  const int per_group = GA * n_b;
  const int g = w / per_group;
  const int first = g * GA;
  const int rows = min(n_a - first, GA);
  const int r = w - g * per_group;
  a = first + r % rows;
  b = r / rows;
}

}  // namespace lce
