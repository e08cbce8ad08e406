// Host side of the C ABI declared in include/lce.h: argument checks,
// workspace layout, launch sequencing on the caller's stream, status codes.
// No device memory is allocated here; the caller passes the workspace.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <set>
#include <cstdint>
#include <cstring>
#include <string>
#include <vector>

#include "lce.h"
#include "lce_kernels.h"

#include <cmath>

static_assert(LCE_REDUCTION_MEAN == lce::kReduceMean && LCE_REDUCTION_SUM == lce::kReduceSum &&
                  LCE_REDUCTION_NONE == lce::kReduceNone,
              "reduction codes of the ABI and the kernels agree");

using namespace lce;

namespace {

constexpr int64_t kVcMax = 32768;    // vocabulary chunk of the gradient tile store
constexpr int kMaxSplit = 64;         // vocabulary splits of the forward pass
constexpr int kDhSlotRows = 4;        // the dH slots hold 4 x Rpad rows of D fp32 values
constexpr int kMaxDhSlots = 16;       // k-splits of the dH GEMM (at most)
constexpr int kCUs = 256;             // MI355X compute units (one 512-thread workgroup each)
// Replay tiles per CU below which a fused launch's replay items take one tile
// each instead of two (measured: 2.5 and 14.5 tiles per CU gain with single
// tiles, 22.5 lose).
constexpr int kFusedTilesPerCu = 16;

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t rup(int64_t a, int64_t b) { return cdiv(a, b) * b; }
size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

// ------------------------------------------------------------------ profiling
struct Prof {
  bool on = false;
  int max = 0, used = 0, pending_kid = -1;
  double pending_flops = 0.0;
  std::vector<hipEvent_t> ev;
  std::vector<int> kid;
  std::vector<double> lflops;  // per recorded launch
  std::vector<std::string> names;
  std::vector<double> ms, flops;
  std::vector<int64_t> cnt;
};
Prof g_prof;

// flops: the launch's algorithmic floating-point operations (0 for the
// kernels outside the GEMMs).
void prof_begin(const char* name, hipStream_t s, double flops = 0.0) {
  Prof& p = g_prof;
  p.pending_kid = -1;
  p.pending_flops = flops;
  if (!p.on || p.used >= p.max) return;
  int id = -1;
  for (size_t i = 0; i < p.names.size(); ++i)
    if (p.names[i] == name) id = (int)i;
  if (id < 0) {
    id = (int)p.names.size();
    p.names.push_back(name);
    p.ms.push_back(0.0);
    p.flops.push_back(0.0);
    p.cnt.push_back(0);
  }
  if (hipEventRecord(p.ev[2 * p.used], s) != hipSuccess) return;
  p.pending_kid = id;
}
void prof_end(hipStream_t s) {
  Prof& p = g_prof;
  if (p.pending_kid < 0) return;
  if (hipEventRecord(p.ev[2 * p.used + 1], s) == hipSuccess) {
    p.kid[p.used] = p.pending_kid;
    p.lflops[p.used] = p.pending_flops;
    p.used++;
  }
  p.pending_kid = -1;
}

#define LCE_LAUNCH(name, kernel, grid, block, shmem, stream, ...) \
  LCE_LAUNCH_F(name, 0.0, kernel, grid, block, shmem, stream, __VA_ARGS__)
// A GEMM launch, with its algorithmic flops for the profiler.
#define LCE_LAUNCH_F(name, flops, kernel, grid, block, shmem, stream, ...)         \
  do {                                                                             \
    prof_begin(name, stream, flops);                                               \
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(block), shmem, stream, __VA_ARGS__); \
    hipError_t e_ = hipGetLastError();                                             \
    prof_end(stream);                                                              \
    if (e_ != hipSuccess) return LCE_ERR_HIP;                                      \
  } while (0)

// ------------------------------------------------------------------ layout
template <typename T> struct Tile {
  static constexpr int BM = Cfg<T>::BM;  // vocabulary tile (forward) / M tile (gradients)
  static constexpr int BN = Cfg<T>::BN;  // row block
};

// A reduction of the per-row CE: mean over C, or sum_i w_i l_i / div, or none.
struct Reduce {
  int kind = kReduceMean;
  const float* weights = nullptr;  // [N] per position (sum only) or null
  double div = 1.0;                // sum only: the divisor (num_label_tokens, else 1)
};

struct Layout {
  // compaction
  size_t counts, bad, offsets, stat;
  // shared by forward and backward
  size_t hc, yc;
  // forward
  size_t pm, ps, tgt, lrow;
  // backward
  size_t mc, lsc, rsc, inv, G, slots, dbp, flags;
  size_t fwd_total;  // compaction + forward calls
  size_t total;      // every call (the backward region is the larger one)
  int64_t Npad, Vpad, Vc, nblk;
  int64_t Rpad;  // rows of the backward arrays: the supervised rows, padded to 256
};

// rows: the supervised rows C the backward region serves (0 <= C <= N), or -1
// for the worst case C = N.  The compaction, shared and forward regions are
// sized by N.
bool make_layout(int64_t N, int64_t D, int64_t V, lce_dtype_t dt, Layout& L, int64_t rows = -1) {
  if (N < 0 || D <= 0 || V <= 0) return false;
  if (dt != LCE_DTYPE_F32 && dt != LCE_DTYPE_BF16) return false;
  if (rows > N) return false;
  const int64_t esz = dt == LCE_DTYPE_BF16 ? 2 : 4;
  const int64_t bn = dt == LCE_DTYPE_BF16 ? Tile<uint16_t>::BN : Tile<float>::BN;
  L.Npad = rup(std::max<int64_t>(N, 1), 256);
  L.Rpad = rows < 0 ? L.Npad : rup(std::max<int64_t>(rows, 1), 256);
  L.nblk = cdiv(std::max<int64_t>(N, 1), kCmpBlock);
  L.Vpad = rup(V, 256);
  L.Vc = std::min<int64_t>(L.Vpad, kVcMax);
  // The GEMM operands are addressed with 32-bit buffer offsets from a tile
  // origin: keep one chunk of G (Rpad x Vc) and of W (Vc x D) within 2 GB.
  const int64_t vc_cap = std::min(((int64_t)1 << 31) / (L.Rpad * esz), ((int64_t)1 << 31) / (D * esz)) / 256 * 256;
  if (vc_cap < 256) return false;
  L.Vc = std::min(L.Vc, vc_cap);
  size_t off = 0;
  auto take = [&](int64_t bytes) {
    const size_t o = off;
    off = a256(off + (size_t)bytes);
    return o;
  };
  L.counts = take(L.nblk * 4);
  L.bad = take(L.nblk * 4);
  L.offsets = take(L.nblk * 4);
  L.stat = take(16);
  L.hc = take(L.Npad * D * esz);
  L.yc = take(L.Npad * 4);
  const size_t common_end = off;
  // forward region
  L.pm = take((int64_t)kMaxSplit * L.Npad * 4);
  L.ps = take((int64_t)kMaxSplit * L.Npad * 4);
  L.tgt = take(L.Npad * 4);
  L.lrow = take(L.Npad * 4);
  const size_t fwd_end = off;
  L.fwd_total = fwd_end;
  // backward region overlays the forward region (the calls never overlap)
  off = common_end;
  L.mc = take(L.Rpad * 4);
  L.lsc = take(L.Rpad * 4);
  L.rsc = take(L.Rpad * 4);
  L.inv = take(std::max<int64_t>(N, 1) * 4);
  // bf16: two chunk buffers of G (and of the filter flags), so that the
  // replay of chunk c+1 can run inside the gradient launch of chunk c.
  const int64_t nbuf = dt == LCE_DTYPE_BF16 ? 2 : 1;
  L.G = take(nbuf * L.Rpad * L.Vc * esz);
  L.slots = take((int64_t)kDhSlotRows * L.Rpad * D * 4);
  L.dbp = take((L.Rpad / bn) * L.Vpad * 4);
  L.flags = take(nbuf * (L.Rpad / 256) * (L.Vc / 32));  // gradient filter: live G blocks of a chunk
  L.total = std::max(off, fwd_end);
  return true;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Once per (device, kernel): each kernel always asks for the same LDS size,
// and the attribute call costs host time that the GPU would wait for.
template <typename T> void set_lds_attr(const void* fn, int bytes) {
  static std::mutex mu;
  static std::set<std::pair<int, const void*>> done;
  int dev = 0;
  (void)hipGetDevice(&dev);
  std::lock_guard<std::mutex> lock(mu);
  if (done.insert({dev, fn}).second) (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

// Number of vocabulary splits for the forward grid: minimise
// (waves of workgroups) x (tiles per split), ties to fewer splits.
int choose_split(int n_rb, int n_vt) {
  int best = 1;
  int64_t best_cost = INT64_MAX;
  for (int ns = 1; ns <= std::min(n_vt, kMaxSplit); ++ns) {
    const int64_t waves = cdiv((int64_t)n_rb * ns, kCUs);
    const int64_t cost = waves * cdiv(n_vt, ns);
    if (cost < best_cost) {
      best_cost = cost;
      best = ns;
    }
  }
  return best;
}

// Makespan of a chunk's gradient items: each of the 8 XCDs takes an equal share of
// the n_a items of length L_a and of the n_b items of length L_b, and runs its
// share on its kCUs/8 workgroup slots, the longer kind first, each item on the
// slot that frees first (the dispatcher's order).
int64_t makespan(int64_t n_a, int64_t L_a, int64_t n_b, int64_t L_b) {
  int64_t worst = 0;
  for (int x = 0; x < 8; ++x) {
    std::vector<int64_t> slot(kCUs / 8, 0);
    auto place = [&](int64_t n, int64_t L) {
      for (int64_t i = 0; i < n; ++i) {
        auto it = std::min_element(slot.begin(), slot.end());
        *it += L;
      }
    };
    const int64_t ca = (x + 1) * n_a / 8 - x * n_a / 8, cb = (x + 1) * n_b / 8 - x * n_b / 8;
    if (L_a >= L_b) {
      place(ca, L_a);
      place(cb, L_b);
    } else {
      place(cb, L_b);
      place(ca, L_a);
    }
    worst = std::max(worst, *std::max_element(slot.begin(), slot.end()));
  }
  return worst;
}

// dH k-splits for one chunk: the split count whose grouped launch (dH tiles of
// K = chunk/S next to dW tiles of K = Cpad) has the shortest makespan.
// S is bounded by the slot memory: S x Cpad rows must fit in kDhSlotRows x Rpad.
int choose_dh_splits(int64_t kpad, int64_t Cpad, int64_t Rpad, int64_t n_dh_tiles_per_split, int64_t n_dw_tiles,
                     int bk) {
  int best = 1;
  int64_t best_t = INT64_MAX;
  const int s_max = (int)std::max<int64_t>(1, std::min<int64_t>(kMaxDhSlots, kDhSlotRows * Rpad / Cpad));
  for (int S = 1; S <= s_max; ++S) {
    const int64_t ks_len = rup(cdiv(kpad, S), bk);
    const int64_t S_eff = cdiv(kpad, ks_len);
    const int64_t t = makespan(n_dh_tiles_per_split * S_eff, ks_len + 2 * bk, n_dw_tiles, Cpad + 2 * bk);
    if (t < best_t) {
      best_t = t;
      best = S;
    }
  }
  return best;
}

// Replay tiles per workgroup (at most 8, ties to fewer): minimises the
// makespan in pipeline stages,
// waves * (tpw * nsteps + kItemStages), where kItemStages stands for the
// per-workgroup cost the tile walk cannot hide (the first stages' load
// latency and the last tile's epilogue).
constexpr int kItemStages = 3;
int choose_tiles_per_wg(int n_rb, int vtiles, int nsteps) {
  int best = 1;
  int64_t best_cost = INT64_MAX;
  for (int tpw = 1; tpw <= std::min(vtiles, 8); ++tpw) {
    const int64_t waves = cdiv((int64_t)n_rb * cdiv(vtiles, tpw), kCUs);
    const int64_t cost = waves * ((int64_t)tpw * nsteps + kItemStages);
    if (cost < best_cost) {
      best_cost = cost;
      best = tpw;
    }
  }
  return best;
}

lce_status_t zero_bytes(void* p, int64_t bytes, hipStream_t s) {
  if (!p || bytes <= 0) return LCE_OK;
  const int64_t n16 = bytes / 16;
  const int tail = (int)(bytes - n16 * 16);
  const int64_t grid = std::max<int64_t>(1, std::min<int64_t>(cdiv(n16, 256), 4096));
  LCE_LAUNCH("k_zero", k_zero, grid, 256, 0, s, (u32x4*)p, n16, (uint8_t*)p + n16 * 16, tail);
  return LCE_OK;
}

// m = log s = -inf and l = 0 at all n positions (each array may be null).
lce_status_t fill_stats(float* m, float* logs, float* row_loss, int64_t n, hipStream_t s) {
  if ((!m && !logs && !row_loss) || n <= 0) return LCE_OK;
  const int64_t grid = std::max<int64_t>(1, std::min<int64_t>(cdiv(n, 256), 4096));
  LCE_LAUNCH("k_fill_stats", k_fill_stats, grid, 256, 0, s, m, logs, row_loss, n);
  return LCE_OK;
}

#define LCE_TRY(x)                       \
  do {                                   \
    lce_status_t st_ = (x);              \
    if (st_ != LCE_OK) return st_;       \
  } while (0)

// ------------------------------------------------------------------ forward
template <typename T>
lce_status_t forward_impl(const T* H, const T* W, const T* b, const int64_t* labels,
                          const int32_t* idx, int64_t C, int64_t N, int64_t D, int64_t V, int64_t label_off,
                          const Reduce& red, float* loss, float* m, float* logs, float* row_loss,
                          float* shard_part, char* ws, const Layout& L, hipStream_t s) {
  using Cf = Cfg<T>;
  const int Cpad = (int)rup(C, 256);
  T* Hc = reinterpret_cast<T*>(ws + L.hc);
  int* yc = reinterpret_cast<int*>(ws + L.yc);
  float* pm = reinterpret_cast<float*>(ws + L.pm);
  float* ps = reinterpret_cast<float*>(ws + L.ps);
  float* tgt = reinterpret_cast<float*>(ws + L.tgt);
  float* lrow = reinterpret_cast<float*>(ws + L.lrow);

  {
    const int64_t vec = (int64_t)Cpad * (D / (16 / (int64_t)sizeof(T)));
    const int64_t grid = std::max<int64_t>(1, std::min<int64_t>(cdiv(vec, 256), 8192));
    // The vocabulary shard path writes no per-position statistics.
    PosFill fill;
    if (!shard_part) {
      fill.m = m;
      fill.logs = logs;
      fill.row_loss = row_loss;
      fill.N = N;
    }
    LCE_LAUNCH("k_gather", (k_gather<T>), grid, 256, 0, s, H, labels, idx, (int)C, Cpad, (int)D, label_off, Hc,
               yc, (const float*)nullptr, (const float*)nullptr, (float*)nullptr, (float*)nullptr, fill);
  }
  const int n_rb = Cpad / Cf::BN;
  const int n_vt = (int)cdiv(V, Cf::BM);
  const int n_split = choose_split(n_rb, n_vt);
  const int n_work = n_rb * n_split;
  const int per_xcd = (int)cdiv(n_work, 8);
  const double fwd_flops = 2.0 * (double)C * (double)V * (double)D;  // one logit per (row, entry)
  if (b) {
    set_lds_attr<T>((const void*)k_fwd<T, true>, gemm_lds_bytes<T>());
    LCE_LAUNCH_F("k_fwd", fwd_flops, (k_fwd<T, true>), per_xcd * 8, kThreads, gemm_lds_bytes<T>(), s, W, b, Hc,
                 yc, Cpad, (int)D, (int)V, n_rb, n_split, n_vt, n_work, per_xcd, pm, ps, tgt);
  } else {
    set_lds_attr<T>((const void*)k_fwd<T, false>, gemm_lds_bytes<T>());
    LCE_LAUNCH_F("k_fwd", fwd_flops, (k_fwd<T, false>), per_xcd * 8, kThreads, gemm_lds_bytes<T>(), s, W, b, Hc,
                 yc, Cpad, (int)D, (int)V, n_rb, n_split, n_vt, n_work, per_xcd, pm, ps, tgt);
  }
  if (shard_part) {  // vocabulary shard: the row partials only
    LCE_LAUNCH("k_shard_partial", k_shard_partial, cdiv(C, 256), 256, 0, s, pm, ps, tgt, n_split, Cpad, (int)C, yc,
               (int)V, shard_part, shard_part + C, shard_part + 2 * C);
    return LCE_OK;
  }
  LCE_LAUNCH("k_merge", k_merge, cdiv(C, 256), 256, 0, s, pm, ps, tgt, n_split, Cpad, (int)C, idx, m,
             logs, row_loss, lrow);
  if (loss)
    LCE_LAUNCH("k_loss_sum", k_loss_sum, 1, 1024, 0, s, lrow, (int)C, (int)red.kind, red.weights, idx,
               red.div, loss);
  return LCE_OK;
}

// ------------------------------------------------------------------ backward
template <typename T>
lce_status_t backward_impl(const T* H, const T* W, const T* b, const int64_t* labels,
                           const int32_t* idx, int64_t C, int64_t N, int64_t D, int64_t V, int64_t label_off,
                           const Reduce& red, const float* m, const float* logs, const float* grad_loss,
                           T* dH, T* dW, T* db, char* ws, const Layout& L, hipStream_t s,
                           float filter_eps = -1.f, int filter_which = 0) {
  using Cf = Cfg<T>;
  const int Cpad = (int)rup(C, 256);
  T* Hc = reinterpret_cast<T*>(ws + L.hc);
  int* yc = reinterpret_cast<int*>(ws + L.yc);
  float* mc = reinterpret_cast<float*>(ws + L.mc);
  float* lsc = reinterpret_cast<float*>(ws + L.lsc);
  float* rsc = reinterpret_cast<float*>(ws + L.rsc);
  int* inv = reinterpret_cast<int*>(ws + L.inv);
  T* Gc = reinterpret_cast<T*>(ws + L.G);
  float* slots = reinterpret_cast<float*>(ws + L.slots);
  float* dbp = reinterpret_cast<float*>(ws + L.dbp);
  const int64_t ldg = L.Vc;
  const int64_t slot_stride = (int64_t)Cpad * D;
  const int64_t lddb = L.Vpad;

  {
    const int64_t vec = (int64_t)Cpad * (D / (16 / (int64_t)sizeof(T)));
    const int64_t grid = std::max<int64_t>(1, std::min<int64_t>(cdiv(vec, 256), 8192));
    PosFill fill;
    fill.inv = inv;
    fill.N = N;
    LCE_LAUNCH("k_gather", (k_gather<T>), grid, 256, 0, s, H, labels, idx, (int)C, Cpad, (int)D, label_off, Hc,
               yc, m, logs, mc, lsc, fill);
  }
  LCE_LAUNCH("k_row_scale", k_row_scale, cdiv(Cpad, 256), 256, 0, s, idx, (int)C, Cpad, (int)red.kind,
             red.weights, (float)red.div, grad_loss, rsc, inv);
  const int n_rb = Cpad / Cf::BN;
  const int n_nt = (int)cdiv(D, Cf::BN);
  const int n_dh_mt = Cpad / Cf::BM;
  const bool filter = filter_eps >= 0.f && filter_which != 0;
  uint8_t* flags = filter ? reinterpret_cast<uint8_t*>(ws + L.flags) : nullptr;
  const int64_t fstride = L.Vc / 32;
  set_lds_attr<T>((const void*)k_replay<T, false, false>, replay_lds_bytes<T, false>());
  set_lds_attr<T>((const void*)k_replay<T, true, false>, replay_lds_bytes<T, true>());
  set_lds_attr<T>((const void*)k_replay<T, false, true>, replay_lds_bytes<T, false>());
  set_lds_attr<T>((const void*)k_replay<T, true, true>, replay_lds_bytes<T, true>());
  set_lds_attr<T>((const void*)k_grad<T>, grad_lds_bytes<T>());

  // Vocabulary chunks of at most L.Vc entries.
  struct Chunk {
    int64_t v0;
    int vc, vtiles, kpad;
  };
  std::vector<Chunk> chunks;
  for (int64_t v0 = 0; v0 < V; v0 += L.Vc) {
    const int vc = (int)std::min<int64_t>(L.Vc, V - v0);
    const int vtiles = (int)cdiv(vc, Cf::BM);
    chunks.push_back(Chunk{v0, vc, vtiles, vtiles * Cf::BM});
  }
  // bf16: chunk c+1's replay runs in chunk c's gradient launch (k_grad_replay),
  // through the other of two G (and flag) buffers.
  constexpr bool kFuse = sizeof(T) == 2;
  const int64_t g_elems = (int64_t)L.Rpad * L.Vc;
  const int64_t f_bytes = (L.Rpad / 256) * (L.Vc / 32);
  auto gbuf = [&](size_t c) { return Gc + (kFuse ? (int64_t)(c & 1) * g_elems : 0); };
  auto fbuf = [&](size_t c) { return flags ? flags + (kFuse ? (int64_t)(c & 1) * f_bytes : 0) : flags; };
  const bool bias_terms = b != nullptr || db != nullptr;  // a bias to add or db partials to form
  // Every flag of the chunk's tiles is written (0 or 1) by the tile's replay.
  auto rargs = [&](size_t c) {
    const Chunk& k = chunks[c];
    ReplayArgs<T> a;
    a.W = W;
    a.bias = b;
    a.Hc = Hc;
    a.yc = yc;
    a.mc = mc;
    a.lsc = lsc;
    a.rsc = rsc;
    a.Cpad = Cpad;
    a.D = (int)D;
    a.V = (int)V;
    a.v0 = (int)k.v0;
    a.vtiles = k.vtiles;
    // Inside a fused launch (chunks 1...) the replay items fill the CUs the
    // gradient items leave: short items pack that tail best, 2 tiles each, or
    // single tiles when the chunk has fewer than kFusedTilesPerCu of them per CU.
    a.tpw = kFuse && c > 0 ? std::min((int64_t)n_rb * k.vtiles < (int64_t)kFusedTilesPerCu * kCUs ? 1 : 2, k.vtiles)
                           : choose_tiles_per_wg(n_rb, k.vtiles, (int)cdiv(D, sizeof(T) == 2 ? 64 : Cf::BK));
    a.n_rb = n_rb;
    a.n_work = n_rb * (int)cdiv(k.vtiles, a.tpw);
    a.per_xcd = (int)cdiv(a.n_work, 8);
    a.Gc = gbuf(c);
    a.ldg = ldg;
    a.dbp = db ? dbp : nullptr;
    a.lddb = lddb;
    a.flags = filter ? fbuf(c) : nullptr;
    a.fstride = fstride;
    a.eps = filter ? filter_eps : 0.f;
    a.zero_dead = filter && filter_which == LCE_FILTER_BOTH ? 1 : 0;
    return a;
  };
  auto replay_flops = [&](size_t c) { return 2.0 * (double)C * (double)chunks[c].vc * (double)D; };
  auto launch_replay = [&](size_t c) -> lce_status_t {
    const ReplayArgs<T> a = rargs(c);
    const int grid = a.per_xcd * 8;
    const double fl = replay_flops(c);
    if (filter && bias_terms)
      LCE_LAUNCH_F("k_replay", fl, (k_replay<T, true, true>), grid, kThreads, (replay_lds_bytes<T, true>()), s, a);
    else if (filter)
      LCE_LAUNCH_F("k_replay", fl, (k_replay<T, true, false>), grid, kThreads, (replay_lds_bytes<T, true>()), s, a);
    else if (bias_terms)
      LCE_LAUNCH_F("k_replay", fl, (k_replay<T, false, true>), grid, kThreads, (replay_lds_bytes<T, false>()), s, a);
    else
      LCE_LAUNCH_F("k_replay", fl, (k_replay<T, false, false>), grid, kThreads, (replay_lds_bytes<T, false>()), s,
                   a);
    return LCE_OK;
  };

  // dH slots: chunk 0 (the widest) fixes their number S and stores every one
  // of them; later chunks, whose splits never outnumber S, add into theirs.
  // k_dh_finalize sums exactly these S slots.
  int S = 0;
  if (kFuse) LCE_TRY(launch_replay(0));
  for (size_t c = 0; c < chunks.size(); ++c) {
    const Chunk& k = chunks[c];
    // K4: replay this chunk into G (bf16: done by the previous launch).
    if (!kFuse) LCE_TRY(launch_replay(c));
    // K5: dH split so that one dH tile's K matches one dW tile's K (= Cpad).
    if (c == 0)
      S = choose_dh_splits(k.kpad, Cpad, L.Rpad, (int64_t)n_dh_mt * n_nt, (int64_t)k.vtiles * n_nt, Cf::BK);
    const int64_t ks_len = rup(cdiv(k.kpad, S), Cf::BK);
    const int S_eff = (int)cdiv(k.kpad, ks_len);  // non-empty splits; a later chunk has ks_len >= kpad / S, so S_eff <= S
    if (c == 0) S = S_eff;
    GradArgs<T> g;
    g.Gc = gbuf(c);
    g.ldg = ldg;
    g.kpad_g = k.kpad;
    g.Hc = Hc;
    g.W = W;
    g.Cpad = Cpad;
    g.D = (int)D;
    g.v0 = (int)k.v0;
    g.vc = k.vc;
    g.w_rows = (int)(V - k.v0);
    g.n_nt = n_nt;
    g.n_dh_mt = n_dh_mt;
    g.ks_len = (int)ks_len;
    g.n_dh = n_dh_mt * n_nt * S_eff;
    g.n_dw_mt = k.vtiles;
    g.dh_first = ks_len >= Cpad ? 1 : 0;
    g.slots = slots;
    g.slot_stride = slot_stride;
    g.accumulate = c == 0 ? 0 : 1;
    g.dW = dW;
    g.flags = filter ? fbuf(c) : nullptr;
    g.fstride = fstride;
    g.fmask = filter_which;
    const int n_dw = k.vtiles * n_nt;
    const int n_grad = (int)(cdiv(g.n_dh, 8) + cdiv(n_dw, 8)) * 8;
    const double gfl = 4.0 * (double)C * (double)k.vc * (double)D;  // dH and dW products of the chunk
    if constexpr (kFuse) {
      if (c + 1 < chunks.size()) {
        const ReplayArgs<T> r = rargs(c + 1);
        const int grid = n_grad + r.per_xcd * 8;
        const double fl = gfl + replay_flops(c + 1);
#define LCE_FUSED(FILT, BIAS)                                                                         \
  do {                                                                                                \
    set_lds_attr<T>((const void*)k_grad_replay<T, FILT, BIAS>, grad_replay_lds_bytes<T, FILT>());     \
    LCE_LAUNCH_F("k_grad_replay", fl, (k_grad_replay<T, FILT, BIAS>), grid, kThreads,                 \
                 (grad_replay_lds_bytes<T, FILT>()), s, g, r, n_grad);                                \
  } while (0)
        if (filter && bias_terms) LCE_FUSED(true, true);
        else if (filter) LCE_FUSED(true, false);
        else if (bias_terms) LCE_FUSED(false, true);
        else LCE_FUSED(false, false);
#undef LCE_FUSED
        continue;
      }
    }
    LCE_LAUNCH_F("k_grad", gfl, (k_grad<T>), n_grad, kThreads, grad_lds_bytes<T>(), s, g);
  }
  {
    const int64_t vec = N * (D / 4);
    const int64_t grid = std::max<int64_t>(1, std::min<int64_t>(cdiv(vec, 256), 8192));
    LCE_LAUNCH("k_dh_finalize", (k_dh_finalize<T>), grid, 256, 0, s, slots, S, slot_stride, inv, N,
               (int)D, dH);
  }
  if (db) {
    const int64_t grid = std::max<int64_t>(1, std::min<int64_t>(cdiv(V, 256), 4096));
    LCE_LAUNCH("k_db_finalize", (k_db_finalize<T>), grid, 256, 0, s, dbp, n_rb, lddb, (int)V, db);
  }
  return LCE_OK;
}

bool dims_ok(int64_t N, int64_t D, int64_t V, lce_dtype_t dt) {
  if (N < 0 || D <= 0 || V <= 0) return false;
  if (dt != LCE_DTYPE_F32 && dt != LCE_DTYPE_BF16) return false;
  return true;
}

lce_status_t shape_supported(int64_t N, int64_t D, int64_t V, lce_dtype_t dt) {
  const int64_t vec = dt == LCE_DTYPE_BF16 ? 8 : 4;
  if (D % vec != 0) return LCE_ERR_UNSUPPORTED;
  if (N > (int64_t)1 << 30 || V > (int64_t)1 << 30 || D > (int64_t)1 << 20) return LCE_ERR_UNSUPPORTED;
  if (N * D > ((int64_t)1 << 40) || V * D > ((int64_t)1 << 40)) return LCE_ERR_UNSUPPORTED;
  // 32-bit buffer offsets: the gathered rows (N x D) and one 256-row chunk of
  // G must each stay within 2 GB.
  const int64_t esz = dt == LCE_DTYPE_BF16 ? 2 : 4;
  if (rup(std::max<int64_t>(N, 1), 256) * D * esz > ((int64_t)1 << 31)) return LCE_ERR_UNSUPPORTED;
  if (rup(std::max<int64_t>(N, 1), 256) * 256 * esz > ((int64_t)1 << 31)) return LCE_ERR_UNSUPPORTED;
  return LCE_OK;
}

lce_status_t make_reduce(int kind, const float* weights, double num, Reduce& r) {
  if (kind != kReduceMean && kind != kReduceSum && kind != kReduceNone) return LCE_ERR_ARG;
  if (!(num >= 0.0) || std::isinf(num)) return LCE_ERR_ARG;  // also rejects NaN
  if (kind != kReduceSum && (weights != nullptr || num != 0.0)) return LCE_ERR_ARG;
  r.kind = kind;
  r.weights = weights;
  r.div = num > 0.0 ? num : 1.0;
  return LCE_OK;
}

// Shared by lce_forward and lce_forward_ex.  `loss` (scalar) and `row_loss`
// ([N]) are each optional; m and logs may be null (no backward follows).
lce_status_t forward_entry(const void* H, const void* W, const void* b, const int64_t* labels,
                           const int32_t* valid_idx, int64_t C, int64_t N, int64_t D, int64_t V,
                           lce_dtype_t dt, const Reduce& red, float* loss, float* m, float* logs,
                           float* row_loss, void* ws, size_t ws_bytes, void* stream, int64_t label_off = 0,
                           float* shard_part = nullptr) {
  try {
    if (!dims_ok(N, D, V, dt) || C < 0 || C > N) return LCE_ERR_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (C == 0) {
      if (loss) LCE_LAUNCH("k_store_scalar", k_store_scalar, 1, 1, 0, s, loss, 0.f);
      LCE_TRY(fill_stats(m, logs, row_loss, N, s));
      return LCE_OK_EMPTY;
    }
    if (!H || !W || !labels || !valid_idx || !ws) return LCE_ERR_ARG;
    if (!aligned16(H) || !aligned16(W) || !aligned16(ws)) return LCE_ERR_ARG;
    LCE_TRY(shape_supported(N, D, V, dt));
    Layout L;
    if (!make_layout(N, D, V, dt, L)) return LCE_ERR_ARG;
    if (ws_bytes < L.fwd_total) return LCE_ERR_WORKSPACE;
    char* w = static_cast<char*>(ws);
    if (dt == LCE_DTYPE_BF16)
      return forward_impl<uint16_t>((const uint16_t*)H, (const uint16_t*)W, (const uint16_t*)b, labels,
                                    valid_idx, C, N, D, V, label_off, red, loss, m, logs, row_loss, shard_part, w,
                                    L, s);
    return forward_impl<float>((const float*)H, (const float*)W, (const float*)b, labels, valid_idx, C,
                               N, D, V, label_off, red, loss, m, logs, row_loss, shard_part, w, L, s);
  } catch (...) {
    return LCE_ERR_HIP;
  }
}

// Shared by lce_backward and lce_backward_ex.
lce_status_t backward_entry(const void* H, const void* W, const void* b, const int64_t* labels,
                            const int32_t* valid_idx, int64_t C, int64_t N, int64_t D, int64_t V,
                            lce_dtype_t dt, const Reduce& red, const float* m, const float* logs,
                            const float* grad_loss, void* dH, void* dW, void* db, void* ws,
                            size_t ws_bytes, void* stream, int64_t label_off = 0, float filter_eps = -1.f,
                            int filter_which = 0) {
  try {
    if (!dims_ok(N, D, V, dt) || C < 0 || C > N) return LCE_ERR_ARG;
    if (!dW || (N > 0 && !dH)) return LCE_ERR_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t esz = dt == LCE_DTYPE_BF16 ? 2 : 4;
    if (C == 0) {
      LCE_TRY(zero_bytes(dH, N * D * esz, s));
      LCE_TRY(zero_bytes(dW, V * D * esz, s));
      LCE_TRY(zero_bytes(db, V * esz, s));
      return LCE_OK_EMPTY;
    }
    if (!H || !W || !labels || !valid_idx || !m || !logs || !ws) return LCE_ERR_ARG;
    if (!aligned16(H) || !aligned16(W) || !aligned16(ws) || !aligned16(dH) || !aligned16(dW))
      return LCE_ERR_ARG;
    LCE_TRY(shape_supported(N, D, V, dt));
    Layout L;
    if (!make_layout(N, D, V, dt, L, C)) return LCE_ERR_ARG;
    if (ws_bytes < L.total) return LCE_ERR_WORKSPACE;
    char* w = static_cast<char*>(ws);
    if (dt == LCE_DTYPE_BF16)
      return backward_impl<uint16_t>((const uint16_t*)H, (const uint16_t*)W, (const uint16_t*)b, labels,
                                     valid_idx, C, N, D, V, label_off, red, m, logs, grad_loss, (uint16_t*)dH,
                                     (uint16_t*)dW, (uint16_t*)db, w, L, s, filter_eps,
                                     filter_which);
    if (filter_eps >= 0.f) return LCE_ERR_UNSUPPORTED;  // the filter runs on the bf16 path only
    return backward_impl<float>((const float*)H, (const float*)W, (const float*)b, labels, valid_idx, C,
                                N, D, V, label_off, red, m, logs, grad_loss, (float*)dH, (float*)dW, (float*)db, w,
                                L, s);
  } catch (...) {
    return LCE_ERR_HIP;
  }
}

// ------------------------------------------------------------------ static scratch
// The no-allocation entry's workspace: a file-scope device array that every
// device the library runs on holds until the process ends.  Host code never
// passes the array's name to a kernel (on the host it is only a stand-in for
// the symbol): the device address of each device's copy is resolved once, on
// the first call on that device, with that device current.
constexpr size_t kScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;  // per device: the address of its `scratch`

lce_status_t scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return LCE_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if ((size_t)dev >= g_scratch_ptr.size()) g_scratch_ptr.resize((size_t)dev + 1, nullptr);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return LCE_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LCE_OK;
}

}  // namespace

// ====================================================================== C ABI
extern "C" {

size_t lce_workspace_size(int64_t N, int64_t D, int64_t V, lce_dtype_t dt) {
  Layout L;
  if (!make_layout(N, D, V, dt, L)) return 0;
  return L.total;
}

size_t lce_backward_workspace_size(int64_t N, int64_t C, int64_t D, int64_t V, lce_dtype_t dt) {
  Layout L;
  if (C < 0 || !make_layout(N, D, V, dt, L, C)) return 0;
  return L.total;
}

size_t lce_forward_workspace_size(int64_t N, int64_t D, int64_t V, lce_dtype_t dt) {
  Layout L;
  if (!make_layout(N, D, V, dt, L)) return 0;
  return L.fwd_total;
}

const char* lce_status_string(lce_status_t st) {
  switch (st) {
    case LCE_OK: return "ok";
    case LCE_OK_EMPTY: return "ok: no supervised positions (C == 0); zero loss and gradients";
    case LCE_ERR_ARG: return "invalid argument";
    case LCE_ERR_LABEL: return "a supervised label lies outside [0, V)";
    case LCE_ERR_WORKSPACE: return "workspace too small";
    case LCE_ERR_HIP: return "HIP runtime error";
    case LCE_ERR_UNSUPPORTED: return "unsupported shape";
    case LCE_ERR_SCRATCH: return "problem too large for the 64 MiB static scratch of the no-allocation entry";
  }
  return "unknown status";
}

lce_status_t lce_compact_valid(const int64_t* labels, const uint8_t* mask, int64_t N, int64_t V,
                               int64_t ignore_index, int32_t* valid_idx, int64_t* C_host, void* ws,
                               size_t ws_bytes, void* stream) {
  try {
    if (!C_host || N < 0 || V <= 0) return LCE_ERR_ARG;
    if (N > 0 && (!labels || !valid_idx || !ws)) return LCE_ERR_ARG;
    if (N > ((int64_t)1 << 30)) return LCE_ERR_UNSUPPORTED;
    *C_host = 0;
    if (N == 0) return LCE_OK_EMPTY;
    const int64_t nblk = cdiv(N, kCmpBlock);
    const size_t need = a256(nblk * 4) * 3 + 256;
    if (ws_bytes < need || !aligned16(ws)) return LCE_ERR_WORKSPACE;
    // Same offsets as the full layout (its compaction part depends on N only).
    Layout L;
    make_layout(N, 8, 1, LCE_DTYPE_BF16, L);
    char* w = static_cast<char*>(ws);
    int* counts = reinterpret_cast<int*>(w + L.counts);
    int* bad = reinterpret_cast<int*>(w + L.bad);
    int* offsets = reinterpret_cast<int*>(w + L.offsets);
    int* stat = reinterpret_cast<int*>(w + L.stat);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (N <= kCmpOneMax) {
      LCE_LAUNCH("k_cmp_one", k_cmp_one, 1, 1024, 0, s, labels, mask, N, V, ignore_index, valid_idx, stat);
    } else {
      LCE_LAUNCH("k_cmp_count", k_cmp_count, nblk, kCmpBlock, 0, s, labels, mask, N, V, ignore_index,
                 counts, bad);
      LCE_LAUNCH("k_cmp_scan", k_cmp_scan, 1, 1024, 0, s, counts, bad, (int)nblk, offsets, stat);
      LCE_LAUNCH("k_cmp_scatter", k_cmp_scatter, nblk, kCmpBlock, 0, s, labels, mask, N, ignore_index,
                 offsets, valid_idx);
    }
    int host_stat[2] = {0, 0};
    if (hipMemcpyAsync(host_stat, stat, sizeof(host_stat), hipMemcpyDeviceToHost, s) != hipSuccess)
      return LCE_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return LCE_ERR_HIP;
    if (host_stat[1]) return LCE_ERR_LABEL;
    *C_host = host_stat[0];
    return host_stat[0] > 0 ? LCE_OK : LCE_OK_EMPTY;
  } catch (...) {
    return LCE_ERR_HIP;
  }
}

lce_status_t lce_forward(const void* H, const void* W, const void* b, const int64_t* labels,
                         const int32_t* valid_idx, int64_t C, int64_t N, int64_t D, int64_t V,
                         lce_dtype_t dt, float* loss, float* m, float* logs, float* row_loss,
                         void* ws, size_t ws_bytes, void* stream) {
  if (!loss || (N > 0 && (!m || !logs))) return LCE_ERR_ARG;
  return forward_entry(H, W, b, labels, valid_idx, C, N, D, V, dt, Reduce{}, loss, m, logs, row_loss, ws,
                       ws_bytes, stream);
}

lce_status_t lce_forward_ex(const void* H, const void* W, const void* b, const int64_t* labels,
                            const int32_t* valid_idx, int64_t C, int64_t N, int64_t D, int64_t V,
                            lce_dtype_t dt, lce_reduction_t reduction, const float* loss_weights,
                            double num_label_tokens, float* loss, float* m, float* logs, void* ws,
                            size_t ws_bytes, void* stream) {
  Reduce red;
  LCE_TRY(make_reduce(reduction, loss_weights, num_label_tokens, red));
  if (!loss) return LCE_ERR_ARG;
  if (red.kind == kReduceNone)  // per-position losses: loss is float[N]
    return forward_entry(H, W, b, labels, valid_idx, C, N, D, V, dt, red, nullptr, m, logs, loss, ws,
                         ws_bytes, stream);
  return forward_entry(H, W, b, labels, valid_idx, C, N, D, V, dt, red, loss, m, logs, nullptr, ws,
                       ws_bytes, stream);
}

lce_status_t lce_forward_ex_noalloc(const void* H, const void* W, const void* b, const int64_t* labels,
                                    const int32_t* valid_idx, int64_t C, int64_t N, int64_t D, int64_t V,
                                    lce_dtype_t dt, lce_reduction_t reduction, const float* loss_weights,
                                    double num_label_tokens, float* loss, float* m, float* logs, void* stream) {
  try {
    Reduce red;
    LCE_TRY(make_reduce(reduction, loss_weights, num_label_tokens, red));
    if (!loss || !dims_ok(N, D, V, dt) || C < 0 || C > N) return LCE_ERR_ARG;
    // Size check first: a problem whose forward workspace exceeds the scratch
    // is refused before any HIP call.
    Layout L;
    if (!make_layout(N, D, V, dt, L)) return LCE_ERR_ARG;
    if (L.fwd_total > kScratchBytes) return LCE_ERR_SCRATCH;
    void* ws = nullptr;
    LCE_TRY(scratch_address(&ws));
    // The forward kernels write every workspace element they later read
    // (gathered rows, split partials, targets of supervised rows, row CE), so
    // the scratch needs no clearing between calls.
    if (red.kind == kReduceNone)
      return forward_entry(H, W, b, labels, valid_idx, C, N, D, V, dt, red, nullptr, m, logs, loss, ws,
                           kScratchBytes, stream);
    return forward_entry(H, W, b, labels, valid_idx, C, N, D, V, dt, red, loss, m, logs, nullptr, ws, kScratchBytes,
                         stream);
  } catch (...) {
    return LCE_ERR_HIP;
  }
}

lce_status_t lce_backward(const void* H, const void* W, const void* b, const int64_t* labels,
                          const int32_t* valid_idx, int64_t C, int64_t N, int64_t D, int64_t V,
                          lce_dtype_t dt, const float* m, const float* logs, const float* grad_loss,
                          void* dH, void* dW, void* db, void* ws, size_t ws_bytes, void* stream) {
  return backward_entry(H, W, b, labels, valid_idx, C, N, D, V, dt, Reduce{}, m, logs, grad_loss, dH, dW,
                        db, ws, ws_bytes, stream);
}

lce_status_t lce_backward_ex(const void* H, const void* W, const void* b, const int64_t* labels,
                             const int32_t* valid_idx, int64_t C, int64_t N, int64_t D, int64_t V,
                             lce_dtype_t dt, lce_reduction_t reduction, const float* loss_weights,
                             double num_label_tokens, const float* m, const float* logs,
                             const float* grad_loss, void* dH, void* dW, void* db, void* ws,
                             size_t ws_bytes, void* stream) {
  Reduce red;
  LCE_TRY(make_reduce(reduction, loss_weights, num_label_tokens, red));
  return backward_entry(H, W, b, labels, valid_idx, C, N, D, V, dt, red, m, logs, grad_loss, dH, dW, db, ws,
                        ws_bytes, stream);
}

lce_status_t lce_forward_shard(const void* H, const void* W_shard, const void* b_shard, const int64_t* labels,
                               const int32_t* valid_idx, int64_t C, int64_t N, int64_t D, int64_t V_shard,
                               int64_t v_begin, lce_dtype_t dt, float* part, void* ws, size_t ws_bytes,
                               void* stream) {
  if (v_begin < 0 || C < 0 || C > N) return LCE_ERR_ARG;
  if (C == 0) return LCE_OK_EMPTY;  // no rows: no partials
  if (!part) return LCE_ERR_ARG;
  return forward_entry(H, W_shard, b_shard, labels, valid_idx, C, N, D, V_shard, dt, Reduce{}, nullptr, nullptr,
                       nullptr, nullptr, ws, ws_bytes, stream, v_begin, part);
}

lce_status_t lce_merge_shards(const float* parts, int32_t P, const int64_t* shard_begin, const int64_t* labels,
                              const int32_t* valid_idx, int64_t C, int64_t N, lce_reduction_t reduction,
                              const float* loss_weights, double num_label_tokens, float* loss, float* m,
                              float* logs, void* ws, size_t ws_bytes, void* stream) {
  try {
    Reduce red;
    LCE_TRY(make_reduce(reduction, loss_weights, num_label_tokens, red));
    if (N < 0 || C < 0 || C > N || !loss || P < 1 || P > kMaxShards || !shard_begin) return LCE_ERR_ARG;
    ShardBounds bounds{};
    if (shard_begin[0] != 0) return LCE_ERR_ARG;
    for (int p = 0; p <= P; ++p) {
      if (p > 0 && shard_begin[p] <= shard_begin[p - 1]) return LCE_ERR_ARG;
      bounds.b[p] = shard_begin[p];
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    float* row_loss = red.kind == kReduceNone ? loss : nullptr;
    if (C == 0) {
      if (red.kind != kReduceNone) LCE_LAUNCH("k_store_scalar", k_store_scalar, 1, 1, 0, s, loss, 0.f);
      LCE_TRY(fill_stats(m, logs, row_loss, N, s));
      return LCE_OK_EMPTY;
    }
    if (!parts || !labels || !valid_idx || !ws) return LCE_ERR_ARG;
    if (ws_bytes < (size_t)C * sizeof(float)) return LCE_ERR_WORKSPACE;
    float* lrow = static_cast<float*>(ws);
    LCE_TRY(fill_stats(m, logs, row_loss, N, s));
    LCE_LAUNCH("k_merge_shards", k_merge_shards, cdiv(C, 256), 256, 0, s, parts, parts + C, parts + 2 * C, (int)P,
               3 * C, bounds, labels, valid_idx, (int)C, m, logs, row_loss, lrow);
    if (red.kind != kReduceNone)
      LCE_LAUNCH("k_loss_sum", k_loss_sum, 1, 1024, 0, s, lrow, (int)C, (int)red.kind, red.weights, valid_idx,
                 red.div, loss);
    return LCE_OK;
  } catch (...) {
    return LCE_ERR_HIP;
  }
}

lce_status_t lce_backward_shard(const void* H, const void* W_shard, const void* b_shard, const int64_t* labels,
                                const int32_t* valid_idx, int64_t C, int64_t N, int64_t D, int64_t V_shard,
                                int64_t v_begin, lce_dtype_t dt, lce_reduction_t reduction,
                                const float* loss_weights, double num_label_tokens, const float* m,
                                const float* logs, const float* grad_loss, void* dH_part, void* dW_shard,
                                void* db_shard, void* ws, size_t ws_bytes, void* stream) {
  Reduce red;
  LCE_TRY(make_reduce(reduction, loss_weights, num_label_tokens, red));
  if (v_begin < 0) return LCE_ERR_ARG;
  return backward_entry(H, W_shard, b_shard, labels, valid_idx, C, N, D, V_shard, dt, red, m, logs, grad_loss,
                        dH_part, dW_shard, db_shard, ws, ws_bytes, stream, v_begin);
}

lce_status_t lce_backward_filtered(const void* H, const void* W, const void* b, const int64_t* labels,
                                   const int32_t* valid_idx, int64_t C, int64_t N, int64_t D, int64_t V,
                                   lce_dtype_t dt, lce_reduction_t reduction, const float* loss_weights,
                                   double num_label_tokens, const float* m, const float* logs,
                                   const float* grad_loss, float eps, int32_t which, void* dH, void* dW,
                                   void* db, void* ws, size_t ws_bytes, void* stream) {
  Reduce red;
  LCE_TRY(make_reduce(reduction, loss_weights, num_label_tokens, red));
  if (!(eps >= 0.f) || std::isinf(eps)) return LCE_ERR_ARG;
  if (which != LCE_FILTER_DH && which != LCE_FILTER_BOTH) return LCE_ERR_ARG;
  if (dt != LCE_DTYPE_BF16) return dims_ok(N, D, V, dt) ? LCE_ERR_UNSUPPORTED : LCE_ERR_ARG;
  return backward_entry(H, W, b, labels, valid_idx, C, N, D, V, dt, red, m, logs, grad_loss, dH, dW, db, ws,
                        ws_bytes, stream, 0, eps, which);
}

lce_status_t lce_profile_start(int32_t max_launches) {
  try {
    Prof& p = g_prof;
    if (max_launches <= 0) return LCE_ERR_ARG;
    if ((int)p.ev.size() < 2 * max_launches) {
      for (hipEvent_t e : p.ev) (void)hipEventDestroy(e);
      p.ev.assign(2 * (size_t)max_launches, nullptr);
      for (auto& e : p.ev)
        if (hipEventCreate(&e) != hipSuccess) return LCE_ERR_HIP;
    }
    p.kid.assign((size_t)max_launches, -1);
    p.lflops.assign((size_t)max_launches, 0.0);
    p.max = max_launches;
    p.used = 0;
    p.names.clear();
    p.ms.clear();
    p.flops.clear();
    p.cnt.clear();
    p.on = true;
    return LCE_OK;
  } catch (...) {
    return LCE_ERR_HIP;
  }
}

lce_status_t lce_profile_stop(void) {
  Prof& p = g_prof;
  p.on = false;
  for (int i = 0; i < p.used; ++i) {
    float ms = 0.f;
    if (hipEventSynchronize(p.ev[2 * i + 1]) != hipSuccess) return LCE_ERR_HIP;
    if (hipEventElapsedTime(&ms, p.ev[2 * i], p.ev[2 * i + 1]) != hipSuccess) return LCE_ERR_HIP;
    p.ms[p.kid[i]] += ms;
    p.flops[p.kid[i]] += p.lflops[i];
    p.cnt[p.kid[i]] += 1;
  }
  p.used = 0;
  return LCE_OK;
}

int32_t lce_profile_count(void) { return (int32_t)g_prof.names.size(); }

lce_status_t lce_profile_entry(int32_t i, char* name, int32_t name_cap, double* total_ms,
                               int64_t* launches, double* flops) {
  Prof& p = g_prof;
  if (i < 0 || i >= (int32_t)p.names.size()) return LCE_ERR_ARG;
  if (name && name_cap > 0) {
    std::strncpy(name, p.names[i].c_str(), (size_t)name_cap - 1);
    name[name_cap - 1] = 0;
  }
  if (total_ms) *total_ms = p.ms[i];
  if (launches) *launches = p.cnt[i];
  if (flops) *flops = p.flops[i];
  return LCE_OK;
}

}  // extern "C"
