/*
 * lce.h -- C ABI of the fused, chunked linear-cross-entropy library for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (page "分块交叉熵：从输出投影开始省保存量", glenzli.com,
 * section 01 "SAME OBJECTIVE", objective equation):
 *
 *   Z_ij = H_i . W_j + b_j                 H[N,D], W[V,D], b[V] (b = 0 if absent)
 *   a_i  = 1[mask_i] * 1[y_i != ignore]    C = sum_i a_i
 *   L    = (1/C) sum_{a_i=1} ( log sum_j exp(Z_ij) - Z_{i,y_i} )
 *
 * computed in T x B score tiles that never form the N x V logits: the forward
 * pass keeps a running row max m and exp-sum s over vocabulary tiles and
 * captures the target score from the tile that holds it (section 02 "RUNNING
 * LSE"); the backward pass replays every tile, rebuilds
 * p = exp((Z - m) - log s), forms G = (lambda a_i / C)(p - onehot(y)) and
 * returns dH = G W, dW = G^T H, db = sum_i G_i (section 04 "RECONSTRUCT AND
 * SUM").  Prompt rows (label == ignore or mask false) never enter the
 * projection (ChunkedLinearCrossEntropy page, m.nxbn.cn, section on filtering
 * tokens with label -100).
 *
 * Conventions for every call
 *  - Device arrays are contiguous, row-major, 16-byte aligned.  H, W and b
 *    share one element type (lce_dtype_t); the projection runs in that type
 *    with fp32 accumulation, the scores Z and every statistic are fp32.
 *  - D must be a multiple of 8 (bf16) or 4 (fp32).
 *  - The caller owns all memory, including the workspace (size it with
 *    lce_workspace_size for every call, lce_forward_workspace_size for the
 *    compaction and forward calls alone, or lce_backward_workspace_size for
 *    the backward calls once C is known).  A call given fewer bytes than it
 *    needs returns LCE_ERR_WORKSPACE before any HIP call.  The library never
 *    allocates device memory.  Its
 *    only state between calls is a per-device record of the kernel
 *    attributes it has set and the optional profiling switch at the end of
 *    this header.  Inputs are never written.
 *  - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream).
 *    Only lce_compact_valid synchronises the stream (to return C).
 *  - No exception crosses the ABI; every call returns an lce_status_t.
 *  - Calls that share a workspace must not overlap in time.
 */
#ifndef LCE_H_
#define LCE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LCE_DTYPE_F32 = 0,  /* IEEE binary32 */
  LCE_DTYPE_BF16 = 1  /* bfloat16 (8 exponent bits, 7 stored mantissa bits) */
} lce_dtype_t;

typedef enum {
  LCE_OK = 0,
  LCE_OK_EMPTY = 1,        /* C == 0: zero loss sentinel / zero gradients written
                              (section 01: the mean is undefined, the caller
                              should skip the optimizer step) */
  LCE_ERR_ARG = -1,        /* null or inconsistent argument, misaligned pointer */
  LCE_ERR_LABEL = -2,      /* a supervised label lies outside [0, V) */
  LCE_ERR_WORKSPACE = -3,  /* ws_bytes below the size the call needs */
  LCE_ERR_HIP = -4,        /* a HIP runtime call or kernel launch failed */
  LCE_ERR_UNSUPPORTED = -5, /* shape outside the documented limits */
  LCE_ERR_SCRATCH = -6      /* lce_forward_ex_noalloc: the forward workspace
                               of these sizes exceeds its static scratch */
} lce_status_t;

/* Reduction of the per-row cross-entropy l_i = log sum_j exp(Z_ij) - Z_{i,y_i}
 * over the supervised rows (NeMo AutoModel chunked_ce page,
 * ChunkedCrossEntropy.forward: `reduction`, `num_label_tokens`,
 * `loss_weights`):
 *   MEAN  L = (1/C) sum_i l_i                      (the page-2 objective)
 *   SUM   L = (sum_i w_i l_i) / n                  w_i = loss_weights[i] (1 if
 *         NULL), n = num_label_tokens (1 if 0)
 *   NONE  the per-position values l_i (0 on unsupervised positions). */
typedef enum {
  LCE_REDUCTION_MEAN = 0,
  LCE_REDUCTION_SUM = 1,
  LCE_REDUCTION_NONE = 2
} lce_reduction_t;

/* Bytes of device workspace that lce_compact_valid, lce_forward and
 * lce_backward need for these sizes (worst case C = N).  It never grows with
 * N x V: the largest pieces are the gathered supervised rows (N x D), the
 * softmax-gradient tile store (two vocabulary chunks of N x min(V, 32768) for
 * bf16, one for fp32) and the fp32 dH accumulators (at most 4 x N x D).
 * Returns 0 for invalid sizes. */
size_t lce_workspace_size(int64_t N, int64_t D, int64_t V, lce_dtype_t dt);

/* Bytes of device workspace that lce_backward, lce_backward_ex,
 * lce_backward_filtered and lce_backward_shard need when C of the N rows are
 * supervised (0 <= C <= N, the count lce_compact_valid returned): the
 * backward's arrays (two vocabulary chunks of the bf16 softmax-gradient tile
 * store, C x min(V, 32768) each; the fp32 dH accumulators, at most 4 x C x D;
 * the row statistics) take C rows, the gathered rows N.  Never more than
 * lce_workspace_size(N, D, V, dt), which is this size at C = N.  Returns 0
 * for invalid sizes or C outside [0, N]. */
size_t lce_backward_workspace_size(int64_t N, int64_t C, int64_t D, int64_t V, lce_dtype_t dt);

/* Bytes of device workspace that the compaction and forward calls alone need
 * (lce_compact_valid, lce_forward, lce_forward_ex, lce_forward_shard with the
 * shard's V): the gathered supervised rows and the per-split row partials,
 * about N x D elements plus 0.5 KB per position.  A caller can free this
 * buffer after the forward call and allocate the lce_backward_workspace_size
 * buffer only for the backward call, so that nothing beyond m and logs (the two
 * N-vectors that section 02 of the glenzli.com page saves) is held between
 * the passes.  Returns 0 for invalid sizes; never more than
 * lce_workspace_size. */
size_t lce_forward_workspace_size(int64_t N, int64_t D, int64_t V, lce_dtype_t dt);

/* Valid-token compaction (section 01 definition of a_i and C; the
 * ChunkedLinearCrossEntropy page's prompt filtering).
 *   labels       int64[N] device; label of each position.
 *   mask         uint8[N] device or NULL (NULL = every position masked in);
 *                nonzero = supervised.
 *   ignore_index label value that marks an unsupervised position (-100).
 *   valid_idx    int32[N] device, written: the C supervised positions in
 *                ascending order in valid_idx[0..C).  Entries >= C untouched.
 *   C_host       host int64, written: C.
 * Checks on the device that every supervised label lies in [0, V); if not,
 * returns LCE_ERR_LABEL (valid_idx contents then unspecified).
 * Synchronises `stream` once.  Returns LCE_OK, LCE_OK_EMPTY when C == 0. */
lce_status_t lce_compact_valid(const int64_t* labels, const uint8_t* mask, int64_t N,
                               int64_t V, int64_t ignore_index, int32_t* valid_idx,
                               int64_t* C_host, void* ws, size_t ws_bytes, void* stream);

/* Forward pass (sections 01-02).
 *   H [N,D], W [V,D], b [V] or NULL: device, element type dt.
 *   labels int64[N], valid_idx int32[C] (from lce_compact_valid), C, N, D, V.
 *   loss      float[1] device, written: mean CE over the C supervised rows.
 *   m, logs   float[N] device, written: the saved statistics.  For supervised
 *             row i, m[i] = max_j Z_ij and logs[i] = log sum_j exp(Z_ij - m[i]);
 *             unsupervised rows keep the recurrence's initial state
 *             (m = -inf, logs = -inf).
 *   row_loss  float[N] device or NULL; if given, written with the per-row CE
 *             (m - Z_{i,y_i}) + logs for supervised rows and 0 elsewhere.
 * C == 0: loss = 0, m = logs = -inf, row_loss = 0, returns LCE_OK_EMPTY.
 * A NaN score makes the loss NaN (it is never hidden). */
lce_status_t lce_forward(const void* H, const void* W, const void* b, const int64_t* labels,
                         const int32_t* valid_idx, int64_t C, int64_t N, int64_t D, int64_t V,
                         lce_dtype_t dt, float* loss, float* m, float* logs, float* row_loss,
                         void* ws, size_t ws_bytes, void* stream);

/* Backward pass (section 04).
 *   Same H, W, b, labels, valid_idx, C, N, D, V, dt as the forward call, and
 *   the m / logs it wrote.
 *   grad_loss float[1] device or NULL: lambda = dJ/dL (NULL means 1).
 *   dH [N,D], dW [V,D]: device, type dt, fully overwritten (not accumulated);
 *   rows of dH for unsupervised positions are exactly 0.
 *   db [V] device, type dt, or NULL (skip the bias gradient).
 * Deterministic: the same inputs give bitwise-identical outputs (ordered
 * reductions; the only floating-point atomics add into partial sums that
 * have one writer per kernel launch, with launches in a fixed order).
 * C == 0: dH, dW and db are zero-filled, returns LCE_OK_EMPTY.
 *   ws: at least lce_backward_workspace_size(N, C, D, V, dt) bytes (the
 *   lce_workspace_size buffer of the forward call also serves). */
lce_status_t lce_backward(const void* H, const void* W, const void* b, const int64_t* labels,
                          const int32_t* valid_idx, int64_t C, int64_t N, int64_t D, int64_t V,
                          lce_dtype_t dt, const float* m, const float* logs,
                          const float* grad_loss, void* dH, void* dW, void* db, void* ws,
                          size_t ws_bytes, void* stream);

/* Forward pass with a chosen reduction; also the forward-only (evaluation)
 * entry: m and logs may be NULL when no backward call follows.
 *   reduction         see lce_reduction_t.
 *   loss_weights      float[N] device or NULL; per-position weights, SUM only
 *                     (LCE_ERR_ARG with another reduction).
 *   num_label_tokens  SUM only: divisor n > 0, or 0 for none (LCE_ERR_ARG if
 *                     negative, infinite, NaN, or nonzero with MEAN / NONE).
 *   loss              MEAN / SUM: float[1]; NONE: float[N] (per-position l_i,
 *                     0 on unsupervised positions).  Device, written.
 *   m, logs           float[N] device or NULL; as in lce_forward.
 * Other arguments and the C == 0 behaviour (loss 0, LCE_OK_EMPTY) as in
 * lce_forward.  The per-row values are those of lce_forward; the sums are
 * float64 in a fixed order. */
lce_status_t lce_forward_ex(const void* H, const void* W, const void* b, const int64_t* labels,
                            const int32_t* valid_idx, int64_t C, int64_t N, int64_t D, int64_t V,
                            lce_dtype_t dt, lce_reduction_t reduction, const float* loss_weights,
                            double num_label_tokens, float* loss, float* m, float* logs, void* ws,
                            size_t ws_bytes, void* stream);

/* lce_forward_ex without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  The workspace is a static device
 * array of the library, 64 MiB on each device the library runs on, held
 * until the process ends; the call itself allocates nothing.  Sizes whose
 * forward workspace (lce_forward_workspace_size(N, D, V, dt)) exceeds it are
 * refused with LCE_ERR_SCRATCH before any HIP call (e.g. N = 16384, D = 1024
 * fits; N = 32768, D = 4096 does not).  The first call on a device resolves
 * the array's address on that device (hipGetSymbolAddress), so make it
 * outside graph capture.  Every call on one device shares that device's
 * array: calls that overlap in time on one device (different streams or
 * threads) race and must be serialised by the caller.  The arrays keep the
 * last call's contents; no call reads what an earlier one left.  Arguments,
 * outputs and statuses otherwise as for lce_forward_ex, whose kernels it
 * runs (the results are bit for bit those of lce_forward_ex). */
lce_status_t lce_forward_ex_noalloc(const void* H, const void* W, const void* b, const int64_t* labels,
                                    const int32_t* valid_idx, int64_t C, int64_t N, int64_t D, int64_t V,
                                    lce_dtype_t dt, lce_reduction_t reduction, const float* loss_weights,
                                    double num_label_tokens, float* loss, float* m, float* logs, void* stream);

/* Backward pass for a chosen reduction (section 04 with the row factor of
 * that reduction): G_ij = r_i (p_ij - 1[j = y_i]) on supervised rows, with
 *   MEAN  r_i = lambda / C,  SUM  r_i = lambda w_i / n,  NONE  r_i = g_i,
 * where lambda = grad_loss[0] (MEAN / SUM; NULL means 1) and g = grad_loss
 * float[N] (NONE: the upstream gradient of each position's loss; NULL means
 * 1 for every position).  reduction, loss_weights and num_label_tokens must
 * be those of the forward call.  Outputs, determinism and the C == 0
 * behaviour as in lce_backward. */
lce_status_t lce_backward_ex(const void* H, const void* W, const void* b, const int64_t* labels,
                             const int32_t* valid_idx, int64_t C, int64_t N, int64_t D, int64_t V,
                             lce_dtype_t dt, lce_reduction_t reduction, const float* loss_weights,
                             double num_label_tokens, const float* m, const float* logs,
                             const float* grad_loss, void* dH, void* dW, void* db, void* ws,
                             size_t ws_bytes, void* stream);

/* Which gradients lce_backward_filtered filters.  The glenzli.com page,
 * section 07, names CCE's embedding-gradient (dH) and classifier-gradient
 * (dW) filters and the variants that turn off the classifier filter, or
 * both (the exact gradient: lce_backward_ex). */
typedef enum {
  LCE_FILTER_DH = 1,   /* embedding gradient only; dW exact */
  LCE_FILTER_BOTH = 3  /* embedding and classifier gradients */
} lce_filter_t;

/* Backward with gradient filtering (the threshold filter of CCE that the
 * glenzli.com page, section 07, describes as an approximation of the full
 * gradient): the supervised rows, in ascending position order, are cut into
 * blocks of 256 and the vocabulary into blocks of 32; a block of G in which
 * every entry of a row with r_i != 0 has p_ij < eps, and which holds no
 * row's target column, is skipped by the products that `which` selects
 * (dH, or dH and dW).  db keeps every contribution.  eps = 0 skips only blocks
 * of exact zeros, so the result is that of lce_backward_ex bit for bit.
 * bf16 only (LCE_ERR_UNSUPPORTED for fp32); eps must be finite and >= 0 and
 * `which` one of lce_filter_t (else LCE_ERR_ARG).  Other arguments as for
 * lce_backward_ex. */
lce_status_t lce_backward_filtered(const void* H, const void* W, const void* b, const int64_t* labels,
                                   const int32_t* valid_idx, int64_t C, int64_t N, int64_t D, int64_t V,
                                   lce_dtype_t dt, lce_reduction_t reduction, const float* loss_weights,
                                   double num_label_tokens, const float* m, const float* logs,
                                   const float* grad_loss, float eps, int32_t which, void* dH, void* dW,
                                   void* db, void* ws, size_t ws_bytes, void* stream);

/* ---- Vocabulary sharding on one device --------------------------------------
 * The exchange that splitting W over P devices needs (glenzli.com page,
 * section 02: the running (m, s) of disjoint vocabulary ranges merge exactly;
 * AIInfraGuide chapter 2, the online-softmax merge): each shard computes
 * per-row partials over its own vocabulary range, one merge combines them in
 * shard order, and each shard's backward uses the merged statistics.  Here
 * the shards run one after another on one device; across devices the parts
 * would travel by an all-gather and the dH partials would be summed by an
 * all-reduce. */

/* Forward partials of one vocabulary shard: rows [v_begin, v_begin + V_shard)
 * of the full W.
 *   W_shard [V_shard, D], b_shard [V_shard] or NULL: device, type dt.
 *   labels, valid_idx, C, N, D: as for lce_forward (labels are full-vocabulary
 *            ids; labels outside the shard simply match no column here).
 *   part     float[3*C] device, written: part[c] = m_c, part[C + c] = s_c
 *            (exp-sum relative to m_c) over the shard's entries, and
 *            part[2C + c] = the score of the row's target when its label lies
 *            in the shard, else 0.
 *   ws       workspace of lce_workspace_size(N, D, V_shard, dt) bytes.
 * C == 0: returns LCE_OK_EMPTY and writes nothing. */
lce_status_t lce_forward_shard(const void* H, const void* W_shard, const void* b_shard, const int64_t* labels,
                               const int32_t* valid_idx, int64_t C, int64_t N, int64_t D, int64_t V_shard,
                               int64_t v_begin, lce_dtype_t dt, float* part, void* ws, size_t ws_bytes,
                               void* stream);

/* Merge of P shard partials (shard order) into the loss and the statistics.
 *   parts        float[P][3*C] device: the `part` outputs of the P shards.
 *   P            1..64 shards.
 *   shard_begin  host int64[P+1]: shard p covers labels [shard_begin[p],
 *                shard_begin[p+1]); shard_begin[0] = 0, strictly increasing,
 *                shard_begin[P] = V.
 *   reduction, loss_weights, num_label_tokens, loss, m, logs: as for
 *                lce_forward_ex (m, logs may be NULL).
 *   ws           device scratch of at least 4*C bytes.
 * C == 0: loss 0 (zeros for NONE), m = logs = -inf, LCE_OK_EMPTY. */
lce_status_t lce_merge_shards(const float* parts, int32_t P, const int64_t* shard_begin, const int64_t* labels,
                              const int32_t* valid_idx, int64_t C, int64_t N, lce_reduction_t reduction,
                              const float* loss_weights, double num_label_tokens, float* loss, float* m,
                              float* logs, void* ws, size_t ws_bytes, void* stream);

/* Backward of one vocabulary shard from the merged m / logs: dW_shard
 * [V_shard, D] and db_shard [V_shard] (or NULL) of the shard's rows, and
 * dH_part [N, D], this shard's share of dH (the sum over shards is dH).
 * Other arguments as for lce_backward_ex; ws as for lce_forward_shard. */
lce_status_t lce_backward_shard(const void* H, const void* W_shard, const void* b_shard, const int64_t* labels,
                                const int32_t* valid_idx, int64_t C, int64_t N, int64_t D, int64_t V_shard,
                                int64_t v_begin, lce_dtype_t dt, lce_reduction_t reduction,
                                const float* loss_weights, double num_label_tokens, const float* m,
                                const float* logs, const float* grad_loss, void* dH_part, void* dW_shard,
                                void* db_shard, void* ws, size_t ws_bytes, void* stream);

/* Static string for a status code. */
const char* lce_status_string(lce_status_t status);

/* ---- Optional kernel timing (benchmarks only; not thread-safe) -------------
 * lce_profile_start(max_launches) makes every following launch record a HIP
 * event pair on its stream (up to max_launches launches); lce_profile_stop()
 * synchronises those events and folds them into per-kernel totals, and turns
 * recording off.  lce_profile_count() gives the number of distinct kernels
 * seen; lce_profile_entry(i, ...) copies kernel i's name, total milliseconds,
 * launch count and total algorithmic flops (any output pointer may be null).
 * The flops of a launch are those of the method's products it computes:
 * 2 C D V_k for the logits of the C supervised rows over a vocabulary range
 * of V_k entries (k_fwd, k_replay), 4 C D V_k for the dH and dW products of
 * a chunk (k_grad), the sum of both for k_grad_replay, and 0 for the kernels
 * outside the GEMMs.  Returns LCE_ERR_HIP if an event call fails. */
lce_status_t lce_profile_start(int32_t max_launches);
lce_status_t lce_profile_stop(void);
int32_t lce_profile_count(void);
lce_status_t lce_profile_entry(int32_t i, char* name, int32_t name_cap, double* total_ms,
                               int64_t* launches, double* flops);

#ifdef __cplusplus
}
#endif

#endif /* LCE_H_ */
