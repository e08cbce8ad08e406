"""Float64 CPU oracle for the fused linear-cross-entropy (LM-head projection + CE).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and its
Python binding) imports, calls or links this file; only the tests, the smoke
check and the CPU-baseline leg of the benchmark do.  It shares no code with the
HIP path.

What it computes (page "分块交叉熵：从输出投影开始省保存量", glenzli.com, section
01 "SAME OBJECTIVE", the objective equation):

    Z_ij = H_i W_j^T + b_j            (b = 0 when there is no bias)
    a_i  = 1[mask_i] * 1[y_i != ignore]     C = sum_i a_i
    L    = (1/C) * sum_{i: a_i = 1} ( log sum_{j<V} exp(Z_ij) - Z_{i,y_i} ),  C > 0

and its first-order gradients (same page, section 04 "RECONSTRUCT AND SUM"):

    p_ij = exp((Z_ij - m_i) - log s_i)
    G_ij = (lambda * a_i / C) * (p_ij - 1[j = y_i])
    dH = G W,   dW = G^T H,   db = sum_i G_i

The chunked method reaches the dense result exactly up to rounding order
(section 02 "RUNNING LSE", the proof that the online statistic equals the
full LSE), so the dense definition is the reference.  ``dense_*`` below is
that definition written out with a textbook max-shifted two-pass log-sum-exp
(AIInfraGuide chapter 2, section 5.3 "LogSumExp").  ``tiled_*`` follows the
page's own tile algorithm (sections 01-04: project a T x B score tile, update
the running (m, s), capture the target from its own tile, replay the tile in
backward) and exists to pin the merge identity and the page's two fault modes;
it is never the reference.

Readings where the pages leave a step open (each also listed in the design
notes of the repository):

* A missing mask means every position is masked in (the NeMo chunked_ce page
  makes the mask optional; zero positions are ignored).
* Supervised labels outside [0, V) are an error, never clamped; unsupervised
  rows may hold any label value.
* m and log s are returned as length-N vectors; unsupervised rows keep the
  recurrence's initial state m = -inf, s = 0, i.e. log s = -inf.
* C = 0: loss 0.0, m = log s = -inf everywhere, all gradients exactly zero
  (section 01, the C=0 sentinel rule).
* lambda is the upstream gradient dJ/dL; the loss value does not depend on it
  (section 04).
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import numpy as np

IGNORE_INDEX = -100


class LabelError(ValueError):
    """A supervised label lies outside [0, V)."""


@dataclass
class ForwardResult:
    loss: float                 # mean CE over the C supervised rows (0.0 when C = 0)
    m: np.ndarray               # [N] row max of Z (-inf on unsupervised rows)
    logs: np.ndarray            # [N] log of the exp-sum relative to m (-inf on unsupervised rows)
    row_loss: np.ndarray        # [N] per-row CE (0.0 on unsupervised rows)
    idx: np.ndarray             # [C] ascending indices of supervised rows
    C: int
    empty: bool                 # True when C = 0 (the zero sentinel case)


@dataclass
class BackwardResult:
    dH: np.ndarray              # [N, D]
    dW: np.ndarray              # [V, D]
    db: np.ndarray              # [V]


def _f64(x) -> Optional[np.ndarray]:
    if x is None:
        return None
    return np.asarray(x, dtype=np.float64)


def supervised_rows(labels, mask=None, ignore_index: int = IGNORE_INDEX):
    """a_i = 1[mask_i] 1[y_i != ignore]; returns (a, idx ascending, C).

    Page glenzli.com chunked-cross-entropy, section 01, definition of a_i and C.
    """
    y = np.asarray(labels, dtype=np.int64)
    a = y != ignore_index
    if mask is not None:
        a = a & np.asarray(mask, dtype=bool)
    idx = np.flatnonzero(a).astype(np.int64)
    return a, idx, int(idx.size)


def check_labels(labels, idx, V: int) -> None:
    y = np.asarray(labels, dtype=np.int64)[idx]
    if y.size and (y.min() < 0 or y.max() >= V):
        raise LabelError("a supervised label lies outside [0, V)")


def logits(H_rows, W, b=None) -> np.ndarray:
    """Z = H W^T + b over the full vocabulary (section 01, objective)."""
    Z = np.asarray(H_rows, dtype=np.float64) @ np.asarray(W, dtype=np.float64).T
    if b is not None:
        Z = Z + np.asarray(b, dtype=np.float64)[None, :]
    return Z


def lse_two_pass(Z: np.ndarray):
    """Row max M and log of sum_j exp(Z_j - M) (textbook stable LSE).

    AIInfraGuide chapter 2, section 5.3: LSE(z) = m + log sum exp(z - m).
    np.max propagates NaN, so a NaN score makes the row's statistics NaN.
    """
    M = np.max(Z, axis=1)
    S = np.sum(np.exp(Z - M[:, None]), axis=1)
    return M, np.log(S)


def _row_blocks(C: int, row_block: Optional[int]):
    step = C if not row_block else row_block
    for lo in range(0, C, max(step, 1)):
        yield lo, min(C, lo + step)


def dense_forward(H, W, b, labels, mask=None, ignore_index: int = IGNORE_INDEX,
                  row_block: Optional[int] = None) -> ForwardResult:
    """Mean CE over supervised rows, with the saved statistics m and log s.

    Rows are independent in the objective, so ``row_block`` (if given) only
    bounds memory by evaluating the same per-row definition a slice at a time.
    """
    H = _f64(H)
    W = _f64(W)
    b = _f64(b)
    N = H.shape[0]
    V = W.shape[0]
    a, idx, C = supervised_rows(labels, mask, ignore_index)
    check_labels(labels, idx, V)
    y = np.asarray(labels, dtype=np.int64)
    m = np.full(N, -np.inf)
    logs = np.full(N, -np.inf)
    row_loss = np.zeros(N)
    if C == 0:
        return ForwardResult(0.0, m, logs, row_loss, idx, 0, True)
    for lo, hi in _row_blocks(C, row_block):
        rows = idx[lo:hi]
        Z = logits(H[rows], W, b)
        M, LS = lse_two_pass(Z)
        zy = Z[np.arange(rows.size), y[rows]]
        m[rows] = M
        logs[rows] = LS
        # l_i = (m_i - Z_{i,y_i}) + log s_i  (section 02: avoids cancellation
        # under a large common shift).
        row_loss[rows] = (M - zy) + LS
    loss = math.fsum(row_loss[idx].tolist()) / C
    return ForwardResult(loss, m, logs, row_loss, idx, C, False)


def reduce_rows(row_loss, idx, C: int, reduction: str = "mean", loss_weights=None,
                num_label_tokens: Optional[float] = None):
    """The loss under one of the reductions of the NeMo AutoModel chunked_ce
    page (ChunkedCrossEntropy.forward: `reduction`, `num_label_tokens`, which
    divides a sum-reduced loss, and `loss_weights`, constant multipliers for
    the sum only):

        mean: (1/C) sum_{i in idx} l_i           (glenzli.com section 01 objective)
        sum:  (sum_{i in idx} w_i l_i) / n       w = 1 without weights,
                                                 n = num_label_tokens (1 if None)
        none: l_i per position (0 on unsupervised positions)
    """
    row_loss = np.asarray(row_loss, dtype=np.float64)
    if reduction == "none":
        out = np.zeros_like(row_loss)
        out[idx] = row_loss[idx]
        return out
    if C == 0:
        return 0.0
    if reduction == "mean":
        return math.fsum(row_loss[idx].tolist()) / C
    if reduction == "sum":
        w = np.ones_like(row_loss) if loss_weights is None else np.asarray(loss_weights, dtype=np.float64)
        total = math.fsum((w[idx] * row_loss[idx]).tolist())
        return total / num_label_tokens if num_label_tokens else total
    raise ValueError(f"unknown reduction {reduction!r}")


def row_factors(N: int, idx, C: int, reduction: str = "mean", grad=1.0, loss_weights=None,
                num_label_tokens: Optional[float] = None) -> np.ndarray:
    """r_i = dJ/dl_i on supervised rows (0 elsewhere), for J = grad * L with
    the mean or sum reduction above, or J = sum_i grad_i l_i for "none"
    (grad then holds one upstream value per position).  With dl_i/dZ_ij =
    p_ij - 1[j = y_i] (glenzli.com section 04; AIInfraGuide section 6.6), the
    score gradient of row i is r_i (p_i - onehot(y_i)).
    """
    r = np.zeros(N)
    if C == 0:
        return r
    if reduction == "none":
        g = np.broadcast_to(np.asarray(grad, dtype=np.float64), (N,))
        r[idx] = g[idx]
    elif reduction == "mean":
        r[idx] = float(grad) / C
    elif reduction == "sum":
        w = np.ones(N) if loss_weights is None else np.asarray(loss_weights, dtype=np.float64)
        r[idx] = float(grad) * w[idx] / (num_label_tokens if num_label_tokens else 1.0)
    else:
        raise ValueError(f"unknown reduction {reduction!r}")
    return r


def dense_backward(H, W, b, labels, m, logs, lam: float = 1.0, mask=None,
                   ignore_index: int = IGNORE_INDEX,
                   row_block: Optional[int] = None,
                   row_factor: Optional[np.ndarray] = None) -> BackwardResult:
    """dH, dW, db of lam * L (section 04 and AIInfraGuide section 6.6).

    p is rebuilt from the saved statistics as exp((Z - m) - log s); the target
    column gets -1; rows are scaled by lam / C, or by row_factor[i] (a
    per-position array from row_factors) when it is given.
    """
    H = _f64(H)
    W = _f64(W)
    b = _f64(b)
    N, D = H.shape
    V = W.shape[0]
    a, idx, C = supervised_rows(labels, mask, ignore_index)
    check_labels(labels, idx, V)
    y = np.asarray(labels, dtype=np.int64)
    dH = np.zeros((N, D))
    dW = np.zeros((V, D))
    db = np.zeros(V)
    if C == 0:
        return BackwardResult(dH, dW, db)
    scale = lam / C
    for lo, hi in _row_blocks(C, row_block):
        rows = idx[lo:hi]
        Z = logits(H[rows], W, b)
        P = np.exp((Z - m[rows][:, None]) - logs[rows][:, None])
        P[np.arange(rows.size), y[rows]] -= 1.0
        G = scale * P if row_factor is None else np.asarray(row_factor, dtype=np.float64)[rows][:, None] * P
        dH[rows] = G @ W
        dW += G.T @ H[rows]
        db += G.sum(axis=0)
    return BackwardResult(dH, dW, db)


def _block_kept(P_block, y_rows, r_rows, v0: int, v1: int, eps: float) -> bool:
    """The filter's decision for one block (rows y_rows, columns [v0, v1),
    probabilities P_block): kept if some row's target column lies in it, or
    if some row with a non-zero factor has p >= eps there."""
    if np.any((y_rows >= v0) & (y_rows < v1)):
        return True
    weighted = r_rows != 0.0
    return bool(np.any(weighted) and np.max(P_block[weighted]) >= eps)


def filtered_backward(H, W, b, labels, m, logs, eps: float, lam: float = 1.0, mask=None,
                      ignore_index: int = IGNORE_INDEX, row_block: int = 256,
                      col_block: int = 32,
                      row_factor: Optional[np.ndarray] = None,
                      filter_dh: bool = True, filter_dw: bool = True) -> BackwardResult:
    """Gradient filtering of small-probability blocks (the CCE threshold
    filter that glenzli.com section 07 describes as an approximation of the
    full gradient).  Reading of the pages: the supervised rows, in ascending
    position order, are cut into blocks of `row_block` rows and the
    vocabulary into blocks of `col_block` entries; a block whose
    probabilities p_ij are all below `eps` and which holds no row's target
    column contributes nothing to dH and dW.  db keeps every contribution.
    eps = 0 keeps every block (the exact gradient).  Rows are scaled by
    lam / C, or by row_factor[i] (from row_factors) when it is given; a row
    whose factor is 0 has a zero gradient row, and its probabilities keep no
    block alive (its target column still does).  Section 07 names the
    embedding-gradient (dH) and classifier-gradient (dW) filters separately;
    filter_dh / filter_dw switch each one, the other gradient being exact.
    """
    H = _f64(H)
    W = _f64(W)
    b = _f64(b)
    N, D = H.shape
    V = W.shape[0]
    a, idx, C = supervised_rows(labels, mask, ignore_index)
    check_labels(labels, idx, V)
    y = np.asarray(labels, dtype=np.int64)
    dH = np.zeros((N, D))
    dW = np.zeros((V, D))
    db = np.zeros(V)
    if C == 0:
        return BackwardResult(dH, dW, db)
    r = np.full(N, lam / C) if row_factor is None else np.asarray(row_factor, dtype=np.float64)
    for lo in range(0, C, row_block):
        rows = idx[lo:lo + row_block]
        Z = logits(H[rows], W, b)
        P = np.exp((Z - m[rows][:, None]) - logs[rows][:, None])
        G = P.copy()
        G[np.arange(rows.size), y[rows]] -= 1.0
        G *= r[rows][:, None]
        db += G.sum(axis=0)
        keep = np.zeros_like(G)
        for v0 in range(0, V, col_block):
            v1 = min(V, v0 + col_block)
            if _block_kept(P[:, v0:v1], y[rows], r[rows], v0, v1, eps):
                keep[:, v0:v1] = 1.0
        Gf = G * keep
        dH[rows] = (Gf if filter_dh else G) @ W
        dW += (Gf if filter_dw else G).T @ H[rows]
    return BackwardResult(dH, dW, db)


def filtered_rows_grad(H, W, b, labels, m, logs, eps: float, rows, cols, lam: float = 1.0, mask=None,
                       ignore_index: int = IGNORE_INDEX, row_block: int = 256, col_block: int = 32):
    """Chosen rows of dH (positions `rows`, all supervised) and of dW
    (vocabulary entries `cols`) of filtered_backward (both gradients
    filtered, rows scaled by lam / C), for checks at sizes where the whole
    filtered gradient is out of reach.  Only the row blocks that hold a
    chosen row, and the column blocks that hold a chosen entry, are
    projected.  Also returns the decision margin: the smallest
    |log(max p / eps)| over the blocks decided by probability alone (inf if
    none), which tells how far every such decision sits from the threshold.
    """
    H = _f64(H)
    W = _f64(W)
    b = _f64(b)
    a, idx, C = supervised_rows(labels, mask, ignore_index)
    check_labels(labels, idx, W.shape[0])
    y = np.asarray(labels, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    assert np.all(a[rows]), "chosen rows must be supervised"
    rank = np.full(H.shape[0], -1, dtype=np.int64)
    rank[idx] = np.arange(C)
    r = np.full(H.shape[0], lam / C)
    margin = np.inf

    def decide(P_block, blk, v0, v1):
        nonlocal margin
        kept = _block_kept(P_block, y[blk], r[blk], v0, v1, eps)
        if not np.any((y[blk] >= v0) & (y[blk] < v1)) and eps > 0:
            margin = min(margin, abs(np.log(np.max(P_block) / eps)))
        return kept

    V = W.shape[0]
    dH_rows = np.zeros((rows.size, H.shape[1]))
    for q in np.unique(rank[rows] // row_block):
        blk = idx[q * row_block:(q + 1) * row_block]
        P = np.exp((logits(H[blk], W, b) - m[blk][:, None]) - logs[blk][:, None])
        live = np.zeros(V, dtype=bool)
        for v0 in range(0, V, col_block):
            v1 = min(V, v0 + col_block)
            live[v0:v1] = decide(P[:, v0:v1], blk, v0, v1)
        for k in np.flatnonzero(rank[rows] // row_block == q):
            i = int(rank[rows[k]]) - q * row_block
            g = P[i].copy()
            g[y[blk[i]]] -= 1.0
            dH_rows[k] = r[blk[i]] * (np.where(live, g, 0.0) @ W)
    dW_rows = np.zeros((cols.size, H.shape[1]))
    for k, v in enumerate(cols):
        v0 = (int(v) // col_block) * col_block
        v1 = min(V, v0 + col_block)
        for lo in range(0, C, row_block):
            blk = idx[lo:lo + row_block]
            bb = None if b is None else b[v0:v1]
            P = np.exp((logits(H[blk], W[v0:v1], bb) - m[blk][:, None]) - logs[blk][:, None])
            if decide(P, blk, v0, v1):
                g = P[:, int(v) - v0] - (y[blk] == v)
                dW_rows[k] += (r[blk] * g) @ H[blk]
    return dH_rows, dW_rows, margin


def dense_forward_backward(H, W, b, labels, mask=None, lam: float = 1.0,
                           ignore_index: int = IGNORE_INDEX,
                           row_block: Optional[int] = None):
    f = dense_forward(H, W, b, labels, mask, ignore_index, row_block)
    g = dense_backward(H, W, b, labels, f.m, f.logs, lam, mask, ignore_index, row_block)
    return f, g


def rows_forward(H_rows, W, b, y_rows):
    """Per-row (m, log s, CE) for a handful of rows, one row at a time.

    Used to check full-size runs at sampled rows: each row's statistics depend
    only on that row (section 01, the objective is a sum over rows).
    """
    H_rows = _f64(H_rows)
    out_m, out_ls, out_l = [], [], []
    for r in range(H_rows.shape[0]):
        z = logits(H_rows[r:r + 1], W, b)
        M, LS = lse_two_pass(z)
        out_m.append(M[0])
        out_ls.append(LS[0])
        out_l.append((M[0] - z[0, int(y_rows[r])]) + LS[0])
    return np.array(out_m), np.array(out_ls), np.array(out_l)


def rows_grad_h(H_rows, W, b, y_rows, scale: float):
    """dH rows = scale * (p - onehot(y)) W for a handful of rows."""
    H_rows = _f64(H_rows)
    W = _f64(W)
    out = np.zeros_like(H_rows)
    for r in range(H_rows.shape[0]):
        z = logits(H_rows[r:r + 1], W, b)
        M, LS = lse_two_pass(z)
        p = np.exp((z[0] - M[0]) - LS[0])
        p[int(y_rows[r])] -= 1.0
        out[r] = scale * (p @ W)
    return out


def cols_grad(H, W, b, labels, m, logs, cols, lam: float = 1.0, mask=None,
              ignore_index: int = IGNORE_INDEX, row_block: Optional[int] = None,
              row_factor: Optional[np.ndarray] = None):
    """Rows `cols` of dW and entries `cols` of db (glenzli.com section 04:
    dW_j = sum_i G_ij H_i, db_j = sum_i G_ij) from the saved statistics m and
    log s of every supervised row, for checks at sizes where the whole dW is
    out of reach: only the score columns Z[:, cols] are formed.  Rows are
    scaled by lam / C, or by row_factor[i] when it is given."""
    H = _f64(H)
    W = _f64(W)
    b = _f64(b)
    cols = np.asarray(cols, dtype=np.int64)
    a, idx, C = supervised_rows(labels, mask, ignore_index)
    check_labels(labels, idx, W.shape[0])
    y = np.asarray(labels, dtype=np.int64)
    dW = np.zeros((cols.size, H.shape[1]))
    db = np.zeros(cols.size)
    if C == 0:
        return dW, db
    Wc = W[cols]
    bc = None if b is None else b[cols]
    for lo, hi in _row_blocks(C, row_block):
        rows = idx[lo:hi]
        Z = logits(H[rows], Wc, bc)
        P = np.exp((Z - m[rows][:, None]) - logs[rows][:, None])
        P -= (y[rows][:, None] == cols[None, :]).astype(np.float64)
        r = np.full(rows.size, lam / C) if row_factor is None else np.asarray(row_factor, dtype=np.float64)[rows]
        G = r[:, None] * P
        dW += G.T @ H[rows]
        db += G.sum(axis=0)
    return dW, db


def tiled_forward_backward(H, W, b, labels, mask=None, lam: float = 1.0, T: int = 16,
                           B: int = 256, ignore_index: int = IGNORE_INDEX, _fault: str = ""):
    """The page's tile algorithm in float64 (pins the merge identity only).

    Forward (section 01 FORWARD/PROJECT and REDUCE/CAPTURE, section 02
    recurrence): for each position tile and each vocabulary tile, project the
    T x B score tile, then
        m' = max(m, max_B Z),  s' = e^(m - m') s + sum_B e^(Z - m'),
    with the first tile's rescale factor defined as 0, and capture the target
    score from the tile that holds y_i, using the global column id.
    Backward (section 04): replay every tile, p = exp((Z - m) - log s),
    subtract 1 at the target, dH_T += G W_B, dW_B += G^T H_T, db_B += sum_T G.

    ``_fault`` plants one of the page's two fault modes, for negative controls
    in the tests only:
      "local_norm"   each vocabulary tile normalised on its own (section 04);
      "dh_overwrite" dH_T written instead of accumulated (section 04).
    """
    H = _f64(H)
    W = _f64(W)
    b = _f64(b)
    N, D = H.shape
    V = W.shape[0]
    a, idx, C = supervised_rows(labels, mask, ignore_index)
    check_labels(labels, idx, V)
    y = np.asarray(labels, dtype=np.int64)
    m = np.full(N, -np.inf)
    s = np.zeros(N)
    target = np.full(N, np.nan)
    dH = np.zeros((N, D))
    dW = np.zeros((V, D))
    db = np.zeros(V)
    if C == 0:
        return 0.0, m, np.full(N, -np.inf), dH, dW, db
    Hs = H[idx]
    ys = y[idx]
    ms = np.full(C, -np.inf)
    ss = np.zeros(C)
    tg = np.full(C, np.nan)
    for t0 in range(0, C, T):
        rt = slice(t0, min(C, t0 + T))
        for v0 in range(0, V, B):
            v1 = min(V, v0 + B)
            Z = Hs[rt] @ W[v0:v1].T
            if b is not None:
                Z = Z + b[v0:v1][None, :]
            m_old = ms[rt]
            m_new = np.maximum(m_old, Z.max(axis=1))
            first = np.isneginf(m_old)
            factor = np.where(first, 0.0, np.exp(np.where(first, 0.0, m_old - m_new)))
            ss[rt] = factor * ss[rt] + np.exp(Z - m_new[:, None]).sum(axis=1)
            ms[rt] = m_new
            # target capture by global column id
            yy = ys[rt]
            hit = (yy >= v0) & (yy < v1)
            rows_hit = np.flatnonzero(hit)
            tg[t0 + rows_hit] = Z[rows_hit, yy[rows_hit] - v0]
    logss = np.log(ss)
    row_loss = (ms - tg) + logss
    loss = math.fsum(row_loss.tolist()) / C
    scale = lam / C
    for t0 in range(0, C, T):
        rt = slice(t0, min(C, t0 + T))
        dH_T = np.zeros((rt.stop - rt.start, D))
        for v0 in range(0, V, B):
            v1 = min(V, v0 + B)
            Z = Hs[rt] @ W[v0:v1].T
            if b is not None:
                Z = Z + b[v0:v1][None, :]
            if _fault == "local_norm":
                zm = Z.max(axis=1, keepdims=True)
                P = np.exp(Z - zm)
                P /= P.sum(axis=1, keepdims=True)
            else:
                P = np.exp((Z - ms[rt][:, None]) - logss[rt][:, None])
            yy = ys[rt]
            hit = np.flatnonzero((yy >= v0) & (yy < v1))
            P[hit, yy[hit] - v0] -= 1.0
            G = scale * P
            if _fault == "dh_overwrite":
                dH_T = G @ W[v0:v1]
            else:
                dH_T += G @ W[v0:v1]
            dW[v0:v1] += G.T @ Hs[rt]
            db[v0:v1] += G.sum(axis=0)
        dH[idx[rt]] = dH_T
    m[idx] = ms
    logs = np.full(N, -np.inf)
    logs[idx] = logss
    return loss, m, logs, dH, dW, db
