"""HIP path at the full workload sizes, in the launch configuration the
benchmark times (same N, D, V; the C-ABI picks tiles, splits and chunks from
the sizes alone), against the float64 oracle.

  * sft, page2, packed: every output element (loss, m, log s and the per-row
    CE of every position, dH, dW, db) against the oracle's dense forward and
    backward over all C supervised rows (the complete comparison of the
    glenzli.com page, section 06);
  * stress: the oracle's statistics of all C rows (loss, m, log s, per-row
    CE everywhere), dW and db at vocabulary rows chosen to cover the +30-bias
    rows, the most frequent labels, the vocabulary chunk boundaries of the
    backward and the last rows, and dH at sampled rows;
  * sparse supervision (a mask that keeps 48 rows of the same inputs): every
    output element, on the launch configuration of a tiny C.
"""

import math

import numpy as np
import pytest
import torch

import oracle as O
from lm_head_projection_amd import _lib
from lm_head_projection_amd import workloads as WL

from lce_harness import assert_grad_close, assert_stat_close, run_gpu, run_gpu_filtered, say, tol

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]

FULL = ("sft", "page2", "packed", "stress")
_cache = {}


def workload(name):
    if name not in _cache:
        say(f"[fullsize] building workload {name}")
        wl = WL.make_workload(name)
        _cache[name] = (wl, wl.W.double().numpy(), None if wl.b is None else wl.b.double().numpy())
    return _cache[name]


def oracle_forward(wl, Wd, bd, groups=8):
    """The oracle's dense forward over every supervised row, a group of rows
    at a time (rows are independent in the objective), with progress lines."""
    y = wl.labels.numpy()
    mask = None if wl.mask is None else wl.mask.numpy()
    _, idx, C = O.supervised_rows(y, mask)
    Hd = wl.H.double().numpy()
    m = np.full(wl.N, -np.inf)
    logs = np.full(wl.N, -np.inf)
    row_loss = np.zeros(wl.N)
    for k, sel in enumerate(np.array_split(idx, groups)):
        f = O.dense_forward(Hd[sel], Wd, bd, y[sel], row_block=256)
        m[sel], logs[sel], row_loss[sel] = f.m, f.logs, f.row_loss
        say(f"[fullsize] {wl.name}: oracle forward, row group {k + 1}/{groups}")
    loss = math.fsum(row_loss[idx].tolist()) / C
    return Hd, idx, C, loss, m, logs, row_loss


def check_statistics(r, idx, C, loss, m, logs, row_loss, t):
    assert r.C == C
    np.testing.assert_array_equal(r.idx, idx)
    assert abs(r.loss - loss) <= t["loss"] * abs(loss), (r.loss, loss)
    assert_stat_close("m", r.m[idx], m[idx], t["stat"])
    assert_stat_close("logs", r.logs[idx], logs[idx], t["stat"])
    assert_stat_close("row_loss", r.row_loss[idx], row_loss[idx], t["stat"])
    a = np.zeros(r.m.size, dtype=bool)
    a[idx] = True
    assert np.all(r.m[~a] == -np.inf) and np.all(r.logs[~a] == -np.inf) and np.all(r.row_loss[~a] == 0.0)
    return a


@pytest.mark.parametrize("name", ("sft", "page2", "packed"))
def test_fullsize_every_element(name):
    wl, Wd, bd = workload(name)
    say(f"[fullsize] {name}: GPU run N={wl.N} D={wl.D} V={wl.V}")
    r = run_gpu(wl)
    assert r.status_c == _lib.LCE_OK and r.status_f == _lib.LCE_OK and r.status_b == _lib.LCE_OK
    t = tol(wl.dtype)
    Hd, idx, C, loss, m, logs, row_loss = oracle_forward(wl, Wd, bd)
    a = check_statistics(r, idx, C, loss, m, logs, row_loss, t)
    say(f"[fullsize] {name}: oracle backward over all {C} rows")
    g = O.dense_backward(Hd, Wd, bd, wl.labels.numpy(), m, logs, 1.0,
                         None if wl.mask is None else wl.mask.numpy(), row_block=256)
    assert np.all(r.dH[~a] == 0.0)
    assert_grad_close("dH", r.dH, g.dH, t["grad"])
    assert_grad_close("dW", r.dW, g.dW, t["grad"])
    if wl.b is not None:
        assert_grad_close("db", r.db, g.db, t["grad"])


def test_fullsize_stress_statistics_and_sampled_gradients():
    wl, Wd, bd = workload("stress")
    say(f"[fullsize] stress: GPU run N={wl.N} D={wl.D} V={wl.V}")
    r = run_gpu(wl, keep_device=True)
    assert r.status_c == _lib.LCE_OK and r.status_f == _lib.LCE_OK and r.status_b == _lib.LCE_OK
    t = tol(wl.dtype)
    Hd, idx, C, loss, m, logs, row_loss = oracle_forward(wl, Wd, bd, groups=16)
    a = check_statistics(r, idx, C, loss, m, logs, row_loss, t)
    y = wl.labels.numpy()
    # vocabulary rows: +30-bias rows, the most frequent labels, the 32768-wide
    # chunk boundaries of the backward, the last rows, and random ones
    rng = np.random.default_rng(41)
    hot = np.flatnonzero(bd == 30.0)
    hot = np.unique(np.concatenate([hot[[0, -1]], rng.choice(hot, 6, replace=False)]))
    freq = np.argsort(np.bincount(y[idx], minlength=wl.V), kind="stable")[-4:]
    rest = np.array([0, 32767, 32768, 65535, 65536, 229375, 229376, wl.V - 2, wl.V - 1])
    rest = np.unique(np.concatenate([rest, freq, rng.choice(wl.V, 6, replace=False)]))
    rest = rest[bd[rest] != 30.0]
    say(f"[fullsize] stress: oracle dW/db at {hot.size} +30-bias rows and {rest.size} other rows")
    dW = r.dW.detach()
    db = r.db.detach()
    for label, cols in (("+30-bias rows", hot), ("other rows", rest)):
        dw_o, db_o = O.cols_grad(Hd, Wd, bd, y, m, logs, cols, row_block=2048)
        assert_grad_close(f"dW {label}", dW[torch.as_tensor(cols, device=dW.device)].double().cpu().numpy(),
                          dw_o, t["grad"])
        assert_grad_close(f"db {label}", db[torch.as_tensor(cols, device=db.device)].double().cpu().numpy(),
                          db_o, t["grad"])
    rows = np.unique(np.concatenate([idx[[0, 255, 256, C - 1]], rng.choice(idx, 6, replace=False)]))
    say(f"[fullsize] stress: oracle dH at {rows.size} rows")
    dh = O.rows_grad_h(Hd[rows], Wd, bd, y[rows], 1.0 / C)
    dH = r.dH.detach()
    assert_grad_close("dH rows", dH[torch.as_tensor(rows, device=dH.device)].double().cpu().numpy(), dh, t["grad"])
    assert int(torch.count_nonzero(dH[torch.as_tensor(np.flatnonzero(~a), device=dH.device)])) == 0


def test_fullsize_packed_forward_only_against_the_oracle():
    """The evaluation entry (m = log s = NULL) at the packed sizes: the mean,
    the weighted sum and the per-position losses against the oracle's
    reductions of its per-row CE over all C supervised rows."""
    from lce_harness import run_gpu_ex
    wl, Wd, bd = workload("packed")
    _, idx, C, loss, m, logs, row_loss = oracle_forward(wl, Wd, bd)
    t = tol(wl.dtype)
    rng = np.random.default_rng(43)
    w = rng.uniform(0.0, 2.0, wl.N).astype(np.float32)
    for red, weights, num in (("mean", None, 0.0), ("sum", w, float(C)), ("none", None, 0.0)):
        say(f"[fullsize] packed: forward-only {red}")
        r = run_gpu_ex(wl, red, weights, num, stats=False)
        assert r.status_f == _lib.LCE_OK and r.m is None and r.C == C
        ref = O.reduce_rows(row_loss, idx, C, red, None if weights is None else weights.astype(np.float64),
                            num if num else None)
        if red == "none":
            assert_stat_close("per-position loss", r.loss[idx], ref[idx], t["stat"])
            a = np.zeros(wl.N, dtype=bool)
            a[idx] = True
            assert np.all(r.loss[~a] == 0.0)
        else:
            assert abs(r.loss[0] - ref) <= t["loss"] * abs(ref), (red, r.loss[0], ref)


@pytest.mark.parametrize("name", FULL)
def test_fullsize_sparse_supervision_elementwise(name):
    wl, Wd, bd = workload(name)
    sub = WL.supervised_subset(wl, 48)
    say(f"[fullsize] {name}: GPU run with 48 supervised rows")
    r = run_gpu(sub)
    say(f"[fullsize] {name}: oracle on the 48 rows")
    f, g = O.dense_forward_backward(sub.H.double().numpy(), Wd, bd, sub.labels.numpy(), sub.mask.numpy(), 1.0)
    t = tol(wl.dtype)
    assert r.C == f.C == 48
    np.testing.assert_array_equal(r.idx, f.idx)
    assert abs(r.loss - f.loss) <= t["loss"] * abs(f.loss)
    assert_stat_close("m", r.m[f.idx], f.m[f.idx], t["stat"])
    assert_stat_close("logs", r.logs[f.idx], f.logs[f.idx], t["stat"])
    assert_grad_close("dH", r.dH, g.dH, t["grad"])
    assert_grad_close("dW", r.dW, g.dW, t["grad"])
    if wl.b is not None:
        assert_grad_close("db", r.db, g.db, t["grad"])


@pytest.mark.parametrize("name", ("packed", "stress"))
def test_fullsize_weighted_sum_and_per_position(name):
    """The reduction variants at full size: per-position losses (reduction
    none) at sampled rows against the oracle; the weighted, divided sum equals
    the fp64 sum of those per-position values; dH of the weighted sum at
    sampled rows against the oracle with each row's factor lambda w_i / n."""
    from lce_harness import run_gpu_ex
    wl, Wd, bd = workload(name)
    rng = np.random.default_rng(23)
    w = rng.uniform(0.0, 2.0, wl.N).astype(np.float32)
    num, lam = 0.5 * wl.N, 1.25
    say(f"[fullsize] {name}: reduction none (forward only)")
    rn = run_gpu_ex(wl, "none", backward=False)
    say(f"[fullsize] {name}: weighted sum, forward + backward")
    rs = run_gpu_ex(wl, "sum", w, num, lam)
    assert rn.status_f == _lib.LCE_OK and rs.status_f == _lib.LCE_OK and rs.status_b == _lib.LCE_OK
    idx = rs.idx
    ref = math.fsum((w[idx].astype(np.float64) * rn.loss[idx]).tolist()) / num
    assert abs(rs.loss[0] - ref) <= 1e-6 * abs(ref)
    rows = np.unique(np.concatenate([np.sort(rng.choice(idx, size=6, replace=False)), idx[[0, -1]]]))
    say(f"[fullsize] {name}: oracle on {rows.size} sampled rows")
    Hs = wl.H[rows].double().numpy()
    ys = wl.labels.numpy()[rows]
    _, _, l = O.rows_forward(Hs, Wd, bd, ys)
    t = tol(wl.dtype)
    assert_stat_close("per-position loss", rn.loss[rows], l, t["stat"])
    dh = np.concatenate([O.rows_grad_h(Hs[k:k + 1], Wd, bd, ys[k:k + 1], lam * float(w[rows[k]]) / num)
                         for k in range(rows.size)])
    assert_grad_close("dH rows", rs.dH[rows], dh, t["grad"])


def test_fullsize_packed_eight_vocabulary_shards():
    """The packed workload split into 8 vocabulary shards of ~31040 rows (one
    tensor-parallel rank's share of an 8-way split) matches the unsharded run:
    loss, m, log s within fp32 rounding of a different merge order; dW rows
    and the summed dH partials within the gradient tolerance."""
    from test_gpu_shards import run_sharded
    wl, Wd, bd = workload("packed")
    V = wl.V
    bounds = [V * p // 8 for p in range(9)]
    say("[fullsize] packed: unsharded")
    r0 = run_gpu(wl)
    say("[fullsize] packed: 8 shards")
    r1 = run_sharded(wl, bounds)
    assert abs(r1["loss"][0] - r0.loss) <= 1e-5 * abs(r0.loss)
    a = np.zeros(wl.N, dtype=bool)
    a[r0.idx] = True
    assert_stat_close("m", r1["m"][a], r0.m[a], 1e-5)
    assert_stat_close("logs", r1["logs"][a], r0.logs[a], 1e-5)
    t = tol(wl.dtype)
    assert_grad_close("dW", r1["dW"], r0.dW, t["grad"])
    assert_grad_close("dH", r1["dH"], r0.dH, t["grad"])


def test_fullsize_packed_filter_sparse_elementwise():
    """Gradient filtering at the packed sizes with 48 supervised rows (one
    row block), eps = 1e-3: every output element against the oracle's
    filtered backward.  Every block decided by probability sits at least a
    factor 4 from eps, so both sides decide alike."""
    wl, Wd, bd = workload("packed")
    sub = WL.supervised_subset(wl, 48)
    eps = 1e-3
    say("[fullsize] packed: filtered backward, 48 supervised rows")
    st, dH, dW, db = run_gpu_filtered(sub, eps)
    assert st == _lib.LCE_OK
    say("[fullsize] packed: oracle filtered backward on the 48 rows")
    Hd, y, mk = sub.H.double().numpy(), sub.labels.numpy(), sub.mask.numpy()
    f = O.dense_forward(Hd, Wd, bd, y, mk)
    g = O.filtered_backward(Hd, Wd, bd, y, f.m, f.logs, eps, 1.0, mk)
    P = np.exp((O.logits(Hd[f.idx], Wd, bd) - f.m[f.idx][:, None]) - f.logs[f.idx][:, None])
    P[np.arange(f.C), y[f.idx]] = 0.0
    tgt = np.zeros(wl.V // 32 + 1, dtype=bool)
    tgt[y[f.idx] // 32] = True
    blk_max = np.max(P[:, :(wl.V // 32) * 32].reshape(f.C, -1, 32), axis=(0, 2))
    free = blk_max[~tgt[:blk_max.size]]
    assert np.all(np.abs(np.log(free / eps)) > np.log(4.0))
    t = tol(wl.dtype)
    assert_grad_close("dH filtered", dH, g.dH, t["grad"])
    assert_grad_close("dW filtered", dW, g.dW, t["grad"])
    assert np.count_nonzero(np.any(dW != 0.0, axis=1)) <= 32 * int(tgt.sum())


def test_fullsize_packed_filter_keeps_target_blocks():
    """Full supervision at the packed sizes, eps = 10 (above every p): only
    blocks holding a target survive.  dW rows of vocabulary blocks that hold
    no label are exactly 0; sampled dH rows of the first and the last
    (ragged) row block against the oracle's filtered rows."""
    wl, Wd, bd = workload("packed")
    say("[fullsize] packed: filtered backward, eps 10")
    st, dH, dW, db = run_gpu_filtered(wl, 10.0)
    assert st == _lib.LCE_OK
    y = wl.labels.numpy()
    _, idx, C = O.supervised_rows(y, None)
    labelled = np.zeros(wl.V // 32 + 1, dtype=bool)
    labelled[y[idx] // 32] = True
    dead = ~labelled[np.arange(wl.V) // 32]
    assert np.all(dW[dead] == 0.0)
    last = (C - 1) // 256
    blocks = np.concatenate([idx[:256], idx[last * 256:]])
    rng = np.random.default_rng(29)
    rows = np.unique(np.concatenate([idx[[0, 255, last * 256, C - 1]],
                                     rng.choice(idx[:256], 2, replace=False),
                                     rng.choice(idx[last * 256:], 2, replace=False)]))
    say(f"[fullsize] packed: oracle statistics of {blocks.size} rows, filtered dH of {rows.size}")
    sel = np.zeros(wl.N, dtype=bool)
    sel[blocks] = True
    Hd = wl.H.double().numpy()
    f = O.dense_forward(Hd, Wd, bd, y, sel)
    dh, _, _ = O.filtered_rows_grad(Hd, Wd, bd, y, f.m, f.logs, 10.0, rows, [], 1.0)
    t = tol(wl.dtype)
    assert_grad_close("dH rows filtered", dH[rows], dh, t["grad"])


def test_fullsize_packed_memory_far_below_dense_logits():
    """A forward + backward through the autograd wrapper at the packed sizes:
    between the two passes it holds only the supervised-row list and the two
    saved N-vectors; the device memory it adds beyond the inputs and the gradient buffers
    (workspace, index and statistics arrays) stays under a quarter of the
    dense bf16 N x V logits, and no block the allocator holds afterwards is
    as large as those logits."""
    from lm_head_projection_amd import linear_cross_entropy
    wl, _, _ = workload("packed")
    dev = "cuda:0"
    H = wl.H.to(dev).requires_grad_(True)
    W = wl.W.to(dev).requires_grad_(True)
    labels = wl.labels.to(dev)
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    loss = linear_cross_entropy(H, W, labels)
    torch.cuda.synchronize()
    held = torch.cuda.memory_allocated() - base
    say(f"[fullsize] packed: held between forward and backward {held / 1e6:.3f} MB")
    # the supervised-row list, m and log s (three N-vectors) and the loss: the
    # forward workspace is gone, and nothing of size N x V or N x D remains
    assert held <= 3 * 4 * wl.N + 64 * 1024, held
    loss.backward()
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    grads = (H.numel() + W.numel()) * H.element_size()
    dense = wl.N * wl.V * 2
    say(f"[fullsize] packed: peak extra {peak / 1e9:.2f} GB (gradients {grads / 1e9:.2f} GB), "
        f"dense logits {dense / 1e9:.2f} GB")
    assert torch.isfinite(loss)
    assert peak - grads < dense / 4
    for seg in torch.cuda.memory_snapshot():
        for blk in seg["blocks"]:
            assert blk["size"] < dense, blk
