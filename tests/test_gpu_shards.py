"""Vocabulary sharding on one device (lce_forward_shard / lce_merge_shards /
lce_backward_shard) against the float64 oracle, through the C ABI.

The shards' running statistics over disjoint vocabulary ranges merge exactly
into the full-vocabulary ones (glenzli.com page, section 02), so the merged
loss, m and log s equal the dense definition, each shard's dW / db rows equal
the matching rows of the dense gradients, and the shards' dH partials sum to
the dense dH.  Per-shard partials are checked against the oracle's two-pass
LSE over the shard's slice of the vocabulary.
"""

import numpy as np
import pytest
import torch

import oracle as O
from lm_head_projection_amd import _lib
from lm_head_projection_amd import workloads as WL

from lce_harness import assert_grad_close, assert_stat_close, run_gpu, say, tol

pytestmark = pytest.mark.gpu


def shard_bounds(V, P, seed=0):
    """P contiguous, uneven, non-empty vocabulary ranges (some not multiples of 256)."""
    rng = np.random.default_rng(seed)
    cuts = np.sort(rng.choice(np.arange(1, V), size=P - 1, replace=False)) if P > 1 else np.array([], int)
    return [0] + [int(c) for c in cuts] + [V]


def run_sharded(wl, bounds, reduction="mean", weights=None, num=0.0, grad=1.0, dev="cuda:0"):
    H = wl.H.to(dev)
    W = wl.W.to(dev)
    b = None if wl.b is None else wl.b.to(dev)
    labels = wl.labels.to(dev)
    mask = None if wl.mask is None else wl.mask.to(torch.uint8).to(dev)
    N, D = H.shape
    V = W.shape[0]
    P = len(bounds) - 1
    ws = torch.empty(_lib.lce_workspace_size(N, D, V, H.dtype), dtype=torch.uint8, device=dev)
    idx = torch.empty(max(N, 1), dtype=torch.int32, device=dev)
    st, C = _lib.lce_compact_valid(labels, mask, V, wl.ignore_index, idx, ws)
    assert st == _lib.LCE_OK
    parts = torch.full((P, 3 * C), float("nan"), dtype=torch.float32, device=dev)
    for p in range(P):
        v0, v1 = bounds[p], bounds[p + 1]
        bs = None if b is None else b[v0:v1]
        st = _lib.lce_forward_shard(H, W[v0:v1], bs, labels, idx, C, v0, parts[p], ws)
        assert st == _lib.LCE_OK, _lib.status_string(st)
    red = _lib.REDUCTIONS[reduction]
    w = None if weights is None else torch.tensor(weights, dtype=torch.float32, device=dev)
    loss = torch.empty(N if reduction == "none" else 1, dtype=torch.float32, device=dev)
    m = torch.empty(N, dtype=torch.float32, device=dev)
    logs = torch.empty(N, dtype=torch.float32, device=dev)
    st = _lib.lce_merge_shards(parts, bounds, labels, idx, C, red, w, num, loss, m, logs, ws)
    assert st == _lib.LCE_OK, _lib.status_string(st)
    g = torch.tensor(np.atleast_1d(np.asarray(grad, dtype=np.float32)), device=dev)
    dH_sum = np.zeros((N, D))
    dW = torch.full_like(W, 7.0)
    db = None if b is None else torch.full_like(b, 7.0)
    for p in range(P):
        v0, v1 = bounds[p], bounds[p + 1]
        bs = None if b is None else b[v0:v1]
        dHp = torch.full_like(H, 7.0)
        st = _lib.lce_backward_shard(H, W[v0:v1], bs, labels, idx, C, v0, red, w, num, m, logs, g, dHp, dW[v0:v1],
                                     None if db is None else db[v0:v1], ws)
        assert st == _lib.LCE_OK, _lib.status_string(st)
        dH_sum += dHp.double().cpu().numpy()  # the all-reduce of a multi-device run
    torch.cuda.synchronize()
    to = lambda t: None if t is None else t.double().cpu().numpy()
    return dict(C=C, idx=idx[:C].cpu().numpy().astype(np.int64), parts=parts.double().cpu().numpy(),
                loss=to(loss), m=to(m), logs=to(logs), dH=dH_sum, dW=to(dW), db=to(db))


def _np(wl):
    return (wl.H.double().numpy(), wl.W.double().numpy(), None if wl.b is None else wl.b.double().numpy(),
            wl.labels.numpy(), None if wl.mask is None else wl.mask.numpy())


@pytest.mark.parametrize("P", [1, 3, 8])
@pytest.mark.parametrize("name", ["tiny", "sft_small", "page2_small", "stress_small"])
def test_sharded_equals_dense(name, P):
    say(f"[shards] {name} P={P}")
    wl = WL.make_workload(name)
    bounds = shard_bounds(wl.V, P, seed=P)
    H, W, b, y, mask = _np(wl)
    f, g = O.dense_forward_backward(H, W, b, y, mask, 1.0, wl.ignore_index)
    r = run_sharded(wl, bounds)
    t = tol(wl.dtype)
    assert r["C"] == f.C
    np.testing.assert_array_equal(r["idx"], f.idx)
    # per-shard partials against the oracle's LSE over the shard's slice
    C = f.C
    for p in range(P):
        v0, v1 = bounds[p], bounds[p + 1]
        Z = O.logits(H[f.idx], W[v0:v1], None if b is None else b[v0:v1])
        Mp, LSp = O.lse_two_pass(Z)
        assert_stat_close(f"m shard {p}", r["parts"][p, :C], Mp, t["stat"])
        assert_stat_close(f"log s shard {p}", np.log(r["parts"][p, C:2 * C]), LSp, t["stat"])
        yy = y[f.idx]
        own = (yy >= v0) & (yy < v1)
        zt = Z[np.arange(C)[own], yy[own] - v0]
        assert_stat_close(f"target shard {p}", r["parts"][p, 2 * C:][own], zt, t["stat"])
    assert abs(r["loss"][0] - f.loss) <= t["loss"] * abs(f.loss)
    a = np.zeros(wl.N, dtype=bool)
    a[f.idx] = True
    assert_stat_close("m", r["m"][a], f.m[a], t["stat"])
    assert_stat_close("logs", r["logs"][a], f.logs[a], t["stat"])
    assert np.all(np.isneginf(r["m"][~a])) and np.all(np.isneginf(r["logs"][~a]))
    assert_grad_close("dH (sum of shard partials)", r["dH"], g.dH, t["grad"])
    assert np.all(r["dH"][~a] == 0.0)
    assert_grad_close("dW (shards)", r["dW"], g.dW, t["grad"])
    if b is not None:
        assert_grad_close("db (shards)", r["db"], g.db, t["grad"])


def test_one_shard_is_bitwise_the_plain_forward():
    wl = WL.make_workload("page2_small")
    r0 = run_gpu(wl, backward=False)
    r1 = run_sharded(wl, [0, wl.V])
    assert np.float32(r0.loss) == np.float32(r1["loss"][0])
    np.testing.assert_array_equal(r0.m, r1["m"])
    np.testing.assert_array_equal(r0.logs, r1["logs"])


@pytest.mark.parametrize("reduction", ["sum", "none"])
def test_sharded_reductions(reduction):
    wl = WL.make_workload("page2_small")
    bounds = shard_bounds(wl.V, 4, seed=11)
    H, W, b, y, mask = _np(wl)
    rng = np.random.default_rng(12)
    if reduction == "sum":
        w, num, grad = rng.uniform(0, 2, wl.N).astype(np.float32), 123.0, 0.9
    else:
        w, num, grad = None, 0.0, rng.standard_normal(wl.N).astype(np.float32)
    f = O.dense_forward(H, W, b, y, mask)
    ref = O.reduce_rows(f.row_loss, f.idx, f.C, reduction, None if w is None else w.astype(np.float64),
                        num if num else None)
    rf = O.row_factors(wl.N, f.idx, f.C, reduction, np.asarray(grad, dtype=np.float64),
                       None if w is None else w.astype(np.float64), num if num else None)
    g = O.dense_backward(H, W, b, y, f.m, f.logs, mask=mask, row_factor=rf)
    r = run_sharded(wl, bounds, reduction, w, num, grad)
    t = tol(wl.dtype)
    if reduction == "none":
        a = np.zeros(wl.N, dtype=bool)
        a[f.idx] = True
        assert_stat_close("per-position loss", r["loss"][a], ref[a], t["stat"])
        assert np.all(r["loss"][~a] == 0.0)
    else:
        assert abs(r["loss"][0] - ref) <= t["loss"] * abs(ref)
    assert_grad_close("dH", r["dH"], g.dH, t["grad"])
    assert_grad_close("dW", r["dW"], g.dW, t["grad"])
    assert_grad_close("db", r["db"], g.db, t["grad"])
