"""Reduction variants and the forward-only entry, HIP path vs the float64
oracle through the C ABI (lce_forward_ex / lce_backward_ex).

The variants are the NeMo chunked_ce interface's: a mean over the supervised
rows, a sum with per-position weights divided by an external token count, and
per-position losses with a per-position upstream gradient.  They change only
the loss reduction and the row factor r_i of G = r_i (p - onehot); the oracle's
reduce_rows / row_factors are pinned against torch's own reductions and
autograd in test_oracle_pins.py.
"""

import math

import numpy as np
import pytest
import torch

import oracle as O
from lm_head_projection_amd import _lib
from lm_head_projection_amd import workloads as WL

from lce_harness import assert_grad_close, assert_stat_close, run_gpu, run_gpu_ex, say, tol

pytestmark = pytest.mark.gpu

CASES = ("tiny", "sft_small", "page2_small", "stress_small")


def _np(wl):
    H, W = wl.H.double().numpy(), wl.W.double().numpy()
    b = None if wl.b is None else wl.b.double().numpy()
    mask = None if wl.mask is None else wl.mask.numpy()
    return H, W, b, wl.labels.numpy(), mask


def _inputs(wl, reduction, seed):
    rng = np.random.default_rng(seed)
    if reduction == "sum_weighted":
        return "sum", rng.uniform(-0.5, 2.0, wl.N).astype(np.float32), 3.5 * wl.N, 1.3
    if reduction == "sum":
        return "sum", None, 0.0, 0.7
    if reduction == "none":
        return "none", None, 0.0, rng.standard_normal(wl.N).astype(np.float32)
    return "mean", None, 0.0, -1.1


@pytest.mark.parametrize("variant", ["sum_weighted", "sum", "none", "mean"])
@pytest.mark.parametrize("name", CASES)
def test_reduction_parity(name, variant):
    say(f"[reduce] {name} {variant}")
    wl = WL.make_workload(name)
    red, w, num, grad = _inputs(wl, variant, 41)
    H, W, b, y, mask = _np(wl)
    f = O.dense_forward(H, W, b, y, mask, wl.ignore_index)
    w64 = None if w is None else w.astype(np.float64)
    ref_loss = O.reduce_rows(f.row_loss, f.idx, f.C, red, w64, num if num else None)
    rf = O.row_factors(wl.N, f.idx, f.C, red, np.asarray(grad, dtype=np.float64), w64, num if num else None)
    g = O.dense_backward(H, W, b, y, f.m, f.logs, mask=mask, ignore_index=wl.ignore_index, row_factor=rf)
    r = run_gpu_ex(wl, red, w, num, grad)
    t = tol(wl.dtype)
    assert r.status_f == _lib.LCE_OK and r.status_b == _lib.LCE_OK
    assert r.C == f.C
    a = np.zeros(wl.N, dtype=bool)
    a[f.idx] = True
    if red == "none":
        assert r.loss.shape == (wl.N,)
        assert_stat_close("per-position loss", r.loss[a], ref_loss[a], t["stat"])
        assert np.all(r.loss[~a] == 0.0)
    else:
        # relative to the sum of magnitudes (signed weights may cancel)
        scale = (np.sum(np.abs(w64[f.idx] * f.row_loss[f.idx])) / num) if w is not None else abs(ref_loss)
        assert abs(r.loss[0] - ref_loss) <= t["loss"] * scale, (r.loss[0], ref_loss)
    assert_stat_close("m", r.m[a], f.m[a], t["stat"])
    assert_stat_close("logs", r.logs[a], f.logs[a], t["stat"])
    assert_grad_close("dH", r.dH, g.dH, t["grad"])
    assert np.all(r.dH[~a] == 0.0)
    assert_grad_close("dW", r.dW, g.dW, t["grad"])
    if wl.b is not None:
        assert_grad_close("db", r.db, g.db, t["grad"])


def test_mean_ex_is_bitwise_the_plain_entry():
    """lce_forward_ex / lce_backward_ex with MEAN run the same kernels as
    lce_forward / lce_backward: identical bits."""
    wl = WL.make_workload("page2_small")
    r0 = run_gpu(wl, lam=0.8)
    r1 = run_gpu_ex(wl, "mean", None, 0.0, 0.8)
    assert np.float32(r0.loss) == np.float32(r1.loss[0])
    np.testing.assert_array_equal(r0.m, r1.m)
    np.testing.assert_array_equal(r0.logs, r1.logs)
    np.testing.assert_array_equal(r0.dH, r1.dH)
    np.testing.assert_array_equal(r0.dW, r1.dW)
    np.testing.assert_array_equal(r0.db, r1.db)


@pytest.mark.parametrize("red", ["mean", "sum", "none"])
@pytest.mark.parametrize("name", ["tiny", "sft_small", "page2_small"])
def test_forward_only_without_saved_statistics(name, red):
    """The evaluation entry (cross-entropy and perplexity without a backward;
    AIInfraGuide chapter 2, section 5): m and logs NULL.  The loss is the
    oracle's reduction of its per-row CE, and its bits equal those of the run
    that saves the statistics."""
    wl = WL.make_workload(name)
    w = np.linspace(-0.5, 1.5, wl.N).astype(np.float32) if red == "sum" else None
    num = 100.0 if red == "sum" else 0.0
    r_eval = run_gpu_ex(wl, red, w, num, stats=False)
    assert r_eval.status_f == _lib.LCE_OK
    assert r_eval.m is None and r_eval.logs is None
    H, W, b, y, mask = _np(wl)
    f = O.dense_forward(H, W, b, y, mask, wl.ignore_index)
    w64 = None if w is None else w.astype(np.float64)
    ref = O.reduce_rows(f.row_loss, f.idx, f.C, red, w64, num if num else None)
    t = tol(wl.dtype)
    if red == "none":
        a = np.zeros(wl.N, dtype=bool)
        a[f.idx] = True
        assert_stat_close("per-position loss", r_eval.loss[a], ref[a], t["stat"])
        assert np.all(r_eval.loss[~a] == 0.0)
    else:
        scale = np.sum(np.abs(w64[f.idx] * f.row_loss[f.idx])) / num if w is not None else abs(ref)
        assert abs(r_eval.loss[0] - ref) <= t["loss"] * scale, (r_eval.loss[0], ref)
        if red == "mean":  # perplexity exp(L): relative error of L times L
            assert abs(math.exp(r_eval.loss[0]) - math.exp(ref)) <= t["loss"] * abs(ref) * 1.01 * math.exp(ref)
    r_stats = run_gpu_ex(wl, red, w, num, backward=False)
    np.testing.assert_array_equal(r_eval.loss, r_stats.loss)


def test_reductions_empty_supervision():
    """C = 0: sum -> 0, none -> all zeros, gradients exactly zero."""
    wl = WL.make_workload("sft_small")
    wl.labels[:] = wl.ignore_index
    for red, grad in (("sum", 2.0), ("none", np.ones(wl.N, dtype=np.float32))):
        r = run_gpu_ex(wl, red, None, 0.0, grad)
        assert r.status_f == _lib.LCE_OK_EMPTY and r.status_b == _lib.LCE_OK_EMPTY
        assert np.all(r.loss == 0.0)
        assert np.all(np.isneginf(r.m)) and np.all(np.isneginf(r.logs))
        assert np.all(r.dH == 0.0) and np.all(r.dW == 0.0)


def test_none_with_null_gradient_means_one_per_position():
    wl = WL.make_workload("page2_small")
    H, W, b, y, mask = _np(wl)
    f = O.dense_forward(H, W, b, y, mask)
    g = O.dense_backward(H, W, b, y, f.m, f.logs, mask=mask,
                         row_factor=O.row_factors(wl.N, f.idx, f.C, "none", np.ones(wl.N)))
    r = run_gpu_ex(wl, "none", None, 0.0, None)
    t = tol(wl.dtype)
    assert_grad_close("dH", r.dH, g.dH, t["grad"])
    assert_grad_close("dW", r.dW, g.dW, t["grad"])
    assert_grad_close("db", r.db, g.db, t["grad"])
