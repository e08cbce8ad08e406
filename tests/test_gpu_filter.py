"""Gradient filtering (lce_backward_filtered) against the oracle's
filtered_backward, through the C ABI.

The filter decides per block (256 supervised rows x 32 vocabulary entries)
from probabilities, so where a block's largest p sits close to eps the
float32 kernel and the float64 oracle could decide differently.  The tests
therefore take eps inside a wide gap of the oracle's block maxima (at least
a factor 4 from every block), where both sides decide alike, plus eps = 0
(nothing dropped: bitwise the unfiltered backward) and eps > 1 (only blocks
holding a target survive).
"""

import numpy as np
import pytest
import torch

import oracle as O
from lm_head_projection_amd import _lib
from lm_head_projection_amd import workloads as WL

from lce_harness import assert_grad_close, run_gpu, run_gpu_filtered, say, tol, to_np

pytestmark = pytest.mark.gpu


def peaked_workload(seed=7, N=700, D=128, V=3001):
    """A bf16 workload with three probability levels set by the bias: targets
    in [0, 512) (b = +4), a middle band [512, 1024) (b = +1.5) and the rest
    (b = -2.5); small scores (w_scale 0.02) keep each level tight, so the
    target-free blocks of the two lower bands sit about e^4 apart."""
    wl = WL.make_random(N, D, V, dtype=torch.bfloat16, seed=seed, ignore_frac=0.15, mask_frac=0.05,
                        w_scale=0.02, b_scale=0.05)
    b = wl.b.float()
    b[:512] += 4.0
    b[512:1024] += 1.5
    b[1024:] -= 2.5
    wl.b = b.to(torch.bfloat16)
    g = torch.Generator().manual_seed(seed + 1)
    keep = wl.labels != wl.ignore_index
    wl.labels[keep] = torch.randint(0, 512, (int(keep.sum()),), generator=g)
    return wl


def block_maxima(wl, f, r=None):
    """Largest p of every (256-row, 32-column) block without a target (oracle),
    over the rows whose factor r_i is not 0 (all rows when r is None)."""
    H, W = wl.H.double().numpy(), wl.W.double().numpy()
    b = None if wl.b is None else wl.b.double().numpy()
    y = wl.labels.numpy()
    out = []
    for lo in range(0, f.C, 256):
        rows = f.idx[lo:lo + 256]
        P = np.exp((O.logits(H[rows], W, b) - f.m[rows][:, None]) - f.logs[rows][:, None])
        if r is not None:
            P = P[r[rows] != 0.0]
        for v0 in range(0, wl.V, 32):
            if P.shape[0] and not np.any((y[rows] >= v0) & (y[rows] < v0 + 32)):
                out.append(P[:, v0:v0 + 32].max())
    return np.array(out)


def gap_eps(maxima, factor=4.0):
    v = np.unique(maxima[maxima > 0])
    ratios = v[1:] / v[:-1]
    k = int(np.argmax(ratios))
    assert ratios[k] >= factor * factor, f"no gap of {factor}x on both sides (best {ratios[k]:.2f})"
    return float(np.sqrt(v[k] * v[k + 1])), int(k + 1), v.size


def run_filtered(wl, eps, reduction="mean", weights=None, num=0.0, grad=None, which=3):
    return run_gpu_filtered(wl, eps, reduction, weights, num, grad, which)


def oracle_filtered(wl, eps):
    H, W = wl.H.double().numpy(), wl.W.double().numpy()
    b = None if wl.b is None else wl.b.double().numpy()
    mask = None if wl.mask is None else wl.mask.numpy()
    f = O.dense_forward(H, W, b, wl.labels.numpy(), mask)
    return f, O.filtered_backward(H, W, b, wl.labels.numpy(), f.m, f.logs, eps, 1.0, mask)


@pytest.mark.parametrize("seed", [7, 8])
def test_filtered_matches_oracle_in_a_gap(seed):
    wl = peaked_workload(seed)
    H, W = wl.H.double().numpy(), wl.W.double().numpy()
    b = None if wl.b is None else wl.b.double().numpy()
    mask = None if wl.mask is None else wl.mask.numpy()
    f = O.dense_forward(H, W, b, wl.labels.numpy(), mask)
    eps, dropped, total = gap_eps(block_maxima(wl, f))
    say(f"[filter] seed {seed}: eps {eps:.3e} drops {dropped} of {total} target-free blocks")
    assert 0 < dropped < total
    g = O.filtered_backward(H, W, b, wl.labels.numpy(), f.m, f.logs, eps, 1.0, mask)
    gx = O.dense_backward(H, W, b, wl.labels.numpy(), f.m, f.logs, 1.0, mask)
    st, dH, dW, db = run_filtered(wl, eps)
    assert st == _lib.LCE_OK, _lib.status_string(st)
    t = tol(wl.dtype)
    assert_grad_close("dH filtered", dH, g.dH, t["grad"])
    assert_grad_close("dW filtered", dW, g.dW, t["grad"])
    # the filter really dropped something: dW rows of dropped blocks differ from the exact ones
    assert np.max(np.abs(g.dW - gx.dW)) > 0.0


@pytest.mark.parametrize("reduction", ["sum", "none"])
def test_filtered_row_factors_match_oracle_in_a_gap(reduction):
    """Weighted sum (some weights 0) and none (per-position upstream values,
    some 0 and some negative): rows with factor 0 keep no block alive."""
    wl = peaked_workload(8)
    N = wl.N
    H, W = wl.H.double().numpy(), wl.W.double().numpy()
    b = None if wl.b is None else wl.b.double().numpy()
    mask = None if wl.mask is None else wl.mask.numpy()
    y = wl.labels.numpy()
    f = O.dense_forward(H, W, b, y, mask)
    rng = np.random.default_rng(21)
    if reduction == "sum":
        weights = rng.uniform(0.2, 2.0, N).astype(np.float32)
        weights[rng.random(N) < 0.3] = 0.0
        num, grad = 333.0, 0.75
        r = O.row_factors(N, f.idx, f.C, "sum", float(np.float32(grad)), weights.astype(np.float64), num)
    else:
        weights, num = None, 0.0
        grad = rng.uniform(-2.0, 2.0, N).astype(np.float32)
        grad[rng.random(N) < 0.3] = 0.0
        r = O.row_factors(N, f.idx, f.C, "none", grad.astype(np.float64))
    eps, dropped, total = gap_eps(block_maxima(wl, f, r))
    say(f"[filter] {reduction}: eps {eps:.3e} drops {dropped} of {total} target-free blocks")
    assert 0 < dropped < total
    g = O.filtered_backward(H, W, b, y, f.m, f.logs, eps, mask=mask, row_factor=r)
    gx = O.dense_backward(H, W, b, y, f.m, f.logs, mask=mask, row_factor=r)
    st, dH, dW, db = run_filtered(wl, eps, reduction, weights, num, grad)
    assert st == _lib.LCE_OK, _lib.status_string(st)
    t = tol(wl.dtype)
    assert_grad_close("dH filtered", dH, g.dH, t["grad"])
    assert_grad_close("dW filtered", dW, g.dW, t["grad"])
    assert_grad_close("db (exact)", db, g.db, t["grad"])
    assert np.max(np.abs(g.dW - gx.dW)) > 0.0


def test_filter_dh_only_keeps_dw_exact():
    """The embedding-gradient filter alone (the variant with an exact
    classifier gradient): dH matches the oracle's filtered dH, dW and db are
    bitwise the unfiltered backward's."""
    wl = peaked_workload(7)
    H, W = wl.H.double().numpy(), wl.W.double().numpy()
    b = None if wl.b is None else wl.b.double().numpy()
    mask = None if wl.mask is None else wl.mask.numpy()
    f = O.dense_forward(H, W, b, wl.labels.numpy(), mask)
    eps, _, _ = gap_eps(block_maxima(wl, f))
    g = O.filtered_backward(H, W, b, wl.labels.numpy(), f.m, f.logs, eps, 1.0, mask, filter_dw=False)
    r = run_gpu(wl)
    st, dH, dW, db = run_filtered(wl, eps, which=_lib.LCE_FILTER_DH)
    assert st == _lib.LCE_OK
    t = tol(wl.dtype)
    assert_grad_close("dH filtered", dH, g.dH, t["grad"])
    assert np.max(np.abs(r.dH - dH)) > 0.0
    np.testing.assert_array_equal(dW, r.dW)
    np.testing.assert_array_equal(db, r.db)


def test_filter_mixed_tiles_drop_dead_blocks_exactly():
    """A 256-wide dW tile whose column blocks are partly live: the dead
    blocks' rows of dW are exactly 0 (eps > 1 keeps only blocks holding a
    target), and the live rows match the oracle."""
    wl = WL.make_workload("sft_small")
    f, g = oracle_filtered(wl, 10.0)
    st, dH, dW, db = run_filtered(wl, 10.0)
    assert st == _lib.LCE_OK
    y = wl.labels.numpy()
    live = np.zeros(wl.V, dtype=bool)
    for lo in range(0, f.C, 256):
        for lab in y[f.idx[lo:lo + 256]]:
            live[(lab // 32) * 32:(lab // 32) * 32 + 32] = True
    assert np.all(dW[~live] == 0.0)
    t = tol(wl.dtype)
    assert_grad_close("dW", dW, g.dW, t["grad"])


def test_filter_eps_zero_is_bitwise_the_unfiltered_backward():
    wl = peaked_workload(9)
    r = run_gpu(wl)
    st, dH, dW, db = run_filtered(wl, 0.0)
    assert st == _lib.LCE_OK
    np.testing.assert_array_equal(dH, r.dH)
    np.testing.assert_array_equal(dW, r.dW)


@pytest.mark.parametrize("name", ["page2_small", "sft_small"])
def test_filter_huge_eps_keeps_target_blocks_only(name):
    wl = WL.make_workload(name)
    f, g = oracle_filtered(wl, 10.0)
    st, dH, dW, db = run_filtered(wl, 10.0)
    assert st == _lib.LCE_OK
    t = tol(wl.dtype)
    assert_grad_close("dH", dH, g.dH, t["grad"])
    assert_grad_close("dW", dW, g.dW, t["grad"])
    if wl.b is not None:
        assert_grad_close("db (exact)", db, g.db, t["grad"])


def test_filter_rejects_fp32_and_bad_eps():
    wl = WL.make_workload("tiny")
    st, *_ = run_filtered(wl, 1e-3)
    assert st == _lib.LCE_ERR_UNSUPPORTED


def test_autograd_filter_eps_matches_the_entry_point():
    """linear_cross_entropy(..., filter_eps=e) runs lce_backward_filtered:
    its gradients equal the entry point's bit for bit (deterministic kernels)."""
    from lm_head_projection_amd import linear_cross_entropy
    wl = WL.make_workload("page2_small")
    dev = "cuda:0"
    st, dH0, dW0, db0 = run_filtered(wl, 10.0)
    assert st == _lib.LCE_OK
    H = wl.H.to(dev).requires_grad_(True)
    W = wl.W.to(dev).requires_grad_(True)
    b = wl.b.to(dev).requires_grad_(True)
    loss = linear_cross_entropy(H, W, wl.labels.to(dev), bias=b, mask=wl.mask.to(dev), filter_eps=10.0)
    loss.backward()
    torch.cuda.synchronize()
    np.testing.assert_array_equal(to_np(H.grad), dH0)
    np.testing.assert_array_equal(to_np(W.grad), dW0)
    np.testing.assert_array_equal(to_np(b.grad), db0)


def test_filter_stage_list_overflow_falls_back_exactly():
    """115000 supervised rows: a dW item's live stage list (one entry per 32
    rows) would overflow its LDS capacity, so the kernel runs the full range,
    where dead blocks of G are stored as zeros.  Labels lie in [0, 64) and
    eps = 10, so only the first two column blocks are live: dW rows from 64
    on are exactly 0, and sampled dW and dH rows match the oracle."""
    wl = WL.make_random(115000, 128, 1024, dtype=torch.bfloat16, seed=41, ignore_frac=0.0, bias=False,
                        w_scale=0.02)
    g = torch.Generator().manual_seed(42)
    wl.labels = torch.randint(0, 64, (wl.N,), generator=g)
    say("[filter] 115000 rows, eps 10: GPU")
    st, dH, dW, db = run_filtered(wl, 10.0)
    assert st == _lib.LCE_OK
    assert np.all(dW[64:] == 0.0)
    say("[filter] 115000 rows: oracle statistics and sampled rows")
    Hd, Wd, y = wl.H.double().numpy(), wl.W.double().numpy(), wl.labels.numpy()
    f = O.dense_forward(Hd, Wd, None, y)
    rng = np.random.default_rng(43)
    rows = np.sort(rng.choice(f.idx, 4, replace=False))
    cols = np.array([0, 17, 40, 63])
    dh, dw, _ = O.filtered_rows_grad(Hd, Wd, None, y, f.m, f.logs, 10.0, rows, cols, 1.0)
    t = tol(wl.dtype)
    assert_grad_close("dH rows", dH[rows], dh, t["grad"])
    assert_grad_close("dW rows", dW[cols], dw, t["grad"])
