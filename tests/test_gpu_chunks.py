"""The backward over several vocabulary chunks (at most 32768 entries each),
against the oracle.  In bf16 the gradients of chunk c and the replay of
chunk c+1 share one launch and two G buffers; the replay takes one of four
forms (with or without a bias, with or without the gradient filter), and
each form is run here over three chunks (32768, 32768 and a ragged 4464).
The small parity workloads fit in one chunk and never reach that launch.
"""

import numpy as np
import pytest
import torch

import oracle as O
from lm_head_projection_amd import _lib
from lm_head_projection_amd import workloads as WL

from lce_harness import (assert_grad_close, check_all, oracle_of, run_gpu, run_gpu_filtered, say, tol)

pytestmark = pytest.mark.gpu

V3 = 70000  # three chunks: 32768 + 32768 + 4464


@pytest.mark.parametrize("bias", [False, True])
def test_three_chunks_match_the_oracle(bias):
    """Plain backward (replay forms without and with a bias), on a workspace of
    exactly lce_backward_workspace_size for the supervised count."""
    wl = WL.make_random(700, 128, V3, dtype=torch.bfloat16, seed=41 + int(bias), bias=bias, ignore_frac=0.2,
                        mask_frac=0.05)
    say(f"[chunks] {wl.name} bias={bias}")
    f, g = oracle_of(wl)
    r = run_gpu(wl, exact_ws=True)
    check_all(wl, r, f, g, wl.dtype)


def peaked_chunks(seed):
    """Three probability levels set by the bias (targets in [0, 512) at +4,
    [512, 1024) at +1.5, the rest at -2.5) over three chunks, with small
    scores: the target-free blocks of the two lower bands sit far apart in p."""
    wl = WL.make_random(700, 128, V3, dtype=torch.bfloat16, seed=seed, ignore_frac=0.15, mask_frac=0.05,
                        w_scale=0.02, b_scale=0.05)
    b = wl.b.float()
    b[:512] += 4.0
    b[512:1024] += 1.5
    b[1024:] -= 2.5
    wl.b = b.to(torch.bfloat16)
    gen = torch.Generator().manual_seed(seed + 1)
    keep = wl.labels != wl.ignore_index
    wl.labels[keep] = torch.randint(0, 512, (int(keep.sum()),), generator=gen)
    return wl


def gap_eps(wl, f):
    """An eps at the geometric middle of the widest gap (>= 16x) between the
    largest p of target-free (256-row, 32-column) blocks (oracle values)."""
    H, W = wl.H.double().numpy(), wl.W.double().numpy()
    b = wl.b.double().numpy()
    y = wl.labels.numpy()
    maxima = []
    for lo in range(0, f.C, 256):
        rows = f.idx[lo:lo + 256]
        P = np.exp((O.logits(H[rows], W, b) - f.m[rows][:, None]) - f.logs[rows][:, None])
        Pb = P[:, : (wl.V // 32) * 32].reshape(len(rows), -1, 32).max(axis=(0, 2))
        tail = P[:, (wl.V // 32) * 32:].max() if wl.V % 32 else None
        has_t = np.zeros(Pb.size + (1 if tail is not None else 0), dtype=bool)
        has_t[np.unique(y[rows] // 32)] = True
        vals = np.concatenate([Pb, [tail]]) if tail is not None else Pb
        maxima.append(vals[~has_t])
    v = np.unique(np.concatenate(maxima))
    v = v[v > 0]
    ratios = v[1:] / v[:-1]
    k = int(np.argmax(ratios))
    assert ratios[k] >= 16.0, f"no 16x gap (best {ratios[k]:.2f})"
    return float(np.sqrt(v[k] * v[k + 1]))


@pytest.mark.parametrize("which", [_lib.LCE_FILTER_BOTH, _lib.LCE_FILTER_DH])
def test_three_chunks_filtered_with_bias_match_the_oracle(which):
    """The filter and a bias (the replay form that votes on blocks and forms db
    partials), with dead G blocks zeroed (both gradients filtered) or kept
    (dH only, whose dW stays exact)."""
    wl = peaked_chunks(51)
    H, W = wl.H.double().numpy(), wl.W.double().numpy()
    b = wl.b.double().numpy()
    y = wl.labels.numpy()
    mask = None if wl.mask is None else wl.mask.numpy()
    f = O.dense_forward(H, W, b, y, mask)
    eps = gap_eps(wl, f)
    say(f"[chunks] filtered which={which} eps {eps:.3e}")
    gf = O.filtered_backward(H, W, b, y, f.m, f.logs, eps, 1.0, mask)
    gx = O.dense_backward(H, W, b, y, f.m, f.logs, 1.0, mask)
    st, dH, dW, db = run_gpu_filtered(wl, eps, which=which)
    assert st == _lib.LCE_OK, _lib.status_string(st)
    t = tol(wl.dtype)
    assert_grad_close("dH filtered", dH, gf.dH, t["grad"])
    assert_grad_close("db (exact)", db, gx.db, t["grad"])
    # Every block of the low band (entries 1024 and up, no targets there) lies
    # below eps in every row block: with both gradients filtered those G
    # blocks are stored as zeros and their dW rows come out exactly 0, in all
    # three chunks; the dH-only filter leaves them exact.
    if which == _lib.LCE_FILTER_BOTH:
        assert_grad_close("dW filtered", dW, gf.dW, t["grad"])
        assert np.all(dW[1024:] == 0.0)
        assert np.all(gf.dW[1024:] == 0.0) and np.max(np.abs(gx.dW[1024:])) > 0.0
    else:
        assert_grad_close("dW (exact)", dW, gx.dW, t["grad"])
        assert np.max(np.abs(dW[1024:])) > 0.0
    assert np.max(np.abs(gf.dH - gx.dH)) > 0.0  # something was dropped


def test_three_chunks_filter_without_bias():
    """The filter without a bias (the replay form that votes but forms no db
    partials): eps = 0 is bitwise the unfiltered backward, and eps > 1 keeps
    exactly the blocks that hold a target."""
    wl = WL.make_random(700, 128, V3, dtype=torch.bfloat16, seed=61, bias=False, ignore_frac=0.2)
    r = run_gpu(wl)
    st, dH, dW, _ = run_gpu_filtered(wl, 0.0)
    assert st == _lib.LCE_OK
    np.testing.assert_array_equal(dH, r.dH)
    np.testing.assert_array_equal(dW, r.dW)
    H, W = wl.H.double().numpy(), wl.W.double().numpy()
    y = wl.labels.numpy()
    f = O.dense_forward(H, W, None, y, None)
    gf = O.filtered_backward(H, W, None, y, f.m, f.logs, 10.0, 1.0, None)
    st, dH, dW, _ = run_gpu_filtered(wl, 10.0)
    assert st == _lib.LCE_OK
    t = tol(wl.dtype)
    assert_grad_close("dH", dH, gf.dH, t["grad"])
    assert_grad_close("dW", dW, gf.dW, t["grad"])


@pytest.mark.parametrize("V", [32768, 32769, 65536])
def test_chunk_boundaries(V):
    """One whole chunk (no fused launch), one chunk plus a single entry (the
    fused launch replays a 1-entry chunk of one ragged tile), and two whole
    chunks, with a bias."""
    wl = WL.make_random(300, 64, V, dtype=torch.bfloat16, seed=71, ignore_frac=0.2)
    say(f"[chunks] boundary V={V}")
    f, g = oracle_of(wl)
    r = run_gpu(wl)
    check_all(wl, r, f, g, wl.dtype)


def test_fp32_several_chunks():
    """fp32 keeps separate replay and gradient launches over one G buffer."""
    wl = WL.make_random(200, 64, 40000, dtype=torch.float32, seed=73, ignore_frac=0.2)
    f, g = oracle_of(wl)
    r = run_gpu(wl)
    check_all(wl, r, f, g, wl.dtype)
