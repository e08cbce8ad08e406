"""HIP path vs the float64 oracle, element by element, through the C ABI.

Sizes: the reduced workloads span several tiles in both axes and end in ragged
tails (N and V not multiples of the 256-wide tiles); the tiny fp32 case is the
exactness case.  Full-size workloads are covered in test_gpu_fullsize.py.
"""

import math

import numpy as np
import pytest
import torch

import oracle as O
from lm_head_projection_amd import _lib
from lm_head_projection_amd import workloads as WL

from lce_harness import (assert_grad_close, assert_stat_close, check_all, oracle_of, run_gpu, say, tol)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", WL.SMALL_CONFIGS)
def test_parity_small_workloads(name):
    say(f"[parity] {name}")
    wl = WL.make_workload(name)
    f, g = oracle_of(wl)
    r = run_gpu(wl)
    check_all(wl, r, f, g, wl.dtype)


@pytest.mark.parametrize("lam", [-2.5, 0.0, 3.0])
def test_upstream_gradient(lam):
    say(f"[parity] lambda={lam}")
    wl = WL.make_workload("page2_small")
    f, g = oracle_of(wl, lam)
    r = run_gpu(wl, lam=lam)
    if lam == 0.0:
        assert r.status_b == _lib.LCE_OK
        assert np.all(r.dH == 0) and np.all(r.dW == 0) and np.all(r.db == 0)
        assert abs(r.loss - f.loss) <= 1e-3 * abs(f.loss)
    else:
        check_all(wl, r, f, g, wl.dtype)


def test_null_grad_pointer_means_one():
    wl = WL.make_workload("sft_small")
    f, g = oracle_of(wl, 1.0)
    r = run_gpu(wl, grad_ptr=False)
    check_all(wl, r, f, g, wl.dtype)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("shape", [(1, 8, 1), (3, 16, 5), (37, 64, 300), (300, 96, 257), (257, 40, 1000)])
def test_odd_shapes(dtype, shape):
    N, D, V = shape
    say(f"[parity] odd shape N={N} D={D} V={V} {dtype}")
    wl = WL.make_random(N, D, V, dtype=dtype, seed=N * 7 + V, ignore_frac=0.2 if N > 2 else 0.0,
                        mask_frac=0.1 if N > 10 else 0.0)
    if V == 1:
        wl.labels[wl.labels != -100] = 0
    f, g = oracle_of(wl)
    r = run_gpu(wl)
    check_all(wl, r, f, g, dtype)


@pytest.mark.parametrize("where", ["first", "last", "tail_tile", "tile_edges"])
def test_target_positions(where):
    """Targets at j=0, j=V-1, inside the ragged last tile, and at tile edges."""
    wl = WL.make_random(64, 64, 700, dtype=torch.float32, seed=5, ignore_frac=0.0)
    V = 700
    if where == "first":
        wl.labels[:] = 0
    elif where == "last":
        wl.labels[:] = V - 1
    elif where == "tail_tile":
        wl.labels[:] = torch.arange(64) % (V - 512) + 512
    else:
        edges = torch.tensor([0, 31, 32, 63, 64, 127, 128, 255, 256, 511, 512, 699])
        wl.labels[:] = edges[torch.arange(64) % edges.numel()]
    f, g = oracle_of(wl)
    r = run_gpu(wl)
    check_all(wl, r, f, g, torch.float32)


def test_large_common_shift_and_late_max():
    """+30 bias on 1 % of rows, plus a +1000 common shift on every score."""
    wl = WL.make_workload("stress_small")
    f, g = oracle_of(wl)
    r = run_gpu(wl)
    check_all(wl, r, f, g, wl.dtype)
    wl2 = WL.make_random(128, 64, 3000, dtype=torch.float32, seed=9)
    wl2.b += 1000.0
    f2, g2 = oracle_of(wl2)
    r2 = run_gpu(wl2)
    check_all(wl2, r2, f2, g2, torch.float32)


def test_empty_supervision():
    """C = 0: zero sentinel, m = log s = -inf, gradients exactly zero."""
    wl = WL.make_workload("sft_small")
    wl.labels[:] = -100
    r = run_gpu(wl)
    assert r.status_c == _lib.LCE_OK_EMPTY and r.C == 0
    assert r.status_f == _lib.LCE_OK_EMPTY and r.loss == 0.0
    assert np.all(np.isneginf(r.m)) and np.all(np.isneginf(r.logs))
    assert r.status_b == _lib.LCE_OK_EMPTY
    assert np.all(r.dH == 0) and np.all(r.dW == 0)
    wl2 = WL.make_workload("page2_small")
    wl2.mask[:] = False
    r2 = run_gpu(wl2)
    assert r2.C == 0 and r2.status_b == _lib.LCE_OK_EMPTY
    assert np.all(r2.db == 0) and np.all(r2.dW == 0) and np.all(r2.dH == 0)


def test_compaction_bit_exact_and_errors():
    for name in WL.SMALL_CONFIGS:
        wl = WL.make_workload(name)
        _, idx, C = O.supervised_rows(wl.labels.numpy(), None if wl.mask is None else wl.mask.numpy())
        r = run_gpu(wl, backward=False)
        assert r.C == C
        np.testing.assert_array_equal(r.idx, idx)
    # ignore_index other than -100
    wl = WL.make_random(1000, 8, 50, seed=3, ignore_frac=0.0)
    wl.ignore_index = 7
    _, idx, C = O.supervised_rows(wl.labels.numpy(), None, 7)
    r = run_gpu(wl, backward=False)
    assert r.C == C and np.array_equal(r.idx, idx)
    # out-of-range supervised label -> LCE_ERR_LABEL; unsupervised rows may hold anything
    wl = WL.make_random(300, 8, 50, seed=4, ignore_frac=0.0)
    wl.labels[123] = 50
    r = run_gpu(wl, backward=False)
    assert r.status_c == _lib.LCE_ERR_LABEL
    wl.labels[123] = -5
    assert run_gpu(wl, backward=False).status_c == _lib.LCE_ERR_LABEL
    wl.mask = torch.ones(300, dtype=torch.bool)
    wl.mask[123] = False
    r = run_gpu(wl, backward=False)
    assert r.status_c == _lib.LCE_OK and r.C == 299


@pytest.mark.parametrize("N", [1, 8191, 8192, 8193, 65536, 65537, 200003])
def test_compaction_sizes_bit_exact(N):
    """Both compaction paths (one workgroup up to 65536 positions, three
    launches above) at the boundaries of the one-workgroup rounds (8192
    positions) and of the switch: indices and C bit-exact with the oracle,
    entries past C untouched, and a bad label at the last position caught."""
    say(f"[compaction] N={N}")
    g = torch.Generator().manual_seed(7000 + N)
    V = 1000
    labels = torch.randint(0, V, (N,), generator=g, dtype=torch.int64)
    labels[torch.rand(N, generator=g) < 0.3] = -100
    mask = (torch.rand(N, generator=g) < 0.9).to(torch.uint8)
    _, idx, C = O.supervised_rows(labels.numpy(), mask.numpy())
    dev = "cuda:0"
    ws = torch.empty(_lib.lce_forward_workspace_size(N, 8, V, torch.bfloat16), dtype=torch.uint8, device=dev)
    out = torch.full((N,), -7, dtype=torch.int32, device=dev)
    st, c = _lib.lce_compact_valid(labels.to(dev), mask.to(dev), V, -100, out, ws)
    assert st == (_lib.LCE_OK if C > 0 else _lib.LCE_OK_EMPTY) and c == C
    got = out.cpu().numpy()
    np.testing.assert_array_equal(got[:C], idx)
    assert np.all(got[C:] == -7)
    bad, mb = labels.clone(), mask.clone()
    bad[N - 1], mb[N - 1] = V, 1
    st, _ = _lib.lce_compact_valid(bad.to(dev), mb.to(dev), V, -100, out, ws)
    assert st == _lib.LCE_ERR_LABEL


def test_nan_propagates():
    wl = WL.make_random(64, 32, 500, dtype=torch.float32, seed=11, ignore_frac=0.0)
    wl.H[5, 3] = float("nan")
    r = run_gpu(wl)
    assert math.isnan(r.loss)


def test_determinism_bitwise():
    """Two runs (one on a second stream) give bitwise-identical outputs."""
    wl = WL.make_workload("packed_small")
    r1 = run_gpu(wl, keep_device=True)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        r2 = run_gpu(wl, keep_device=True)
    s.synchronize()
    assert r1.loss == r2.loss
    assert np.array_equal(r1.m, r2.m) and np.array_equal(r1.logs, r2.logs)
    assert torch.equal(r1.dH, r2.dH) and torch.equal(r1.dW, r2.dW)


def test_inputs_not_mutated():
    wl = WL.make_workload("page2_small")
    dev = "cuda:0"
    H, W, b = wl.H.to(dev), wl.W.to(dev), wl.b.to(dev)
    labels, mask = wl.labels.to(dev), wl.mask.to(dev)
    copies = [t.clone() for t in (H, W, b, labels, mask)]
    from lm_head_projection_amd.functional import linear_cross_entropy
    Hr, Wr, br = H.clone().requires_grad_(True), W.clone().requires_grad_(True), b.clone().requires_grad_(True)
    loss = linear_cross_entropy(Hr, Wr, labels, bias=br, mask=mask)
    loss.backward()
    for t, c in zip((Hr.detach(), Wr.detach(), br.detach(), labels, mask), copies):
        assert torch.equal(t, c)


def test_autograd_wrapper_matches_oracle():
    wl = WL.make_workload("page2_small")
    dev = "cuda:0"
    from lm_head_projection_amd.functional import linear_cross_entropy
    H = wl.H.to(dev).requires_grad_(True)
    W = wl.W.to(dev).requires_grad_(True)
    b = wl.b.to(dev).requires_grad_(True)
    loss = linear_cross_entropy(H, W, wl.labels.to(dev), bias=b, mask=wl.mask.to(dev))
    (2.0 * loss).backward()
    f, g = oracle_of(wl, 2.0)
    assert abs(loss.item() - f.loss) <= 1e-3 * abs(f.loss)
    assert_grad_close("dH", H.grad.double().cpu().numpy(), g.dH, 1e-2)
    assert_grad_close("dW", W.grad.double().cpu().numpy(), g.dW, 1e-2)
    assert_grad_close("db", b.grad.double().cpu().numpy(), g.db, 1e-2)


def test_host_argument_errors():
    dev = "cuda:0"
    wl = WL.make_workload("tiny")
    H, W = wl.H.to(dev), wl.W.to(dev)
    labels = wl.labels.to(dev)
    N, D = H.shape
    V = W.shape[0]
    ws = torch.empty(_lib.lce_workspace_size(N, D, V, H.dtype), dtype=torch.uint8, device=dev)
    idx = torch.empty(N, dtype=torch.int32, device=dev)
    st, C = _lib.lce_compact_valid(labels, None, V, -100, idx, ws)
    assert st == _lib.LCE_OK
    loss = torch.empty(1, device=dev)
    m = torch.empty(N, device=dev)
    logs = torch.empty(N, device=dev)
    small = ws[:1024]
    assert _lib.lce_forward(H, W, None, labels, idx, C, loss, m, logs, None, small) == _lib.LCE_ERR_WORKSPACE
    assert _lib.lce_forward(H, W, None, labels, idx, N + 1, loss, m, logs, None, ws) == _lib.LCE_ERR_ARG
    Hodd = torch.zeros(N, 6, device=dev)
    Wodd = torch.zeros(V, 6, device=dev)
    assert _lib.lce_forward(Hodd, Wodd, None, labels, idx, C, loss, m, logs, None, ws) == _lib.LCE_ERR_UNSUPPORTED


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_no_positions_at_all(dtype):
    """N = 0 (an empty batch, not only C = 0): the loss is exactly 0 and the
    gradients are exactly 0 (dH is empty), through the autograd wrapper."""
    from lm_head_projection_amd import linear_cross_entropy
    dev = "cuda:0"
    g = torch.Generator().manual_seed(5)
    H = torch.zeros(0, 64, dtype=dtype, device=dev, requires_grad=True)
    W = (0.02 * torch.randn(300, 64, generator=g)).to(dtype).to(dev).requires_grad_(True)
    b = (0.01 * torch.randn(300, generator=g)).to(dtype).to(dev).requires_grad_(True)
    labels = torch.zeros(0, dtype=torch.int64, device=dev)
    loss = linear_cross_entropy(H, W, labels, bias=b)
    loss.backward()
    torch.cuda.synchronize()
    assert loss.item() == 0.0
    assert H.grad.shape == (0, 64)
    assert torch.count_nonzero(W.grad).item() == 0 and torch.count_nonzero(b.grad).item() == 0


def test_unsupported_shape_is_refused():
    """bf16 rows must be whole 16-byte vectors (D a multiple of 8): D = 12 is
    refused with LCE_ERR_UNSUPPORTED before any kernel runs."""
    from lm_head_projection_amd import linear_cross_entropy
    dev = "cuda:0"
    H = torch.randn(16, 12, device=dev).to(torch.bfloat16)
    W = torch.randn(40, 12, device=dev).to(torch.bfloat16)
    labels = torch.randint(0, 40, (16,), device=dev)
    with pytest.raises(_lib.LCEError) as e:
        linear_cross_entropy(H, W, labels)
    assert e.value.status == _lib.LCE_ERR_UNSUPPORTED


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_many_positions_narrow_chunks(dtype):
    """N = 40000 positions: the padded rows (40192) cap one chunk of the
    gradient tile store at 2 GB of 32-bit buffer offsets, so the backward
    runs in chunks of 26624 (bf16) or 13312 (fp32) vocabulary entries, a
    width that is no power of two, with a ragged last chunk.  64 supervised
    rows keep the oracle cheap; every output element is checked."""
    wl = WL.make_random(40000, 256, 60000, dtype=dtype, seed=31, ignore_frac=0.1)
    sub = WL.supervised_subset(wl, 64)
    say(f"[parity] N=40000 D=256 V=60000 {dtype}: 64 supervised rows")
    r = run_gpu(sub)
    Hd, Wd = sub.H.double().numpy(), sub.W.double().numpy()
    bd = sub.b.double().numpy()
    f, g = O.dense_forward_backward(Hd, Wd, bd, sub.labels.numpy(), sub.mask.numpy(), 1.0)
    t = tol(dtype)
    assert r.C == f.C == 64
    assert abs(r.loss - f.loss) <= t["loss"] * abs(f.loss)
    assert_stat_close("m", r.m[f.idx], f.m[f.idx], t["stat"])
    assert_stat_close("logs", r.logs[f.idx], f.logs[f.idx], t["stat"])
    assert_grad_close("dH", r.dH, g.dH, t["grad"])
    assert_grad_close("dW", r.dW, g.dW, t["grad"])
    assert_grad_close("db", r.db, g.db, t["grad"])
