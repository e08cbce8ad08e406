"""Shared helpers for the GPU tests: run the HIP path through the C ABI on a
workload and compare with the oracle at the stated tolerances.

Tolerances (derived from the arithmetic and the target bar):
  bf16 inputs: loss |L - L*| <= 1e-3 |L*|; m, log s: |x - x*| <= 1e-3 max(1, |x*|);
               dH, dW, db: max |x - x*| <= 1e-2 max |x*|.
  fp32 inputs: every quantity within 1e-5 relative (same forms, r = 1e-5).
"""

from __future__ import annotations

import dataclasses
import sys
from typing import Optional

import numpy as np
import torch

import oracle as O
from lm_head_projection_amd import _lib
from lm_head_projection_amd.workloads import Workload


def tol(dtype):
    if dtype == torch.float32:
        return dict(loss=1e-5, stat=1e-5, grad=1e-5)
    return dict(loss=1e-3, stat=1e-3, grad=1e-2)


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


@dataclasses.dataclass
class GpuResult:
    status_c: int
    C: int
    idx: np.ndarray
    status_f: int
    loss: float
    m: np.ndarray
    logs: np.ndarray
    row_loss: np.ndarray
    status_b: Optional[int] = None
    dH: Optional[np.ndarray] = None
    dW: Optional[np.ndarray] = None
    db: Optional[np.ndarray] = None


def to_np(t):
    return None if t is None else t.detach().to("cpu", torch.float64).numpy()


def run_gpu(wl: Workload, lam: float = 1.0, backward: bool = True, grad_ptr: bool = True,
            dev: str = "cuda:0", keep_device: bool = False, exact_ws: bool = False):
    """compact -> forward -> backward through the C ABI; results on the host.
    exact_ws: one workspace of exactly lce_backward_workspace_size(N, C, ...)
    bytes for the workload's supervised count C (else the worst case C = N)."""
    H = wl.H.to(dev)
    W = wl.W.to(dev)
    b = None if wl.b is None else wl.b.to(dev)
    labels = wl.labels.to(dev)
    mask = None if wl.mask is None else wl.mask.to(torch.uint8).to(dev)
    N, D = H.shape
    V = W.shape[0]
    if exact_ws:
        sup = wl.labels != wl.ignore_index
        if wl.mask is not None:
            sup &= wl.mask.bool()
        nbytes = _lib.lce_backward_workspace_size(N, int(sup.sum()), D, V, H.dtype)
    else:
        nbytes = _lib.lce_workspace_size(N, D, V, H.dtype)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    idx = torch.full((max(N, 1),), -7, dtype=torch.int32, device=dev)
    st_c, C = _lib.lce_compact_valid(labels, mask, V, wl.ignore_index, idx, ws)
    loss = torch.full((1,), float("nan"), dtype=torch.float32, device=dev)
    m = torch.full((N,), 12345.0, dtype=torch.float32, device=dev)
    logs = torch.full((N,), 12345.0, dtype=torch.float32, device=dev)
    row_loss = torch.full((N,), 12345.0, dtype=torch.float32, device=dev)
    st_f = None
    if st_c in (_lib.LCE_OK, _lib.LCE_OK_EMPTY):
        st_f = _lib.lce_forward(H, W, b, labels, idx, C, loss, m, logs, row_loss, ws)
    torch.cuda.synchronize()
    r = GpuResult(st_c, C, idx[:C].cpu().numpy().astype(np.int64), st_f,
                  float(loss.item()), to_np(m), to_np(logs), to_np(row_loss))
    if backward and st_f in (_lib.LCE_OK, _lib.LCE_OK_EMPTY):
        g = torch.tensor([lam], dtype=torch.float32, device=dev) if grad_ptr else None
        dH = torch.full_like(H, 7.0)
        dW = torch.full_like(W, 7.0)
        db = None if b is None else torch.full_like(b, 7.0)
        r.status_b = _lib.lce_backward(H, W, b, labels, idx, C, m, logs, g, dH, dW, db, ws)
        torch.cuda.synchronize()
        if keep_device:
            r.dH, r.dW, r.db = dH, dW, db
        else:
            r.dH, r.dW, r.db = to_np(dH), to_np(dW), to_np(db)
    return r


def max_rel_err(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    scale = np.max(np.abs(ref)) if ref.size else 0.0
    err = np.max(np.abs(x - ref)) if ref.size else 0.0
    return err / scale if scale > 0 else err


def assert_grad_close(name, x, ref, r):
    e = max_rel_err(x, ref)
    assert np.all(np.isfinite(x)), f"{name}: non-finite values"
    assert e <= r, f"{name}: max|x-ref|/max|ref| = {e:.3e} > {r:.1e}"
    return e


def assert_stat_close(name, x, ref, r):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    bound = r * np.maximum(1.0, np.abs(ref))
    bad = np.abs(x - ref) > bound
    assert not np.any(bad), f"{name}: {int(bad.sum())} entries off, worst {np.max(np.abs(x - ref)):.3e}"


@dataclasses.dataclass
class GpuResultEx:
    status_f: int
    loss: np.ndarray            # [1] (mean / sum) or [N] (none)
    m: Optional[np.ndarray]
    logs: Optional[np.ndarray]
    status_b: Optional[int] = None
    dH: Optional[np.ndarray] = None
    dW: Optional[np.ndarray] = None
    db: Optional[np.ndarray] = None
    C: int = 0
    idx: Optional[np.ndarray] = None


def run_gpu_ex(wl: Workload, reduction: str, weights=None, num: float = 0.0, grad=None,
               stats: bool = True, backward: bool = True, dev: str = "cuda:0"):
    """compact -> lce_forward_ex -> lce_backward_ex through the C ABI.

    weights: float[N] (host, numpy) or None; grad: None, a scalar (mean/sum)
    or a float[N] array (none)."""
    H = wl.H.to(dev)
    W = wl.W.to(dev)
    b = None if wl.b is None else wl.b.to(dev)
    labels = wl.labels.to(dev)
    mask = None if wl.mask is None else wl.mask.to(torch.uint8).to(dev)
    N, D = H.shape
    V = W.shape[0]
    red = _lib.REDUCTIONS[reduction]
    ws = torch.empty(_lib.lce_workspace_size(N, D, V, H.dtype), dtype=torch.uint8, device=dev)
    idx = torch.full((max(N, 1),), -7, dtype=torch.int32, device=dev)
    st_c, C = _lib.lce_compact_valid(labels, mask, V, wl.ignore_index, idx, ws)
    assert st_c in (_lib.LCE_OK, _lib.LCE_OK_EMPTY), st_c
    w = None if weights is None else torch.tensor(weights, dtype=torch.float32, device=dev)
    loss = torch.full((N if red == _lib.LCE_REDUCTION_NONE else 1,), float("nan"), dtype=torch.float32,
                      device=dev)
    m = torch.full((N,), 12345.0, dtype=torch.float32, device=dev) if stats else None
    logs = torch.full((N,), 12345.0, dtype=torch.float32, device=dev) if stats else None
    st_f = _lib.lce_forward_ex(H, W, b, labels, idx, C, red, w, num, loss, m, logs, ws)
    torch.cuda.synchronize()
    r = GpuResultEx(st_f, to_np(loss), to_np(m), to_np(logs), C=C,
                    idx=idx[:C].cpu().numpy().astype(np.int64))
    if backward and stats and st_f in (_lib.LCE_OK, _lib.LCE_OK_EMPTY):
        g = None
        if grad is not None:
            g = torch.tensor(np.atleast_1d(np.asarray(grad, dtype=np.float32)), device=dev)
        dH = torch.full_like(H, 7.0)
        dW = torch.full_like(W, 7.0)
        db = None if b is None else torch.full_like(b, 7.0)
        r.status_b = _lib.lce_backward_ex(H, W, b, labels, idx, C, red, w, num, m, logs, g, dH, dW, db, ws)
        torch.cuda.synchronize()
        r.dH, r.dW, r.db = to_np(dH), to_np(dW), to_np(db)
    return r


def run_gpu_filtered(wl: Workload, eps: float, reduction: str = "mean", weights=None, num: float = 0.0,
                     grad=None, which: int = 3, dev: str = "cuda:0"):
    """compact -> lce_forward -> lce_backward_filtered through the C ABI.
    Returns (status, dH, dW, db) as host arrays."""
    H = wl.H.to(dev)
    W = wl.W.to(dev)
    b = None if wl.b is None else wl.b.to(dev)
    labels = wl.labels.to(dev)
    mask = None if wl.mask is None else wl.mask.to(torch.uint8).to(dev)
    N, D = H.shape
    V = W.shape[0]
    ws = torch.empty(_lib.lce_workspace_size(N, D, V, H.dtype), dtype=torch.uint8, device=dev)
    idx = torch.empty(max(N, 1), dtype=torch.int32, device=dev)
    st, C = _lib.lce_compact_valid(labels, mask, V, wl.ignore_index, idx, ws)
    assert st == _lib.LCE_OK
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    m = torch.empty(N, dtype=torch.float32, device=dev)
    logs = torch.empty(N, dtype=torch.float32, device=dev)
    assert _lib.lce_forward(H, W, b, labels, idx, C, loss, m, logs, None, ws) == _lib.LCE_OK
    dH = torch.full_like(H, 7.0)
    dW = torch.full_like(W, 7.0)
    db = None if b is None else torch.full_like(b, 7.0)
    g = torch.tensor(np.atleast_1d(np.asarray(1.0 if grad is None else grad, dtype=np.float32)), device=dev)
    w = None if weights is None else torch.tensor(weights, dtype=torch.float32, device=dev)
    st = _lib.lce_backward_filtered(H, W, b, labels, idx, C, _lib.REDUCTIONS[reduction], w, num, m, logs, g, eps,
                                    dH, dW, db, ws, which=which)
    torch.cuda.synchronize()
    return st, to_np(dH), to_np(dW), to_np(db)


def oracle_of(wl, lam=1.0):
    """The oracle's dense forward and backward of a workload (float64)."""
    H, W = wl.H.double().numpy(), wl.W.double().numpy()
    b = None if wl.b is None else wl.b.double().numpy()
    mask = None if wl.mask is None else wl.mask.numpy()
    return O.dense_forward_backward(H, W, b, wl.labels.numpy(), mask, lam, wl.ignore_index)


def check_all(wl, r, f, g, dtype):
    """Every output of run_gpu against the oracle (f, g) at the stated tolerances."""
    t = tol(dtype)
    assert r.status_c == _lib.LCE_OK, r.status_c
    assert r.C == f.C
    np.testing.assert_array_equal(r.idx, f.idx)
    assert r.status_f == _lib.LCE_OK
    assert abs(r.loss - f.loss) <= t["loss"] * abs(f.loss), (r.loss, f.loss)
    a = np.zeros(wl.N, dtype=bool)
    a[f.idx] = True
    assert_stat_close("m", r.m[a], f.m[a], t["stat"])
    assert_stat_close("logs", r.logs[a], f.logs[a], t["stat"])
    assert_stat_close("row_loss", r.row_loss[a], f.row_loss[a], t["stat"])
    assert np.all(np.isneginf(r.m[~a])) and np.all(np.isneginf(r.logs[~a]))
    assert np.all(r.row_loss[~a] == 0.0)
    assert r.status_b == _lib.LCE_OK
    assert_grad_close("dH", r.dH, g.dH, t["grad"])
    assert np.all(r.dH[~a] == 0.0), "unsupervised dH rows must be exactly 0"
    assert_grad_close("dW", r.dW, g.dW, t["grad"])
    if wl.b is not None:
        assert_grad_close("db", r.db, g.db, t["grad"])
