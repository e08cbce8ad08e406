"""The no-allocation forward entry (lce_forward_ex_noalloc) through the C
ABI: on two calls in a row, the second on a smaller problem, its outputs are
bit for bit those of lce_forward_ex with a caller workspace, and within the
oracle's tolerance; with every reduction."""

import numpy as np
import pytest
import torch

import oracle as O
from lm_head_projection_amd import _lib
from lm_head_projection_amd import workloads as WL

from lce_harness import assert_stat_close, say, tol

pytestmark = pytest.mark.gpu


def _run(wl, red, noalloc, dev="cuda:0"):
    H, W = wl.H.to(dev), wl.W.to(dev)
    b = None if wl.b is None else wl.b.to(dev)
    labels = wl.labels.to(dev)
    mask = None if wl.mask is None else wl.mask.to(torch.uint8).to(dev)
    N, D = H.shape
    V = W.shape[0]
    ws = torch.empty(_lib.lce_forward_workspace_size(N, D, V, H.dtype), dtype=torch.uint8, device=dev)
    idx = torch.empty(N, dtype=torch.int32, device=dev)
    st, C = _lib.lce_compact_valid(labels, mask, V, wl.ignore_index, idx, ws)
    assert st == _lib.LCE_OK
    rcode = _lib.REDUCTIONS[red]
    w = torch.linspace(0.25, 1.75, N, device=dev) if red == "sum" else None
    num = float(C) if red == "sum" else 0.0
    loss = torch.full((N if red == "none" else 1,), float("nan"), device=dev)
    m = torch.full((N,), 12345.0, device=dev)
    logs = torch.full((N,), 12345.0, device=dev)
    if noalloc:
        del ws  # the entry must not need a caller workspace
        st = _lib.lce_forward_ex_noalloc(H, W, b, labels, idx, C, rcode, w, num, loss, m, logs)
    else:
        st = _lib.lce_forward_ex(H, W, b, labels, idx, C, rcode, w, num, loss, m, logs, ws)
    torch.cuda.synchronize()
    assert st == _lib.LCE_OK, _lib.status_string(st)
    return (loss.cpu().numpy(), m.cpu().numpy(), logs.cpu().numpy(), C,
            None if w is None else w.cpu().numpy().astype(np.float64), num)


@pytest.mark.parametrize("red", ["mean", "sum", "none"])
def test_noalloc_forward_equals_the_workspace_entry_on_two_calls(red):
    for name in ("sft", "packed_small"):  # the second problem is the smaller one
        say(f"[noalloc] {name} {red}")
        wl = WL.make_workload(name)
        ref = _run(wl, red, noalloc=False)
        got = _run(wl, red, noalloc=True)
        for a, b_ in zip(got[:3], ref[:3]):
            np.testing.assert_array_equal(a, b_)
        loss, m, logs, C, w, num = got
        H, W = wl.H.double().numpy(), wl.W.double().numpy()
        b = None if wl.b is None else wl.b.double().numpy()
        f = O.dense_forward(H, W, b, wl.labels.numpy(), None if wl.mask is None else wl.mask.numpy())
        assert C == f.C
        t = tol(wl.dtype)
        want = O.reduce_rows(f.row_loss, f.idx, f.C, red, w, num if num else None)
        if red == "none":
            assert_stat_close("per-position loss", loss[f.idx], want[f.idx], t["stat"])
        else:
            assert abs(loss[0] - want) <= t["loss"] * abs(want)
        assert_stat_close("m", m[f.idx], f.m[f.idx], t["stat"])
        assert_stat_close("logs", logs[f.idx], f.logs[f.idx], t["stat"])
