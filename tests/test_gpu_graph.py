"""A HIP graph of the no-allocation forward (lce_forward_ex_noalloc) and the
backward on a workspace allocated beforehand, over three vocabulary chunks
(so the graph holds the fused gradient-and-replay launches): each of three
replays, with eager work and synchronisations between them, reproduces the
eager outputs bit for bit, and those match the oracle."""

import numpy as np
import pytest
import torch

from lm_head_projection_amd import _lib
from lm_head_projection_amd import workloads as WL

from lce_harness import assert_grad_close, assert_stat_close, oracle_of, say, tol

pytestmark = pytest.mark.gpu


def test_graph_replays_the_noalloc_forward_and_the_backward():
    dev = "cuda:0"
    wl = WL.make_random(600, 128, 70000, dtype=torch.bfloat16, seed=81, ignore_frac=0.2)
    H, W, b = wl.H.to(dev), wl.W.to(dev), wl.b.to(dev)
    labels = wl.labels.to(dev)
    N, D = H.shape
    V = W.shape[0]
    idx = torch.empty(N, dtype=torch.int32, device=dev)
    ws_f = torch.empty(_lib.lce_forward_workspace_size(N, D, V, H.dtype), dtype=torch.uint8, device=dev)
    st, C = _lib.lce_compact_valid(labels, None, V, wl.ignore_index, idx, ws_f)
    assert st == _lib.LCE_OK
    ws = torch.empty(_lib.lce_backward_workspace_size(N, C, D, V, H.dtype), dtype=torch.uint8, device=dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    m = torch.empty(N, dtype=torch.float32, device=dev)
    logs = torch.empty(N, dtype=torch.float32, device=dev)
    grad = torch.ones(1, dtype=torch.float32, device=dev)
    dH, dW, db = torch.empty_like(H), torch.empty_like(W), torch.empty_like(b)
    outs = (loss, m, logs, dH, dW, db)

    def step():
        s1 = _lib.lce_forward_ex_noalloc(H, W, b, labels, idx, C, _lib.LCE_REDUCTION_MEAN, None, 0.0, loss, m, logs)
        s2 = _lib.lce_backward(H, W, b, labels, idx, C, m, logs, grad, dH, dW, db, ws)
        return s1, s2

    # Eager first: it also resolves the static scratch's address outside capture.
    assert step() == (_lib.LCE_OK, _lib.LCE_OK)
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        captured = step()
    assert captured == (_lib.LCE_OK, _lib.LCE_OK)
    for rep in range(3):
        for t in outs:
            t.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(f"[graph] replay {rep}")
        for name, t, r in zip(("loss", "m", "logs", "dH", "dW", "db"), outs, ref):
            assert torch.equal(t, r), f"replay {rep}: {name} differs from the eager run"

    f, gr = oracle_of(wl)
    t = tol(wl.dtype)
    assert C == f.C
    assert abs(float(ref[0].item()) - f.loss) <= t["loss"] * abs(f.loss)
    a = np.zeros(N, dtype=bool)
    a[f.idx] = True
    assert_stat_close("m", ref[1].cpu().double().numpy()[a], f.m[a], t["stat"])
    assert_stat_close("logs", ref[2].cpu().double().numpy()[a], f.logs[a], t["stat"])
    assert_grad_close("dH", ref[3].cpu().double().numpy(), gr.dH, t["grad"])
    assert_grad_close("dW", ref[4].cpu().double().numpy(), gr.dW, t["grad"])
    assert_grad_close("db", ref[5].cpu().double().numpy(), gr.db, t["grad"])
