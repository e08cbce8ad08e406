"""The library's launch profiler (lce_profile_*), which bench.py's roofline
reads: over a compaction, forward and backward across three vocabulary
chunks, the kernels launched and their algorithmic flops.  bf16 runs the
first chunk's replay alone, then one fused gradient-and-replay launch per
following chunk, then the last chunk's gradients; fp32 keeps the replay and
gradient launches apart.  The flops of each GEMM launch are 2 C D V_k
(logits over V_k entries) and 4 C D V_k (dH and dW of a chunk of V_k), and
a step's total is 8 C D V."""

import numpy as np
import pytest
import torch

from lm_head_projection_amd import _lib
from lm_head_projection_amd import workloads as WL

from lce_harness import run_gpu, say

pytestmark = pytest.mark.gpu

CHUNKS = [32768, 32768, 4464]  # V = 70000 in entries of at most 32768


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_profile_reports_the_launches_and_their_flops(dtype):
    V = sum(CHUNKS)
    wl = WL.make_random(500, 64, V, dtype=dtype, seed=91, ignore_frac=0.2)
    C = int((wl.labels != wl.ignore_index).sum())
    N, D = wl.N, wl.D
    _lib.profile_start(4096)
    try:
        r = run_gpu(wl)
    finally:
        prof = _lib.profile_stop()
    assert r.status_b == _lib.LCE_OK
    say(f"[profile] {dtype}: " + ", ".join(f"{k} x{v[1]}" for k, v in prof.items()))
    launches = {k: v[1] for k, v in prof.items()}
    flops = {k: v[2] for k, v in prof.items()}
    assert launches["k_fwd"] == 1 and flops["k_fwd"] == pytest.approx(2.0 * C * D * V, rel=1e-12)
    if dtype == torch.bfloat16:
        assert launches["k_replay"] == 1 and launches["k_grad_replay"] == 2 and launches["k_grad"] == 1
        assert flops["k_replay"] == pytest.approx(2.0 * C * D * CHUNKS[0], rel=1e-12)
        assert flops["k_grad_replay"] == pytest.approx(
            4.0 * C * D * (CHUNKS[0] + CHUNKS[1]) + 2.0 * C * D * (CHUNKS[1] + CHUNKS[2]), rel=1e-12)
        assert flops["k_grad"] == pytest.approx(4.0 * C * D * CHUNKS[2], rel=1e-12)
    else:
        assert "k_grad_replay" not in launches
        assert launches["k_replay"] == 3 and launches["k_grad"] == 3
        assert flops["k_replay"] == pytest.approx(2.0 * C * D * V, rel=1e-12)
        assert flops["k_grad"] == pytest.approx(4.0 * C * D * V, rel=1e-12)
    # the kernels outside the GEMMs report none; the step's total is 8 C D V
    assert all(f == 0.0 for k, f in flops.items() if k not in ("k_fwd", "k_replay", "k_grad", "k_grad_replay"))
    assert sum(flops.values()) == pytest.approx(8.0 * C * D * V, rel=1e-12)
    assert all(v[0] > 0.0 for v in prof.values())
