"""Seeded synthetic inputs for the fused linear-cross-entropy workloads.

This module only draws random inputs.  It holds none of the loss arithmetic,
so both the float64 oracle (through the tests) and the HIP path consume the
very same tensors from here.

Workload shapes follow the pages' own examples:

* "tiny"   : the exactness case (fp32, bias, 25 % ignored labels).
* "sft"    : short-sequence SFT; the first 40 % of positions are prompt
             tokens labelled ignore (ChunkedLinearCrossEntropy page, section
             on filtering prompt tokens).
* "page2"  : the 8,192 x 131,072 example of the exact chunked-CE page
             (section 05, the FP16 logits ledger), bias, random 90 % mask,
             Zipf(1.1) labels.
* "packed" : a 16k packed sequence with vocab 248,320 (ChunkedLinearCrossEntropy
             page, problem statement), 8 documents, first 30 % of each document
             ignored, Zipf(1.1) labels.
* "stress" : large hidden size, +30 added to the bias of 1 % of vocabulary
             rows so the running max must be rescaled late.

Every "<name>_small" variant keeps the structure (bias, mask, ignore pattern,
label law) at a size a CPU float64 oracle finishes in a second or two, with
ragged tails in both the position and the vocabulary axes.

Recipe (all draws on one ``torch.Generator('cpu')`` seeded with 1000+k for the
k-th workload, small variants use 2000+k):

1. normals are drawn in fp32, scaled, then rounded to nearest-even to the
   workload dtype (bf16 or fp32);
2. integer labels come from ``randint``/``randperm`` on the same generator;
3. Zipf(s) labels use the finite inverse CDF: P(id=k) proportional to
   (k+1)^-s for k in [0, V), a float64 cumulative sum and ``searchsorted`` of
   uniform draws; the id is the rank (no permutation);
4. percentages are exact counts floor(p * N), positions chosen by ``randperm``.
"""

from __future__ import annotations

import dataclasses
import hashlib
from typing import Optional

import numpy as np
import torch

IGNORE_INDEX = -100


@dataclasses.dataclass
class Workload:
    name: str
    H: torch.Tensor                # [N, D] (bf16 or fp32, CPU)
    W: torch.Tensor                # [V, D]
    b: Optional[torch.Tensor]      # [V] or None
    labels: torch.Tensor           # [N] int64
    mask: Optional[torch.Tensor]   # [N] bool or None (None = all True)
    ignore_index: int = IGNORE_INDEX
    lam: float = 1.0

    @property
    def N(self) -> int:
        return self.H.shape[0]

    @property
    def D(self) -> int:
        return self.H.shape[1]

    @property
    def V(self) -> int:
        return self.W.shape[0]

    @property
    def dtype(self) -> torch.dtype:
        return self.H.dtype

    def sha256(self) -> dict:
        out = {}
        for k in ("H", "W", "b", "labels", "mask"):
            t = getattr(self, k)
            if t is None:
                out[k] = None
                continue
            raw = t.contiguous().view(torch.uint8) if t.dtype != torch.bool else t.to(torch.uint8)
            out[k] = hashlib.sha256(raw.numpy().tobytes()).hexdigest()
        return out


# Shapes: (N, D, V, dtype)
SHAPES = {
    "tiny": (64, 128, 1000, torch.float32),
    "sft": (2048, 1024, 151936, torch.bfloat16),
    "page2": (8192, 2048, 131072, torch.bfloat16),
    "packed": (16384, 1024, 248320, torch.bfloat16),
    "stress": (32768, 4096, 248320, torch.bfloat16),
    # Reduced sizes with the same structure; V and N are deliberately ragged.
    "sft_small": (384, 256, 5000, torch.bfloat16),
    "page2_small": (520, 256, 4099, torch.bfloat16),
    "packed_small": (1029, 128, 7777, torch.bfloat16),
    "stress_small": (600, 512, 3001, torch.bfloat16),
}

SEEDS = {"tiny": 1001, "sft": 1002, "page2": 1003, "packed": 1004, "stress": 1005,
         "sft_small": 2002, "page2_small": 2003, "packed_small": 2004, "stress_small": 2005}

FULL_CONFIGS = ("tiny", "sft", "page2", "packed", "stress")
SMALL_CONFIGS = ("tiny", "sft_small", "page2_small", "packed_small", "stress_small")


def _normal(g: torch.Generator, shape, scale: float, dtype: torch.dtype) -> torch.Tensor:
    x = torch.randn(*shape, generator=g, dtype=torch.float32)
    if scale != 1.0:
        x.mul_(scale)
    return x.to(dtype)


def zipf_labels(g: torch.Generator, n: int, V: int, s: float = 1.1) -> torch.Tensor:
    """n draws of a finite Zipf(s) law over [0, V) by inverse CDF."""
    ranks = np.arange(1, V + 1, dtype=np.float64)
    cdf = np.cumsum(ranks ** (-s))
    cdf /= cdf[-1]
    u = torch.rand(n, generator=g, dtype=torch.float64).numpy()
    ids = np.searchsorted(cdf, u, side="right")
    ids = np.minimum(ids, V - 1)
    return torch.from_numpy(ids.astype(np.int64))


def _base(name: str):
    base = name[:-6] if name.endswith("_small") else name
    return base


def make_workload(name: str, seed: Optional[int] = None) -> Workload:
    """Builds workload ``name`` (see module docstring) deterministically."""
    if name not in SHAPES:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(SHAPES)}")
    N, D, V, dt = SHAPES[name]
    g = torch.Generator("cpu")
    g.manual_seed(SEEDS[name] if seed is None else seed)
    base = _base(name)
    b = None
    mask = None
    if base == "tiny":
        H = _normal(g, (N, D), 0.02, dt)
        W = _normal(g, (V, D), 0.02, dt)
        b = _normal(g, (V,), 0.01, dt)
        labels = torch.randint(0, V, (N,), generator=g, dtype=torch.int64)
        ign = torch.randperm(N, generator=g)[: (N * 25) // 100]
        labels[ign] = IGNORE_INDEX
        mask = torch.ones(N, dtype=torch.bool)
    elif base == "sft":
        H = _normal(g, (N, D), 1.0, dt)
        W = _normal(g, (V, D), 0.02, dt)
        labels = torch.randint(0, V, (N,), generator=g, dtype=torch.int64)
        labels[: (N * 40) // 100] = IGNORE_INDEX
    elif base == "page2":
        H = _normal(g, (N, D), 1.0, dt)
        W = _normal(g, (V, D), 0.02, dt)
        b = _normal(g, (V,), 0.01, dt)
        labels = zipf_labels(g, N, V, 1.1)
        mask = torch.zeros(N, dtype=torch.bool)
        mask[torch.randperm(N, generator=g)[: (N * 90) // 100]] = True
    elif base == "packed":
        H = _normal(g, (N, D), 1.0, dt)
        W = _normal(g, (V, D), 0.02, dt)
        cuts = torch.sort(torch.randperm(N - 1, generator=g)[:7] + 1).values.tolist()
        bounds = [0] + cuts + [N]
        labels = zipf_labels(g, N, V, 1.1)
        for k in range(8):
            lo, hi = bounds[k], bounds[k + 1]
            labels[lo: lo + ((hi - lo) * 30) // 100] = IGNORE_INDEX
    elif base == "stress":
        H = _normal(g, (N, D), 1.0, dt)
        W = _normal(g, (V, D), 0.015, dt)
        b = torch.zeros(V, dtype=dt)
        b[torch.randperm(V, generator=g)[: V // 100]] = 30.0
        labels = torch.randint(0, V, (N,), generator=g, dtype=torch.int64)
        labels[torch.randperm(N, generator=g)[: (N * 20) // 100]] = IGNORE_INDEX
    else:  # pragma: no cover
        raise KeyError(name)
    return Workload(name=name, H=H, W=W, b=b, labels=labels, mask=mask)


def make_random(N: int, D: int, V: int, *, dtype=torch.float32, seed: int = 0,
                bias: bool = True, ignore_frac: float = 0.25, mask_frac: float = 0.0,
                h_scale: float = 1.0, w_scale: float = 0.05, b_scale: float = 0.1) -> Workload:
    """A generic seeded case for edge tests (any N, D, V)."""
    g = torch.Generator("cpu")
    g.manual_seed(seed)
    H = _normal(g, (N, D), h_scale, dtype)
    W = _normal(g, (V, D), w_scale, dtype)
    b = _normal(g, (V,), b_scale, dtype) if bias else None
    labels = torch.randint(0, V, (N,), generator=g, dtype=torch.int64)
    n_ign = int(N * ignore_frac)
    if n_ign:
        labels[torch.randperm(N, generator=g)[:n_ign]] = IGNORE_INDEX
    mask = None
    n_off = int(N * mask_frac)
    if n_off:
        mask = torch.ones(N, dtype=torch.bool)
        mask[torch.randperm(N, generator=g)[:n_off]] = False
    return Workload(name=f"random_{N}x{D}x{V}", H=H, W=W, b=b, labels=labels, mask=mask)


def supervised_subset(w: Workload, keep: int, seed: int = 7) -> Workload:
    """Same tensors, but a mask that leaves only ``keep`` supervised rows.

    Used to check full-size shapes (N, D, V and the launch configuration) against
    the oracle at a cost the CPU can afford.
    """
    g = torch.Generator("cpu")
    g.manual_seed(seed)
    base = torch.ones(w.N, dtype=torch.bool) if w.mask is None else w.mask.clone()
    base &= w.labels != w.ignore_index
    cand = torch.nonzero(base).flatten()
    pick = cand[torch.randperm(cand.numel(), generator=g)[:keep]]
    m = torch.zeros(w.N, dtype=torch.bool)
    m[pick] = True
    return dataclasses.replace(w, name=w.name + f"_sub{keep}", mask=m)
