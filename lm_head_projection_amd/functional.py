"""PyTorch-facing API: linear_cross_entropy as a torch.autograd.Function.

PyTorch only provides device memory and the current stream; compaction,
projection, online log-sum-exp, replay and every gradient run in liblce.so.
"""

from __future__ import annotations

from typing import Optional

import torch

from . import _lib

IGNORE_INDEX = -100


class Saved:
    """Device buffers of one call (caller-owned memory for the C ABI)."""

    def __init__(self, H, W, b, labels, mask, ignore_index):
        dev = H.device
        N, D = H.shape
        V = W.shape[0]
        self.N, self.D, self.V = N, D, V
        self.ws = torch.empty(_lib.lce_workspace_size(N, D, V, H.dtype), dtype=torch.uint8, device=dev)
        self.valid_idx = torch.empty(max(N, 1), dtype=torch.int32, device=dev)
        self.m = torch.empty(N, dtype=torch.float32, device=dev)
        self.logs = torch.empty(N, dtype=torch.float32, device=dev)
        self.loss = torch.empty(1, dtype=torch.float32, device=dev)
        self.ignore_index = ignore_index
        self.mask_u8 = None if mask is None else mask.to(torch.uint8).contiguous()
        self.C = 0


def _check(st: int, where: str, allow_empty: bool = True):
    if st == _lib.LCE_OK or (allow_empty and st == _lib.LCE_OK_EMPTY):
        return
    raise _lib.LCEError(st, where)


class LinearCrossEntropyFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, H, W, b, labels, mask, ignore_index):
        H = H.contiguous()
        W = W.contiguous()
        b = None if b is None else b.contiguous()
        labels = labels.contiguous().to(torch.int64)
        if W.dtype != H.dtype or (b is not None and b.dtype != H.dtype):
            raise TypeError("H, W and b must share one dtype")
        s = Saved(H, W, b, labels, mask, ignore_index)
        st, C = _lib.lce_compact_valid(labels, s.mask_u8, s.V, ignore_index, s.valid_idx, s.ws)
        _check(st, "lce_compact_valid")
        s.C = C
        st = _lib.lce_forward(H, W, b, labels, s.valid_idx, C, s.loss, s.m, s.logs, None, s.ws)
        _check(st, "lce_forward")
        ctx.s = s
        ctx.save_for_backward(H, W, b, labels)
        ctx.has_bias = b is not None
        return s.loss[0].clone()

    @staticmethod
    def backward(ctx, grad):
        H, W, b, labels = ctx.saved_tensors
        s = ctx.s
        dH = torch.empty_like(H)
        dW = torch.empty_like(W)
        db = torch.empty_like(b) if ctx.has_bias else None
        g = grad.reshape(1).to(torch.float32).contiguous()
        st = _lib.lce_backward(H, W, b, labels, s.valid_idx, s.C, s.m, s.logs, g, dH, dW, db, s.ws)
        _check(st, "lce_backward")
        return dH, dW, db, None, None, None


def linear_cross_entropy(hidden: torch.Tensor, weight: torch.Tensor, labels: torch.Tensor,
                         bias: Optional[torch.Tensor] = None, mask: Optional[torch.Tensor] = None,
                         ignore_index: int = IGNORE_INDEX) -> torch.Tensor:
    """Mean CE over supervised rows of (hidden @ weight.T + bias) without forming the logits.

    hidden [N, D], weight [V, D], bias [V] (optional), labels [N] (int),
    mask [N] (optional bool; False = unsupervised).  Returns an fp32 scalar;
    with no supervised rows it returns 0 and every gradient is exactly 0.
    """
    if hidden.dim() != 2:
        hidden = hidden.reshape(-1, hidden.shape[-1])
        labels = labels.reshape(-1)
        if mask is not None:
            mask = mask.reshape(-1)
    return LinearCrossEntropyFunction.apply(hidden, weight, bias, labels, mask, ignore_index)
