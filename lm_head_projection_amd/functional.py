"""PyTorch-facing API: linear_cross_entropy as a torch.autograd.Function.

PyTorch only provides device memory and the current stream; compaction,
projection, online log-sum-exp, replay and every gradient run in liblce.so.
"""

from __future__ import annotations

from typing import Optional

import torch

from . import _lib

IGNORE_INDEX = -100
_FILTERS = {"dh": _lib.LCE_FILTER_DH, "both": _lib.LCE_FILTER_BOTH}


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
    def forward(ctx, H, W, b, labels, mask, ignore_index, reduction, loss_weights, num_label_tokens, filter_eps,
                filter_grads):
        H = H.contiguous()
        W = W.contiguous()
        b = None if b is None else b.contiguous()
        labels = labels.contiguous().to(torch.int64)
        if W.dtype != H.dtype or (b is not None and b.dtype != H.dtype):
            raise TypeError("H, W and b must share one dtype")
        red = _lib.REDUCTIONS[reduction]
        w = None if loss_weights is None else loss_weights.to(torch.float32).contiguous()
        num = 0.0 if num_label_tokens is None else float(num_label_tokens)
        s = Saved(H, W, b, labels, mask, ignore_index)
        st, C = _lib.lce_compact_valid(labels, s.mask_u8, s.V, ignore_index, s.valid_idx, s.ws)
        _check(st, "lce_compact_valid")
        s.C = C
        out = torch.empty(s.N if red == _lib.LCE_REDUCTION_NONE else 1, dtype=torch.float32, device=H.device)
        st = _lib.lce_forward_ex(H, W, b, labels, s.valid_idx, C, red, w, num, out, s.m, s.logs, s.ws)
        _check(st, "lce_forward_ex")
        ctx.s = s
        ctx.red, ctx.w, ctx.num = red, w, num
        ctx.filter_eps = filter_eps
        ctx.filter_which = _FILTERS[filter_grads]
        ctx.save_for_backward(H, W, b, labels)
        ctx.has_bias = b is not None
        return out.clone() if red == _lib.LCE_REDUCTION_NONE else out[0].clone()

    @staticmethod
    def backward(ctx, grad):
        H, W, b, labels = ctx.saved_tensors
        s = ctx.s
        dH = torch.empty_like(H)
        dW = torch.empty_like(W)
        db = torch.empty_like(b) if ctx.has_bias else None
        g = grad.reshape(-1).to(torch.float32).contiguous()
        if ctx.filter_eps is None:
            st = _lib.lce_backward_ex(H, W, b, labels, s.valid_idx, s.C, ctx.red, ctx.w, ctx.num, s.m, s.logs,
                                      g, dH, dW, db, s.ws)
            _check(st, "lce_backward_ex")
        else:
            st = _lib.lce_backward_filtered(H, W, b, labels, s.valid_idx, s.C, ctx.red, ctx.w, ctx.num, s.m,
                                            s.logs, g, ctx.filter_eps, dH, dW, db, s.ws, which=ctx.filter_which)
            _check(st, "lce_backward_filtered")
        return dH, dW, db, None, None, None, None, None, None, None, None


def linear_cross_entropy(hidden: torch.Tensor, weight: torch.Tensor, labels: torch.Tensor,
                         bias: Optional[torch.Tensor] = None, mask: Optional[torch.Tensor] = None,
                         ignore_index: int = IGNORE_INDEX, reduction: str = "mean",
                         loss_weights: Optional[torch.Tensor] = None,
                         num_label_tokens: Optional[float] = None,
                         filter_eps: Optional[float] = None, filter_grads: str = "both") -> torch.Tensor:
    """CE of (hidden @ weight.T + bias) over supervised rows without forming the logits.

    hidden [N, D], weight [V, D], bias [V] (optional), labels [N] (int),
    mask [N] (optional bool; False = unsupervised).
    reduction "mean" (over the supervised rows), "sum" (optionally weighted by
    loss_weights [N] and divided by num_label_tokens) or "none" (per-position
    losses [N], 0 on unsupervised positions).  With no supervised rows the
    loss is 0 and every gradient is exactly 0.
    filter_eps (bf16 only): the backward drops the dH/dW contribution of every
    block of 256 supervised rows x 32 vocabulary entries that holds no target
    and whose probabilities are all below filter_eps (an approximation of the
    gradient; db stays exact).  None or 0 gives the exact gradient.
    filter_grads: "both", or "dh" (the embedding gradient only; dW exact).
    """
    if filter_grads not in _FILTERS:
        raise ValueError(f"filter_grads must be one of {sorted(_FILTERS)}")
    if hidden.dim() != 2:
        lead = labels.shape
        hidden = hidden.reshape(-1, hidden.shape[-1])
        labels = labels.reshape(-1)
        if mask is not None:
            mask = mask.reshape(-1)
        if loss_weights is not None:
            loss_weights = loss_weights.reshape(-1)
        out = LinearCrossEntropyFunction.apply(hidden, weight, bias, labels, mask, ignore_index, reduction,
                                               loss_weights, num_label_tokens, filter_eps, filter_grads)
        return out.reshape(lead) if reduction == "none" else out
    return LinearCrossEntropyFunction.apply(hidden, weight, bias, labels, mask, ignore_index, reduction,
                                           loss_weights, num_label_tokens, filter_eps, filter_grads)
