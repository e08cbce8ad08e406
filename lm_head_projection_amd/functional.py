"""PyTorch-facing API: linear_cross_entropy as a torch.autograd.Function.

PyTorch only provides device memory and the current stream; compaction,
projection, online log-sum-exp, replay and every gradient run in liblce.so.
"""

from __future__ import annotations

import math
from typing import Optional

import torch

from . import _lib

IGNORE_INDEX = -100
_FILTERS = {"dh": _lib.LCE_FILTER_DH, "both": _lib.LCE_FILTER_BOTH}


class Saved:
    """What one call keeps between its forward and backward passes: the
    supervised-row list, C and the two saved N-vectors m and log s (the
    statistics that section 02 of the glenzli.com page saves).  The
    workspaces are allocated per pass and released with it."""

    def __init__(self, N: int, dev):
        self.valid_idx = torch.empty(max(N, 1), dtype=torch.int32, device=dev)
        self.m = torch.empty(N, dtype=torch.float32, device=dev)
        self.logs = torch.empty(N, dtype=torch.float32, device=dev)
        self.C = 0


def _validate(H, W, b, labels, mask, reduction, loss_weights, num_label_tokens, filter_eps, filter_grads):
    """Every check that the C ABI cannot make on raw pointers, before any
    allocation or library call: shapes and element counts (a wrong one would
    make the kernels read past a buffer), dtypes, and one CUDA device for
    every tensor (a host pointer would reach the kernels otherwise)."""
    if reduction not in _lib.REDUCTIONS:
        raise ValueError(f"reduction must be one of {sorted(_lib.REDUCTIONS)}, not {reduction!r}")
    if filter_grads not in _FILTERS:
        raise ValueError(f"filter_grads must be one of {sorted(_FILTERS)}")
    if filter_eps is not None and not (math.isfinite(float(filter_eps)) and float(filter_eps) >= 0.0):
        raise ValueError("filter_eps must be finite and >= 0")
    if num_label_tokens is not None and not (math.isfinite(float(num_label_tokens))
                                             and float(num_label_tokens) >= 0.0):
        raise ValueError("num_label_tokens must be finite and >= 0")
    if H.dim() != 2 or W.dim() != 2:
        raise ValueError(f"hidden must be [N, D] and weight [V, D] (got {tuple(H.shape)}, {tuple(W.shape)})")
    N, D = H.shape
    V = W.shape[0]
    if W.shape[1] != D:
        raise ValueError(f"hidden has D = {D} but weight has {W.shape[1]} columns")
    if V == 0 or D == 0:
        raise ValueError("weight must have at least one row and one column")
    if H.dtype not in (torch.bfloat16, torch.float32):
        raise TypeError(f"unsupported dtype {H.dtype} (bf16 or fp32)")
    if W.dtype != H.dtype or (b is not None and b.dtype != H.dtype):
        raise TypeError("hidden, weight and bias must share one dtype")
    if b is not None and (b.dim() != 1 or b.shape[0] != V):
        raise ValueError(f"bias must be [V] = [{V}] (got {tuple(b.shape)})")
    if labels.numel() != N:
        raise ValueError(f"labels has {labels.numel()} elements for N = {N} positions")
    if labels.dtype.is_floating_point or labels.dtype == torch.bool or labels.is_complex():
        raise TypeError(f"labels must be an integer tensor (got {labels.dtype})")
    if mask is not None and mask.numel() != N:
        raise ValueError(f"mask has {mask.numel()} elements for N = {N} positions")
    if loss_weights is not None:
        if reduction != "sum":
            raise ValueError("loss_weights apply to reduction='sum' only")
        if loss_weights.numel() != N:
            raise ValueError(f"loss_weights has {loss_weights.numel()} elements for N = {N} positions")
    if filter_eps is not None and H.dtype != torch.bfloat16:
        raise TypeError("filter_eps needs bf16 inputs")
    tensors = [t for t in (H, W, b, labels, mask, loss_weights) if t is not None]
    if not all(t.is_cuda for t in tensors):
        raise ValueError("every tensor must be on a CUDA (HIP) device")
    if len({t.device for t in tensors}) != 1:
        raise ValueError("every tensor must be on the same device")


def _check(st: int, where: str, allow_empty: bool = True):
    if st == _lib.LCE_OK or (allow_empty and st == _lib.LCE_OK_EMPTY):
        return
    raise _lib.LCEError(st, where)


class LinearCrossEntropyFunction(torch.autograd.Function):
    @staticmethod
    def forward(ctx, H, W, b, labels, mask, ignore_index, reduction, loss_weights, num_label_tokens, filter_eps,
                filter_grads):
        _validate(H, W, b, labels, mask, reduction, loss_weights, num_label_tokens, filter_eps, filter_grads)
        H = H.contiguous()
        W = W.contiguous()
        b = None if b is None else b.contiguous()
        labels = labels.contiguous().to(torch.int64)
        mask_u8 = None if mask is None else mask.to(torch.uint8).contiguous()
        red = _lib.REDUCTIONS[reduction]
        w = None if loss_weights is None else loss_weights.to(torch.float32).contiguous()
        num = 0.0 if num_label_tokens is None else float(num_label_tokens)
        N, D = H.shape
        V = W.shape[0]
        s = Saved(N, H.device)
        # The compaction and forward need only the forward part of the workspace;
        # it is released when forward() returns.
        ws = torch.empty(_lib.lce_forward_workspace_size(N, D, V, H.dtype), dtype=torch.uint8, device=H.device)
        st, C = _lib.lce_compact_valid(labels, mask_u8, V, ignore_index, s.valid_idx, ws)
        _check(st, "lce_compact_valid")
        s.C = C
        out = torch.empty(N if red == _lib.LCE_REDUCTION_NONE else 1, dtype=torch.float32, device=H.device)
        st = _lib.lce_forward_ex(H, W, b, labels, s.valid_idx, C, red, w, num, out, s.m, s.logs, ws)
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
        N, D = H.shape
        V = W.shape[0]
        dH = torch.empty_like(H)
        dW = torch.empty_like(W)
        db = torch.empty_like(b) if ctx.has_bias else None
        g = grad.reshape(-1).to(torch.float32).contiguous()
        # Sized for the C supervised rows (the backward's arrays take C rows).
        ws = torch.empty(_lib.lce_backward_workspace_size(N, s.C, D, V, H.dtype), dtype=torch.uint8,
                         device=H.device)
        if ctx.filter_eps is None:
            st = _lib.lce_backward_ex(H, W, b, labels, s.valid_idx, s.C, ctx.red, ctx.w, ctx.num, s.m, s.logs,
                                      g, dH, dW, db, ws)
            _check(st, "lce_backward_ex")
        else:
            st = _lib.lce_backward_filtered(H, W, b, labels, s.valid_idx, s.C, ctx.red, ctx.w, ctx.num, s.m,
                                            s.logs, g, ctx.filter_eps, dH, dW, db, ws, which=ctx.filter_which)
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
    if reduction not in _lib.REDUCTIONS:
        raise ValueError(f"reduction must be one of {sorted(_lib.REDUCTIONS)}, not {reduction!r}")
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
