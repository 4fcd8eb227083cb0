"""torch.autograd wrapper: mean cross-entropy of X·Wᵀ without the logits.

Only the per-row LSE is saved for the backward, besides the inputs; the
backward recomputes the logit tiles inside the kernels (blog "最贵的一层：深入浅出
Liger Kernel 与 Cut Cross-Entropy", §三; Unsloth fused cross-entropy chapter, §7:
the LSE is the one activation kept for the backward).
"""
from __future__ import annotations

import torch

from . import _lib


class LinearCrossEntropy(torch.autograd.Function):
    @staticmethod
    def forward(ctx, X, W, labels, ignore_index=-100, softcap=0.0):
        out = _lib.lce_forward(X, W, labels, ignore_index, softcap)
        ctx.save_for_backward(X, W, labels, out["lse"])
        ctx.ignore_index = int(ignore_index)
        ctx.softcap = float(softcap)
        return out["mean"]

    @staticmethod
    def backward(ctx, grad_mean):
        X, W, labels, lse = ctx.saved_tensors
        dX, dW = _lib.lce_backward(X, W, labels, lse, grad_mean.float(), ctx.ignore_index,
                                   ctx.softcap, dX_dtype=X.dtype, dW_dtype=W.dtype)
        return dX, dW, None, None, None


def linear_cross_entropy(X, W, labels, ignore_index: int = -100, softcap: float = 0.0):
    """Mean over valid targets of LSE(x_i·Wᵀ) − x_i·w_{y_i}; labels pre-shifted."""
    return LinearCrossEntropy.apply(X, W, labels, ignore_index, softcap)
