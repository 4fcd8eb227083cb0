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
    def forward(ctx, X, W, labels, ignore_index=-100, softcap=0.0, logit_scale=1.0,
                label_smoothing=0.0, z_loss=0.0, reduction="mean", filter_eps=0.0, precise=False):
        opts = dict(ignore_index=int(ignore_index), softcap=float(softcap),
                    logit_scale=float(logit_scale), label_smoothing=float(label_smoothing),
                    z_loss=float(z_loss), reduction=reduction)
        out = _lib.lce_forward_ex(X, W, labels, **opts)
        ctx.save_for_backward(X, W, labels, out["lse"])
        ctx.opts = dict(opts, filter_eps=float(filter_eps), precise=bool(precise))
        return out["loss"] if reduction == "none" else out["reduced"]

    @staticmethod
    def backward(ctx, grad):
        X, W, labels, lse = ctx.saved_tensors
        dX, dW = _lib.lce_backward_ex(X, W, labels, lse, grad.float(), dX_dtype=X.dtype,
                                      dW_dtype=W.dtype, **ctx.opts)
        return dX, dW, None, None, None, None, None, None, None, None, None


def linear_cross_entropy(X, W, labels, ignore_index: int = -100, softcap: float = 0.0,
                         logit_scale: float = 1.0, label_smoothing: float = 0.0,
                         z_loss: float = 0.0, reduction: str = "mean",
                         filter_eps: float = 0.0, precise: bool = False):
    """Cross-entropy of X·Wᵀ over pre-shifted labels without the logits: the
    mean over valid targets (or the sum, or the per-row losses for
    reduction="none") of LSE − (1 − e)·z_y − (e/V)·Σ z + l·LSE².  filter_eps > 0
    turns on the non-exact gradient filter of the backward; precise=True its
    two-part gradient chunk."""
    return LinearCrossEntropy.apply(X, W, labels, ignore_index, softcap, logit_scale,
                                    label_smoothing, z_loss, reduction, filter_eps, precise)
