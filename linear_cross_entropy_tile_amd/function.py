"""``linear_cross_entropy``: the head as a torch autograd function, in the
call shape of the API example of verl pull request #462 (section "API"):
``linear_cross_entropy(hidden, weight, labels, reduction="mean")`` returns two
outputs, the label log-probability and the entropy. Following that page's
"Equivalent compute logic", the first output is the log-probability of the
label (minus the cross-entropy), not the cross-entropy itself.

Marshalling only: the forward calls flce_forward through ``flce.forward``
and keeps the per-token lse and entropy; the backward hands the upstream
gradients of the two outputs to flce_backward through ``flce.backward``.
"""
from __future__ import annotations

import torch

from . import flce

__all__ = ["LinearCrossEntropy", "linear_cross_entropy"]


class LinearCrossEntropy(torch.autograd.Function):
    """(logprob, entropy) of the fused head; see ``linear_cross_entropy``."""

    @staticmethod
    def forward(ctx, hidden, weight, labels, reduction="mean", ignore_index=-100, softcap=0.0,
                class_weight=None):
        out = flce.forward(hidden, weight, labels, ignore_index=ignore_index, softcap=softcap,
                           reduction=reduction, class_weight=class_weight)
        ctx.save_for_backward(hidden, weight, labels, out["lse"], out["entropy"])
        ctx.class_weight = class_weight
        ctx.reduction = reduction
        ctx.ignore_index = ignore_index
        ctx.softcap = softcap
        if reduction == "none":
            return out["logprob"], out["entropy"]
        return (out[f"logprob_{reduction}"].reshape(()), out[f"entropy_{reduction}"].reshape(()))

    @staticmethod
    def backward(ctx, grad_logprob, grad_entropy):
        hidden, weight, labels, lse, entropy = ctx.saved_tensors
        n = hidden.shape[0] if ctx.reduction == "none" else 1

        def prep(g):
            return None if g is None else g.float().reshape(n).contiguous()

        gh, gw = flce.backward(hidden, weight, labels, lse, entropy, prep(grad_logprob),
                               prep(grad_entropy), ignore_index=ctx.ignore_index,
                               softcap=ctx.softcap, reduction=ctx.reduction,
                               class_weight=ctx.class_weight)
        return gh, gw, None, None, None, None, None


def linear_cross_entropy(hidden, weight, labels, reduction="mean", ignore_index=-100,
                         softcap=0.0, class_weight=None):
    """(logprob, entropy) for hidden bf16 [N,H], weight bf16 [H,V], labels
    int64 [N]: per token ([N] fp32) under reduction "none", else the mean over
    the non-ignored tokens ("mean") or their sum ("sum"), 0-d fp32 tensors.
    class_weight (fp32 [V], "mean" / "sum" only) weights token t by
    class_weight[labels[t]] in both reductions; the mean then divides by the
    weight sum of the non-ignored tokens. Differentiable with respect to
    hidden and weight (gradients in bf16)."""
    return LinearCrossEntropy.apply(hidden, weight, labels, reduction, ignore_index, softcap,
                                    class_weight)
