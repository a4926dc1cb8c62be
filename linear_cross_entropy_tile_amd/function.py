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
                class_weight=None, entropy_reduction=None):
        out = flce.forward(hidden, weight, labels, ignore_index=ignore_index, softcap=softcap,
                           reduction=reduction, class_weight=class_weight)
        ctx.save_for_backward(hidden, weight, labels, out["lse"], out["entropy"])
        ctx.class_weight = class_weight
        ctx.reduction = reduction
        ctx.ignore_index = ignore_index
        ctx.softcap = softcap
        ctx.entropy_tokens = reduction == "none" or entropy_reduction == "none"
        ctx.entropy_reduction = entropy_reduction
        lp = out["logprob"] if reduction == "none" else out[f"logprob_{reduction}"].reshape(())
        ent = out["entropy"] if ctx.entropy_tokens else out[f"entropy_{reduction}"].reshape(())
        return lp, ent

    @staticmethod
    def backward(ctx, grad_logprob, grad_entropy):
        hidden, weight, labels, lse, entropy = ctx.saved_tensors
        n = hidden.shape[0]

        def prep(g, size):
            return None if g is None else g.float().reshape(size).contiguous()

        gh, gw = flce.backward(hidden, weight, labels, lse, entropy,
                               prep(grad_logprob, n if ctx.reduction == "none" else 1),
                               prep(grad_entropy, n if ctx.entropy_tokens else 1),
                               ignore_index=ctx.ignore_index, softcap=ctx.softcap,
                               reduction=ctx.reduction, class_weight=ctx.class_weight,
                               entropy_reduction=ctx.entropy_reduction)
        return gh, gw, None, None, None, None, None, None


def linear_cross_entropy(hidden, weight, labels, reduction="mean", ignore_index=-100,
                         softcap=0.0, class_weight=None, entropy_reduction=None):
    """(logprob, entropy) for hidden bf16 [N,H], weight bf16 [H,V], labels
    int64 [N]: per token ([N] fp32) under reduction "none", else the mean over
    the non-ignored tokens ("mean") or their sum ("sum"), 0-d fp32 tensors.
    ``entropy_reduction="none"`` returns the entropy per token ([N], 0 at
    ignored tokens) beside the reduced logprob, the output shapes of the verl
    pull request #462 "Equivalent compute logic"; None reduces both alike.
    class_weight (fp32 [V], "mean" / "sum" only) weights token t by
    class_weight[labels[t]] in the reductions; the mean then divides by the
    weight sum of the non-ignored tokens. Differentiable with respect to
    hidden and weight (gradients in bf16)."""
    return LinearCrossEntropy.apply(hidden, weight, labels, reduction, ignore_index, softcap,
                                    class_weight, entropy_reduction)
