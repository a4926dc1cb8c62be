"""The autograd wrapper linear_cross_entropy against the float64 oracle: the
two outputs under each reduction, and the gradients that torch's backward
produces for a loss built from both outputs (tolerances as in the other
parity tests)."""
import numpy as np
import pytest
import torch

import oracle
import gpu_helpers as G
from linear_cross_entropy_tile_amd import workloads as W
from linear_cross_entropy_tile_amd.function import linear_cross_entropy

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,reduction", [("odd_tails", "mean"), ("mean_ignore", "mean"),
                                            ("tiny", "none"), ("dw_split", "sum")])
def test_autograd_matches_oracle(name, reduction):
    wl = W.WORKLOADS[name]
    x = W.make_inputs(wl)
    t = G.upload(x)
    h = t["hidden"].clone().requires_grad_(True)
    w = t["weight"].clone().requires_grad_(True)
    lp, ent = linear_cross_entropy(h, w, t["labels"], reduction=reduction,
                                   ignore_index=wl.ignore_index, softcap=wl.softcap)
    rng = np.random.default_rng(wl.seed + 3)
    if reduction == "none":
        a = rng.standard_normal(wl.N).astype(np.float32)
        b = rng.standard_normal(wl.N).astype(np.float32)
        loss = (lp * torch.from_numpy(a).to(G.dev())).sum() + (ent * torch.from_numpy(b).to(G.dev())).sum()
        ga, gb = a, b
    else:
        a, b = -1.0, 0.01  # a loss -logprob + 0.01 entropy
        loss = a * lp + b * ent
        ga, gb = np.array([a], np.float32), np.array([b], np.float32)
    loss.backward()
    torch.cuda.synchronize()
    hf = W.bf16_bits_to_f32(x["hidden"])
    wf = W.bf16_bits_to_f32(x["weight"])
    fw = oracle.forward(hf, wf, x["labels"], ignore_index=wl.ignore_index, softcap_c=wl.softcap,
                        reduction=reduction)
    dh, dw = oracle.backward(hf, wf, x["labels"], ignore_index=wl.ignore_index,
                             softcap_c=wl.softcap, reduction=reduction, grad_logprob=ga,
                             grad_entropy=gb)
    if reduction == "none":
        assert G.stat_err(lp.detach().cpu().numpy(), fw["logprob"]) <= 1.0
        assert G.stat_err(ent.detach().cpu().numpy(), fw["entropy"]) <= 1.0
    else:
        assert lp.dim() == 0 and ent.dim() == 0
        assert G.stat_err([lp.item()], [fw[f"logprob_{reduction}"]]) <= 1.0
        assert G.stat_err([ent.item()], [fw[f"entropy_{reduction}"]]) <= 1.0
    assert h.grad.dtype == torch.bfloat16 and w.grad.dtype == torch.bfloat16
    e = G.rel_l2(h.grad.float().cpu().numpy(), dh)
    assert e <= G.GRAD_REL_L2, f"{name} grad_hidden rel L2 {e:.2e}"
    e = G.rel_l2(w.grad.float().cpu().numpy(), dw)
    assert e <= G.GRAD_REL_L2, f"{name} grad_weight rel L2 {e:.2e}"


def test_autograd_one_output_used():
    """Only the entropy enters the loss: the logprob gradient is None."""
    wl = W.WORKLOADS["odd_tails"]
    x = W.make_inputs(wl)
    t = G.upload(x)
    h = t["hidden"].clone().requires_grad_(True)
    w = t["weight"].clone().requires_grad_(True)
    _, ent = linear_cross_entropy(h, w, t["labels"], reduction="mean", ignore_index=wl.ignore_index)
    ent.backward()
    torch.cuda.synchronize()
    hf = W.bf16_bits_to_f32(x["hidden"])
    wf = W.bf16_bits_to_f32(x["weight"])
    dh, dw = oracle.backward(hf, wf, x["labels"], ignore_index=wl.ignore_index, reduction="mean",
                             grad_logprob=np.array([0.0], np.float32),
                             grad_entropy=np.array([1.0], np.float32))
    assert G.rel_l2(h.grad.float().cpu().numpy(), dh) <= G.GRAD_REL_L2
    assert G.rel_l2(w.grad.float().cpu().numpy(), dw) <= G.GRAD_REL_L2


def test_autograd_class_weights():
    """Class weights through the autograd wrapper: the weighted means and the
    gradients of -logprob + 0.01 entropy against the oracle."""
    wl = W.WORKLOADS["odd_tails"]
    x = W.make_inputs(wl)
    t = G.upload(x)
    cw = W.make_class_weights(wl.V, wl.seed + 9, 0.1)
    h = t["hidden"].clone().requires_grad_(True)
    w = t["weight"].clone().requires_grad_(True)
    lp, ent = linear_cross_entropy(h, w, t["labels"], reduction="mean",
                                   ignore_index=wl.ignore_index,
                                   class_weight=torch.from_numpy(cw).to(G.dev()))
    (-lp + 0.01 * ent).backward()
    torch.cuda.synchronize()
    hf = W.bf16_bits_to_f32(x["hidden"])
    wf = W.bf16_bits_to_f32(x["weight"])
    fw = oracle.forward(hf, wf, x["labels"], ignore_index=wl.ignore_index, reduction="mean",
                        class_weight=cw)
    dh, dw = oracle.backward(hf, wf, x["labels"], ignore_index=wl.ignore_index, reduction="mean",
                             grad_logprob=np.array([-1.0], np.float32),
                             grad_entropy=np.array([0.01], np.float32), class_weight=cw)
    assert G.stat_err([lp.item()], [fw["logprob_mean"]]) <= 1.0
    assert G.stat_err([ent.item()], [fw["entropy_mean"]]) <= 1.0
    assert G.rel_l2(h.grad.float().cpu().numpy(), dh) <= G.GRAD_REL_L2
    assert G.rel_l2(w.grad.float().cpu().numpy(), dw) <= G.GRAD_REL_L2


@pytest.mark.parametrize("reduction,fused", [("mean", False), ("sum", False), ("mean", True)])
def test_entropy_per_token_beside_reduced_logprob(reduction, fused):
    """entropy_reduction="none": a reduced logprob beside the per-token
    entropy (the output shapes of the verl pull request #462 "Equivalent
    compute logic"). The oracle's gradient for a scalar logprob gradient a and
    per-token entropy gradients b is the sum of its "mean"/"sum" gradient
    for (a, 0) and its "none" gradient for (0, b): the gradient is linear in
    the upstream gradients."""
    wl = W.WORKLOADS["mean_ignore"].with_(N=600, H=256, V=3000)
    x = W.make_inputs(wl)
    t = G.upload(x)
    rng = np.random.default_rng(wl.seed + 17)
    a = np.array([-1.25], np.float32)
    b = rng.standard_normal(wl.N).astype(np.float32)
    hf = W.bf16_bits_to_f32(x["hidden"])
    wf = W.bf16_bits_to_f32(x["weight"])
    fw = oracle.forward(hf, wf, x["labels"], ignore_index=wl.ignore_index, reduction=reduction)
    dh1, dw1 = oracle.backward(hf, wf, x["labels"], ignore_index=wl.ignore_index,
                               reduction=reduction, grad_logprob=a,
                               grad_entropy=np.array([0.0], np.float32))
    dh2, dw2 = oracle.backward(hf, wf, x["labels"], ignore_index=wl.ignore_index,
                               reduction="none", grad_logprob=np.zeros(wl.N, np.float32),
                               grad_entropy=b)
    dh, dw = dh1 + dh2, dw1 + dw2
    if fused:
        from linear_cross_entropy_tile_amd import flce
        res = flce.forward_backward(t["hidden"], t["weight"], t["labels"],
                                    torch.from_numpy(a).to(G.dev()),
                                    torch.from_numpy(b).to(G.dev()),
                                    ignore_index=wl.ignore_index, reduction=reduction,
                                    entropy_reduction="none")
        torch.cuda.synchronize()
        lp, ent = res[f"logprob_{reduction}"], res["entropy"]
        gh, gw = res["grad_hidden"], res["grad_weight"]
    else:
        h = t["hidden"].clone().requires_grad_(True)
        w = t["weight"].clone().requires_grad_(True)
        lp, ent = linear_cross_entropy(h, w, t["labels"], reduction=reduction,
                                       ignore_index=wl.ignore_index, entropy_reduction="none")
        assert lp.dim() == 0 and ent.shape == (wl.N,)
        loss = float(a[0]) * lp + (ent * torch.from_numpy(b).to(G.dev())).sum()
        loss.backward()
        torch.cuda.synchronize()
        gh, gw = h.grad, w.grad
    assert G.stat_err([lp.reshape(()).item()], [fw[f"logprob_{reduction}"]]) <= 1.0
    assert G.stat_err(ent.detach().cpu().numpy(), fw["entropy"]) <= 1.0
    e = G.rel_l2(gh.float().cpu().numpy(), dh)
    assert e <= G.GRAD_REL_L2, f"grad_hidden rel L2 {e:.2e}"
    e = G.rel_l2(gw.float().cpu().numpy(), dw)
    assert e <= G.GRAD_REL_L2, f"grad_weight rel L2 {e:.2e}"
