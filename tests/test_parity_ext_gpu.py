"""GPU parity of the extended entry points (flce_forward_ex / flce_backward_ex)
against the float64 oracle on the same seeded bf16 inputs: the uniform
cross-entropy and z-loss outputs, the "sum" reduction, gradients of all four
per-token outputs, and fp32 gradient outputs.

Tolerances as for the plain entry points: per-token and reduced outputs
within 2e-3 absolute or 1e-3 relative, gradients within 1e-2 relative L2.
Two exact checks: bf16 gradients equal the fp32 ones rounded to nearest even
(both come from the same fp32 arithmetic), and "sum" with scalar upstream
gradients equals "none" with those values on every token, bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import gpu_helpers as G
from linear_cross_entropy_tile_amd import flce, workloads as W

pytestmark = pytest.mark.gpu

# (workload, reduction, z-loss scale)
CASES = [("tiny", "none", 0.0), ("odd_tails", "sum", 0.05), ("mean_ignore", "mean", 0.02),
         ("dw_split", "sum", 0.1), ("softcap_saturation", "none", 0.01)]
OUTS = ("logprob", "entropy", "uniform_ce", "z_loss")


def _grads(N, reduction, seed):
    rng = np.random.default_rng(seed)
    if reduction == "none":
        return [rng.standard_normal(N).astype(np.float32) for _ in OUTS]
    return [np.array([v], dtype=np.float32) for v in rng.standard_normal(4)]


def _gpu(t, wl, reduction, lam, grads, grad_dtype):
    out = flce.forward(t["hidden"], t["weight"], t["labels"], ignore_index=wl.ignore_index,
                       softcap=wl.softcap, reduction=reduction, z_loss_scale=lam, aux=True)
    g = [torch.from_numpy(a).to(G.dev()) for a in grads]
    gh, gw = flce.backward(t["hidden"], t["weight"], t["labels"], out["lse"], out["entropy"],
                           g[0], g[1], ignore_index=wl.ignore_index, softcap=wl.softcap,
                           reduction=reduction, grad_uniform_ce=g[2], grad_z_loss=g[3],
                           z_loss_scale=lam, grad_dtype=grad_dtype)
    torch.cuda.synchronize()
    return out, gh, gw


@pytest.mark.parametrize("name,reduction,lam", CASES, ids=[f"{c[0]}-{c[1]}" for c in CASES])
def test_extended_parity(name, reduction, lam):
    wl = W.WORKLOADS[name]
    x = W.make_inputs(wl)
    print(f"[ext] {name} N={wl.N} H={wl.H} V={wl.V} {reduction} lam={lam}", flush=True)
    t = G.upload(x)
    grads = _grads(wl.N, reduction, wl.seed + 77)
    out, gh32, gw32 = _gpu(t, wl, reduction, lam, grads, "f32")
    _, gh16, gw16 = _gpu(t, wl, reduction, lam, grads, "bf16")
    assert gh32.dtype == torch.float32 and gh16.dtype == torch.bfloat16

    hf = W.bf16_bits_to_f32(x["hidden"])
    wf = W.bf16_bits_to_f32(x["weight"])
    fw = oracle.forward(hf, wf, x["labels"], ignore_index=wl.ignore_index, softcap_c=wl.softcap,
                        reduction=reduction, z_loss_scale=lam)
    dh, dw = oracle.backward(hf, wf, x["labels"], ignore_index=wl.ignore_index,
                             softcap_c=wl.softcap, reduction=reduction, grad_logprob=grads[0],
                             grad_entropy=grads[1], grad_uniform_ce=grads[2],
                             grad_z_loss=grads[3], z_loss_scale=lam)
    for k in ("lse",) + OUTS:
        e = G.stat_err(out[k].cpu().numpy(), fw[k])
        assert e <= 1.0, f"{name} {k}: error {e:.3f} x tolerance"
    if reduction != "none":
        for k in OUTS:
            key = f"{k}_{reduction}"
            e = G.stat_err(out[key].cpu().numpy(), [fw[key]])
            assert e <= 1.0, f"{name} {key}: error {e:.3f} x tolerance"
    for got, ref, what in ((gh32, dh, "grad_hidden f32"), (gw32, dw, "grad_weight f32"),
                           (gh16, dh, "grad_hidden bf16"), (gw16, dw, "grad_weight bf16")):
        e = G.rel_l2(got.float().cpu().numpy(), ref)
        assert e <= G.GRAD_REL_L2, f"{name} {what} rel L2 {e:.2e}"
    # Same fp32 arithmetic, rounded to bf16 or not.
    assert torch.equal(gh32.to(torch.bfloat16), gh16), f"{name}: bf16 dH != round(fp32 dH)"
    assert torch.equal(gw32.to(torch.bfloat16), gw16), f"{name}: bf16 dW != round(fp32 dW)"
    ign = torch.from_numpy(x["labels"] == wl.ignore_index).to(G.dev())
    if bool(ign.any()):
        for k in OUTS:
            assert torch.count_nonzero(out[k][ign]).item() == 0
        assert torch.count_nonzero(gh32[ign]).item() == 0


def test_sum_equals_none_with_constant_grads():
    wl = W.WORKLOADS["odd_tails"]
    x = W.make_inputs(wl)
    t = G.upload(x)
    scal = [0.7, -0.3, 0.25, 1.5]
    lam = 0.05
    s_grads = [np.array([v], dtype=np.float32) for v in scal]
    n_grads = [np.full(wl.N, v, dtype=np.float32) for v in scal]
    out_s, gh_s, gw_s = _gpu(t, wl, "sum", lam, s_grads, "f32")
    out_n, gh_n, gw_n = _gpu(t, wl, "none", lam, n_grads, "f32")
    assert torch.equal(gh_s, gh_n) and torch.equal(gw_s, gw_n)
    for k in ("lse",) + OUTS:
        assert torch.equal(out_s[k], out_n[k])
    valid = torch.from_numpy(x["labels"] != wl.ignore_index).to(G.dev())
    for k in OUTS:
        ref = out_n[k][valid].double().sum().item()
        assert abs(out_s[f"{k}_sum"].item() - ref) <= 1e-5 * max(1.0, abs(ref))


def test_z_loss_off_matches_plain_entry_points():
    """lam = 0 and zero auxiliary gradients: the extended path reproduces the
    plain flce_forward / flce_backward results bit for bit."""
    wl = W.WORKLOADS["tiny"]
    x = W.make_inputs(wl)
    t = G.upload(x)
    a = flce.forward(t["hidden"], t["weight"], t["labels"])
    b = flce.forward(t["hidden"], t["weight"], t["labels"], aux=True)
    for k in ("lse", "logprob", "entropy"):
        assert torch.equal(a[k], b[k])
    g = t["grad_logprob"], t["grad_entropy"]
    gh_a, gw_a = flce.backward(t["hidden"], t["weight"], t["labels"], a["lse"], a["entropy"], *g)
    gh_b, gw_b = flce.backward(t["hidden"], t["weight"], t["labels"], a["lse"], a["entropy"], *g,
                               grad_dtype="f32")
    assert torch.equal(gh_b.to(torch.bfloat16), gh_a) and torch.equal(gw_b.to(torch.bfloat16), gw_a)
