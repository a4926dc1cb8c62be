"""GPU parity for vocabularies that are not a multiple of 8 (the weight is
read from a padded copy with 16-byte aligned rows and dW is formed in a
padded buffer, both in the workspace) against the float64 oracle on the same
seeded bf16 inputs: forward statistics and reductions, both gradients in bf16
and fp32, the cap, several vocabulary chunks with an odd last one, the
token-split dW, class weights, odd vocabulary slices and the fused call
(one chunk and several, bf16 and fp32).

Tolerances as everywhere: statistics within 2e-3 absolute or 1e-3
relative, gradients within 1e-2 relative L2.
"""
import numpy as np
import pytest
import torch

import oracle
import gpu_helpers as G
from linear_cross_entropy_tile_amd import flce, workloads as W

pytestmark = pytest.mark.gpu

OUTS = ("logprob", "entropy", "uniform_ce", "z_loss")

# (workload, reduction, softcap, z-loss scale, FLCE_D_BUDGET columns or 0, grad dtype)
CASES = [("odd_vocab", "none", 0.0, 0.0, 0, "bf16"),
         ("odd_vocab", "mean", 5.0, 0.02, 0, "f32"),
         ("odd_vocab", "sum", 0.0, 0.05, 256, "bf16"),      # four chunks, the last 233 wide
         ("odd_vocab_dw_split", "none", 3.0, 0.0, 0, "bf16")]  # dW split over tokens


def _grads(wl, reduction, seed):
    rng = np.random.default_rng(seed)
    if reduction == "none":
        return [rng.standard_normal(wl.N).astype(np.float32) for _ in OUTS]
    return [np.array([v], dtype=np.float32) for v in rng.standard_normal(4)]


@pytest.mark.parametrize("name,reduction,cap,lam,cols,gdt", CASES,
                         ids=[f"{c[0]}-{c[1]}-cap{c[2]:g}-cols{c[4]}-{c[5]}" for c in CASES])
def test_odd_vocab_parity(name, reduction, cap, lam, cols, gdt, monkeypatch):
    wl = W.WORKLOADS[name]
    assert wl.V % 8 != 0
    x = W.make_inputs(wl)
    print(f"[odd V] {name} N={wl.N} H={wl.H} V={wl.V} {reduction} cap={cap} cols={cols}",
          flush=True)
    t = G.upload(x)
    if cols:
        monkeypatch.setenv("FLCE_D_BUDGET", str(2 * wl.N * cols))
    grads = _grads(wl, reduction, wl.seed + 5)
    g = [torch.from_numpy(a).to(G.dev()) for a in grads]
    out = flce.forward(t["hidden"], t["weight"], t["labels"], ignore_index=wl.ignore_index,
                       softcap=cap, reduction=reduction, z_loss_scale=lam, aux=True)
    gh, gw = flce.backward(t["hidden"], t["weight"], t["labels"], out["lse"], out["entropy"],
                           g[0], g[1], ignore_index=wl.ignore_index, softcap=cap,
                           reduction=reduction, grad_uniform_ce=g[2], grad_z_loss=g[3],
                           z_loss_scale=lam, grad_dtype=gdt)
    torch.cuda.synchronize()
    assert gw.shape == (wl.H, wl.V)
    hf = W.bf16_bits_to_f32(x["hidden"])
    wf = W.bf16_bits_to_f32(x["weight"])
    fw = oracle.forward(hf, wf, x["labels"], ignore_index=wl.ignore_index, softcap_c=cap,
                        reduction=reduction, z_loss_scale=lam)
    dh, dw = oracle.backward(hf, wf, x["labels"], ignore_index=wl.ignore_index, softcap_c=cap,
                             reduction=reduction, grad_logprob=grads[0], grad_entropy=grads[1],
                             grad_uniform_ce=grads[2], grad_z_loss=grads[3], z_loss_scale=lam)
    for k in ("lse",) + OUTS:
        e = G.stat_err(out[k].cpu().numpy(), fw[k])
        assert e <= 1.0, f"{name} {k}: error {e:.3f} x tolerance"
    if reduction != "none":
        for k in OUTS:
            e = G.stat_err(out[f"{k}_{reduction}"].cpu().numpy(), [fw[f"{k}_{reduction}"]])
            assert e <= 1.0, f"{name} {k}_{reduction}: error {e:.3f} x tolerance"
    assert G.rel_l2(gh.float().cpu().numpy(), dh) <= G.GRAD_REL_L2
    assert G.rel_l2(gw.float().cpu().numpy(), dw) <= G.GRAD_REL_L2


def test_odd_vocab_class_weights():
    wl = W.WORKLOADS["odd_vocab"]
    x = W.make_inputs(wl)
    t = G.upload(x)
    cw = W.make_class_weights(wl.V, wl.seed + 6, 0.1)
    cwt = torch.from_numpy(cw).to(G.dev())
    grads = _grads(wl, "mean", wl.seed + 7)
    g = [torch.from_numpy(a).to(G.dev()) for a in grads]
    out = flce.forward(t["hidden"], t["weight"], t["labels"], reduction="mean", class_weight=cwt)
    gh, gw = flce.backward(t["hidden"], t["weight"], t["labels"], out["lse"], out["entropy"],
                           g[0], g[1], reduction="mean", class_weight=cwt)
    torch.cuda.synchronize()
    hf = W.bf16_bits_to_f32(x["hidden"])
    wf = W.bf16_bits_to_f32(x["weight"])
    fw = oracle.forward(hf, wf, x["labels"], reduction="mean", class_weight=cw)
    dh, dw = oracle.backward(hf, wf, x["labels"], reduction="mean", grad_logprob=grads[0],
                             grad_entropy=grads[1], class_weight=cw)
    for k in ("logprob", "entropy"):
        assert G.stat_err(out[f"{k}_mean"].cpu().numpy(), [fw[f"{k}_mean"]]) <= 1.0
    assert G.rel_l2(gh.float().cpu().numpy(), dh) <= G.GRAD_REL_L2
    assert G.rel_l2(gw.float().cpu().numpy(), dw) <= G.GRAD_REL_L2


def test_odd_vocab_slices():
    """Odd and 6-mod-8 slice widths through the sharded calls, against the
    oracle (merged statistics; the slices' dW columns side by side and the
    summed partial dH)."""
    wl = W.WORKLOADS["odd_vocab"]
    bounds = (0, 333, 667, 1001)
    x = W.make_inputs(wl)
    t = G.upload(x)
    dev = G.dev()
    N, H, V = wl.N, wl.H, wl.V
    opt = flce.FlceOptions(wl.ignore_index, 0.0, flce.FLCE_REDUCTION_NONE, 0.0,
                           flce.FLCE_GRAD_F32, None)
    st = torch.cuda.current_stream().cuda_stream
    S = len(bounds) - 1
    f32 = dict(dtype=torch.float32, device=dev)
    states = torch.empty((S, N, 4), **f32)
    zl = torch.empty((S, N), **f32)
    shards = [t["weight"][:, bounds[s]:bounds[s + 1]].contiguous() for s in range(S)]
    for s in range(S):
        a, b = bounds[s], bounds[s + 1]
        fb, bb = flce.flce_workspace_size(N, H, b - a, 0)
        wk = torch.empty(max(fb, bb), dtype=torch.uint8, device=dev)
        flce.flce_forward_shard(t["hidden"].data_ptr(), shards[s].data_ptr(), t["labels"].data_ptr(),
                                N, H, b - a, a, V, opt, states[s].data_ptr(), zl[s].data_ptr(),
                                wk.data_ptr(), wk.numel(), st)
    mb = flce.flce_merge_workspace_size(N)
    mw = torch.empty(mb, dtype=torch.uint8, device=dev)
    out = {k: torch.empty(N, **f32) for k in ("lse",) + OUTS}
    flce.flce_merge_shards(states.data_ptr(), zl.data_ptr(), S, t["labels"].data_ptr(), N, V, opt,
                           out["lse"].data_ptr(), out["logprob"].data_ptr(),
                           out["entropy"].data_ptr(), out["uniform_ce"].data_ptr(),
                           out["z_loss"].data_ptr(), None, mw.data_ptr(), mb, st)
    g = torch.from_numpy(x["grad_logprob"]).to(dev)
    e = torch.from_numpy(x["grad_entropy"]).to(dev)
    gh = torch.zeros((N, H), **f32)
    gws = []
    for s in range(S):
        a, b = bounds[s], bounds[s + 1]
        _, bb = flce.flce_workspace_size(N, H, b - a, 0)
        wk = torch.empty(bb, dtype=torch.uint8, device=dev)
        ghp = torch.empty((N, H), **f32)
        gwp = torch.empty((H, b - a), **f32)
        flce.flce_backward_shard(t["hidden"].data_ptr(), shards[s].data_ptr(),
                                 t["labels"].data_ptr(), N, H, b - a, a, V, opt,
                                 out["lse"].data_ptr(), out["entropy"].data_ptr(), g.data_ptr(),
                                 e.data_ptr(), None, None, ghp.data_ptr(), gwp.data_ptr(),
                                 wk.data_ptr(), wk.numel(), st)
        gh += ghp
        gws.append(gwp)
    torch.cuda.synchronize()
    hf = W.bf16_bits_to_f32(x["hidden"])
    wf = W.bf16_bits_to_f32(x["weight"])
    fw = oracle.forward(hf, wf, x["labels"])
    dh, dw = oracle.backward(hf, wf, x["labels"], grad_logprob=x["grad_logprob"],
                             grad_entropy=x["grad_entropy"])
    for k in ("lse", "logprob", "entropy"):
        assert G.stat_err(out[k].cpu().numpy(), fw[k]) <= 1.0, k
    assert G.rel_l2(gh.cpu().numpy(), dh) <= G.GRAD_REL_L2
    assert G.rel_l2(torch.cat(gws, dim=1).cpu().numpy(), dw) <= G.GRAD_REL_L2


@pytest.mark.parametrize("chunk,gdt", [(0, "bf16"), (256, "bf16"), (256, "f32")])
def test_odd_vocab_fused(chunk, gdt):
    """The fused call with V = 1001: one chunk, and 256-token chunks whose dW
    accumulates in fp32 across chunks (in a padded buffer)."""
    wl = W.WORKLOADS["odd_vocab"]
    x = W.make_inputs(wl)
    print(f"[odd V fused] chunk={chunk} {gdt}", flush=True)
    t = G.upload(x)
    res = flce.forward_backward(t["hidden"], t["weight"], t["labels"], t["grad_logprob"],
                                t["grad_entropy"], ignore_index=wl.ignore_index, softcap=4.0,
                                grad_dtype=gdt, chunk_tokens=chunk)
    torch.cuda.synchronize()
    assert res["grad_weight"].shape == (wl.H, wl.V)
    hf = W.bf16_bits_to_f32(x["hidden"])
    wf = W.bf16_bits_to_f32(x["weight"])
    fw = oracle.forward(hf, wf, x["labels"], ignore_index=wl.ignore_index, softcap_c=4.0)
    dh, dw = oracle.backward(hf, wf, x["labels"], ignore_index=wl.ignore_index, softcap_c=4.0,
                             grad_logprob=x["grad_logprob"], grad_entropy=x["grad_entropy"])
    for k in ("lse", "logprob", "entropy"):
        assert G.stat_err(res[k].cpu().numpy(), fw[k]) <= 1.0, k
    assert G.rel_l2(res["grad_hidden"].float().cpu().numpy(), dh) <= G.GRAD_REL_L2
    assert G.rel_l2(res["grad_weight"].float().cpu().numpy(), dw) <= G.GRAD_REL_L2
