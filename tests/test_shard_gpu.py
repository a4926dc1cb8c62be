"""GPU parity of the vocabulary-sharded head on one GPU: the vocabulary is cut
into uneven slices, each slice runs flce_forward_shard on its own weight
columns, flce_merge_shards merges the slice states (the step an all-gather
feeds across GPUs), and flce_backward_shard gives each slice's dW columns and
partial dH, whose sum is dH (the step an all-reduce performs).

Compared with the float64 oracle (per-token outputs within 2e-3 absolute or
1e-3 relative; gradients within 1e-2 relative L2) and with the unsharded
library (within 1e-4: only the merge and summation order differ).
"""
import numpy as np
import pytest
import torch

import oracle
import gpu_helpers as G
from linear_cross_entropy_tile_amd import flce, workloads as W

pytestmark = pytest.mark.gpu

CASES = [("odd_tails", (0, 256, 600, 1000)), ("tiny", (0, 1024, 4096)),
         ("mean_ignore", (0, 8000, 19992, 32000)), ("softcap_saturation", (0, 100000, 256000))]
OUTS = ("logprob", "entropy", "uniform_ce", "z_loss")


def _sharded(t, wl, bounds, lam, grads):
    dev = G.dev()
    N, H = t["hidden"].shape
    V = t["weight"].shape[1]
    red = flce._REDUCTIONS[wl.reduction]
    opt = flce.FlceOptions(wl.ignore_index, wl.softcap, red, lam, flce.FLCE_GRAD_F32)
    stream = torch.cuda.current_stream().cuda_stream
    S = len(bounds) - 1
    states = torch.empty((S, N, 4), dtype=torch.float32, device=dev)
    zl = torch.empty((S, N), dtype=torch.float32, device=dev)
    shards = []
    for s in range(S):
        a, b = bounds[s], bounds[s + 1]
        ws_ = t["weight"][:, a:b].contiguous()
        shards.append(ws_)
        fb, bb = flce.flce_workspace_size(N, H, b - a, red)
        wk = torch.empty(max(fb, bb), dtype=torch.uint8, device=dev)
        flce.flce_forward_shard(t["hidden"].data_ptr(), ws_.data_ptr(), t["labels"].data_ptr(), N,
                                H, b - a, a, V, opt, states[s].data_ptr(), zl[s].data_ptr(),
                                wk.data_ptr(), wk.numel(), stream)
    mb = flce.flce_merge_workspace_size(N)
    mw = torch.empty(mb, dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    out = {k: torch.empty(N, **f32) for k in ("lse",) + OUTS}
    reduced = torch.empty(4, **f32)
    flce.flce_merge_shards(states.data_ptr(), zl.data_ptr(), S, t["labels"].data_ptr(), N, V, opt,
                           out["lse"].data_ptr(), out["logprob"].data_ptr(),
                           out["entropy"].data_ptr(), out["uniform_ce"].data_ptr(),
                           out["z_loss"].data_ptr(), reduced.data_ptr(), mw.data_ptr(), mb, stream)
    g = [torch.from_numpy(x).to(dev) for x in grads]
    gh = torch.zeros((N, H), **f32)
    gws = []
    for s in range(S):
        a, b = bounds[s], bounds[s + 1]
        _, bb = flce.flce_workspace_size(N, H, b - a, red)
        wk = torch.empty(bb, dtype=torch.uint8, device=dev)
        ghp = torch.empty((N, H), **f32)
        gwp = torch.empty((H, b - a), **f32)
        flce.flce_backward_shard(t["hidden"].data_ptr(), shards[s].data_ptr(),
                                 t["labels"].data_ptr(), N, H, b - a, a, V, opt,
                                 out["lse"].data_ptr(), out["entropy"].data_ptr(),
                                 g[0].data_ptr(), g[1].data_ptr(), g[2].data_ptr(),
                                 g[3].data_ptr(), ghp.data_ptr(), gwp.data_ptr(), wk.data_ptr(),
                                 wk.numel(), stream)
        gh += ghp
        gws.append(gwp)
    torch.cuda.synchronize()
    return out, reduced, gh, torch.cat(gws, dim=1)


@pytest.mark.parametrize("name,bounds", CASES, ids=[c[0] for c in CASES])
def test_sharded_head(name, bounds):
    wl = W.WORKLOADS[name]
    x = W.make_inputs(wl)
    print(f"[shard] {name} N={wl.N} H={wl.H} V={wl.V} slices={bounds}", flush=True)
    t = G.upload(x)
    lam = 0.03
    rng = np.random.default_rng(wl.seed + 5)
    if wl.reduction == "none":
        grads = [rng.standard_normal(wl.N).astype(np.float32) for _ in OUTS]
    else:
        grads = [np.array([v], dtype=np.float32) for v in rng.standard_normal(4)]
    out, reduced, gh, gw = _sharded(t, wl, bounds, lam, grads)

    # The unsharded library on the same inputs.
    ref = flce.forward(t["hidden"], t["weight"], t["labels"], ignore_index=wl.ignore_index,
                       softcap=wl.softcap, reduction=wl.reduction, z_loss_scale=lam, aux=True)
    gt = [torch.from_numpy(a).to(G.dev()) for a in grads]
    gh1, gw1 = flce.backward(t["hidden"], t["weight"], t["labels"], ref["lse"], ref["entropy"],
                             gt[0], gt[1], ignore_index=wl.ignore_index, softcap=wl.softcap,
                             reduction=wl.reduction, grad_uniform_ce=gt[2], grad_z_loss=gt[3],
                             z_loss_scale=lam, grad_dtype="f32")
    for k in ("lse",) + OUTS:
        d = (out[k] - ref[k]).abs().max().item()
        assert d <= 1e-4 * max(1.0, ref[k].abs().max().item()), f"{name} {k} vs unsharded: {d}"
    assert G.rel_l2(gh.cpu().numpy(), gh1.cpu().numpy()) <= 1e-4
    assert G.rel_l2(gw.cpu().numpy(), gw1.cpu().numpy()) <= 1e-4

    hf = W.bf16_bits_to_f32(x["hidden"])
    wf = W.bf16_bits_to_f32(x["weight"])
    fw = oracle.forward(hf, wf, x["labels"], ignore_index=wl.ignore_index, softcap_c=wl.softcap,
                        reduction=wl.reduction, z_loss_scale=lam)
    dh, dw = oracle.backward(hf, wf, x["labels"], ignore_index=wl.ignore_index,
                             softcap_c=wl.softcap, reduction=wl.reduction, grad_logprob=grads[0],
                             grad_entropy=grads[1], grad_uniform_ce=grads[2],
                             grad_z_loss=grads[3], z_loss_scale=lam)
    for k in ("lse",) + OUTS:
        e = G.stat_err(out[k].cpu().numpy(), fw[k])
        assert e <= 1.0, f"{name} {k}: error {e:.3f} x tolerance"
    if wl.reduction != "none":
        for i, k in enumerate(OUTS):
            e = G.stat_err(reduced[i:i + 1].cpu().numpy(), [fw[f"{k}_{wl.reduction}"]])
            assert e <= 1.0, f"{name} reduced {k}: error {e:.3f} x tolerance"
    assert G.rel_l2(gh.cpu().numpy(), dh) <= G.GRAD_REL_L2
    assert G.rel_l2(gw.cpu().numpy(), dw) <= G.GRAD_REL_L2
