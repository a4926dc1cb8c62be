"""GPU parity of target (class) weights in the mean and sum reductions
against the float64 oracle, on the same seeded bf16 inputs and seeded class
weights: the recompute path (flce_forward_ex / flce_backward_ex), the fused
forward + backward and the vocabulary-sharded calls.

Tolerances as for the other outputs: per-token and reduced outputs within
2e-3 absolute or 1e-3 relative, gradients within 1e-2 relative L2. One exact
check: when every valid token's class weight is 0 the means and both
gradients are exactly 0.
"""
import numpy as np
import pytest
import torch

import oracle
import gpu_helpers as G
from linear_cross_entropy_tile_amd import flce, workloads as W

pytestmark = pytest.mark.gpu

OUTS = ("logprob", "entropy", "uniform_ce", "z_loss")

# (workload, reduction, softcap, z-loss scale, fraction of zero class weights)
CASES = [("odd_tails", "mean", 0.0, 0.0, 0.1), ("odd_tails", "sum", 5.0, 0.05, 0.0),
         ("tiny", "mean", 0.0, 0.02, 0.3), ("mean_ignore", "mean", 0.0, 0.02, 0.05),
         ("dw_split", "sum", 0.0, 0.0, 0.1)]


def _scalars(seed):
    return [np.array([v], dtype=np.float32) for v in np.random.default_rng(seed).standard_normal(4)]


def _oracle(x, wl, reduction, cap, lam, cw, grads):
    hf = W.bf16_bits_to_f32(x["hidden"])
    wf = W.bf16_bits_to_f32(x["weight"])
    fw = oracle.forward(hf, wf, x["labels"], ignore_index=wl.ignore_index, softcap_c=cap,
                        reduction=reduction, z_loss_scale=lam, class_weight=cw)
    dh, dw = oracle.backward(hf, wf, x["labels"], ignore_index=wl.ignore_index, softcap_c=cap,
                             reduction=reduction, grad_logprob=grads[0], grad_entropy=grads[1],
                             grad_uniform_ce=grads[2], grad_z_loss=grads[3], z_loss_scale=lam,
                             class_weight=cw)
    return fw, dh, dw


def _check(name, out, reduced_of, gh, gw, fw, dh, dw, reduction):
    for k in ("lse",) + OUTS:
        e = G.stat_err(out[k].cpu().numpy(), fw[k])
        assert e <= 1.0, f"{name} {k}: error {e:.3f} x tolerance"
    for k in OUTS:
        key = f"{k}_{reduction}"
        e = G.stat_err(reduced_of(k).cpu().numpy(), [fw[key]])
        assert e <= 1.0, f"{name} {key}: error {e:.3f} x tolerance"
    for got, ref, what in ((gh, dh, "grad_hidden"), (gw, dw, "grad_weight")):
        e = G.rel_l2(got.float().cpu().numpy(), ref)
        assert e <= G.GRAD_REL_L2, f"{name} {what} rel L2 {e:.2e}"


@pytest.mark.parametrize("name,reduction,cap,lam,zf", CASES,
                         ids=[f"{c[0]}-{c[1]}-cap{c[2]:g}" for c in CASES])
def test_class_weight_parity(name, reduction, cap, lam, zf):
    wl = W.WORKLOADS[name]
    x = W.make_inputs(wl)
    print(f"[cw] {name} N={wl.N} H={wl.H} V={wl.V} {reduction} cap={cap} lam={lam}", flush=True)
    t = G.upload(x)
    cw = W.make_class_weights(wl.V, wl.seed + 31, zf)
    cwt = torch.from_numpy(cw).to(G.dev())
    grads = _scalars(wl.seed + 41)
    g = [torch.from_numpy(a).to(G.dev()) for a in grads]
    out = flce.forward(t["hidden"], t["weight"], t["labels"], ignore_index=wl.ignore_index,
                       softcap=cap, reduction=reduction, z_loss_scale=lam, aux=True,
                       class_weight=cwt)
    gh, gw = flce.backward(t["hidden"], t["weight"], t["labels"], out["lse"], out["entropy"],
                           g[0], g[1], ignore_index=wl.ignore_index, softcap=cap,
                           reduction=reduction, grad_uniform_ce=g[2], grad_z_loss=g[3],
                           z_loss_scale=lam, class_weight=cwt)
    torch.cuda.synchronize()
    fw, dh, dw = _oracle(x, wl, reduction, cap, lam, cw, grads)
    _check(name, out, lambda k: out[f"{k}_{reduction}"], gh, gw, fw, dh, dw, reduction)


@pytest.mark.parametrize("name,reduction", [("odd_tails", "mean"), ("mean_ignore", "sum")])
def test_class_weight_fused(name, reduction):
    wl = W.WORKLOADS[name]
    x = W.make_inputs(wl)
    print(f"[cw fused] {name} N={wl.N} H={wl.H} V={wl.V} {reduction}", flush=True)
    t = G.upload(x)
    cw = W.make_class_weights(wl.V, wl.seed + 32, 0.1)
    cwt = torch.from_numpy(cw).to(G.dev())
    grads = _scalars(wl.seed + 42)
    g = [torch.from_numpy(a).to(G.dev()) for a in grads]
    lam = 0.03
    res = flce.forward_backward(t["hidden"], t["weight"], t["labels"], g[0], g[1],
                                ignore_index=wl.ignore_index, reduction=reduction,
                                grad_uniform_ce=g[2], grad_z_loss=g[3], z_loss_scale=lam,
                                aux=True, class_weight=cwt)
    torch.cuda.synchronize()
    fw, dh, dw = _oracle(x, wl, reduction, 0.0, lam, cw, grads)
    _check(name, res, lambda k: res[f"{k}_{reduction}"], res["grad_hidden"], res["grad_weight"],
           fw, dh, dw, reduction)


def test_class_weight_sharded():
    wl = W.WORKLOADS["mean_ignore"]
    bounds = (0, 8000, 19992, 32000)
    x = W.make_inputs(wl)
    print(f"[cw shard] mean_ignore slices={bounds}", flush=True)
    t = G.upload(x)
    dev = G.dev()
    N, H, V = wl.N, wl.H, wl.V
    cw = W.make_class_weights(V, wl.seed + 33, 0.05)
    cwt = torch.from_numpy(cw).to(dev)
    grads = _scalars(wl.seed + 43)
    g = [torch.from_numpy(a).to(dev) for a in grads]
    lam = 0.02
    opt = flce.FlceOptions(wl.ignore_index, 0.0, flce.FLCE_REDUCTION_MEAN, lam, flce.FLCE_GRAD_F32,
                           cwt.data_ptr())
    stream = torch.cuda.current_stream().cuda_stream
    S = len(bounds) - 1
    f32 = dict(dtype=torch.float32, device=dev)
    states = torch.empty((S, N, 4), **f32)
    zl = torch.empty((S, N), **f32)
    shards = [t["weight"][:, bounds[s]:bounds[s + 1]].contiguous() for s in range(S)]
    for s in range(S):
        a, b = bounds[s], bounds[s + 1]
        fb, bb = flce.flce_workspace_size(N, H, b - a, flce.FLCE_REDUCTION_MEAN)
        wk = torch.empty(max(fb, bb), dtype=torch.uint8, device=dev)
        flce.flce_forward_shard(t["hidden"].data_ptr(), shards[s].data_ptr(),
                                t["labels"].data_ptr(), N, H, b - a, a, V, opt,
                                states[s].data_ptr(), zl[s].data_ptr(), wk.data_ptr(), wk.numel(),
                                stream)
    mb = flce.flce_merge_workspace_size(N)
    mw = torch.empty(mb, dtype=torch.uint8, device=dev)
    out = {k: torch.empty(N, **f32) for k in ("lse",) + OUTS}
    reduced = torch.empty(4, **f32)
    flce.flce_merge_shards(states.data_ptr(), zl.data_ptr(), S, t["labels"].data_ptr(), N, V, opt,
                           out["lse"].data_ptr(), out["logprob"].data_ptr(),
                           out["entropy"].data_ptr(), out["uniform_ce"].data_ptr(),
                           out["z_loss"].data_ptr(), reduced.data_ptr(), mw.data_ptr(), mb, stream)
    gh = torch.zeros((N, H), **f32)
    gws = []
    for s in range(S):
        a, b = bounds[s], bounds[s + 1]
        _, bb = flce.flce_workspace_size(N, H, b - a, flce.FLCE_REDUCTION_MEAN)
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
    fw, dh, dw = _oracle(x, wl, "mean", 0.0, lam, cw, grads)
    _check("sharded", out, lambda k: reduced[OUTS.index(k):OUTS.index(k) + 1], gh,
           torch.cat(gws, dim=1), fw, dh, dw, "mean")


def test_zero_class_weights_give_zero():
    wl = W.WORKLOADS["odd_tails"]
    x = W.make_inputs(wl)
    t = G.upload(x)
    cwt = torch.zeros(wl.V, dtype=torch.float32, device=G.dev())
    one = torch.ones(1, dtype=torch.float32, device=G.dev())
    out = flce.forward(t["hidden"], t["weight"], t["labels"], reduction="mean", class_weight=cwt)
    gh, gw = flce.backward(t["hidden"], t["weight"], t["labels"], out["lse"], out["entropy"],
                           one, one, reduction="mean", class_weight=cwt)
    res = flce.forward_backward(t["hidden"], t["weight"], t["labels"], one, one,
                                reduction="mean", class_weight=cwt)
    torch.cuda.synchronize()
    for o in (out, res):
        assert o["logprob_mean"].item() == 0.0 and o["entropy_mean"].item() == 0.0
    for a in (gh, gw, res["grad_hidden"], res["grad_weight"]):
        assert torch.count_nonzero(a).item() == 0


def test_class_weights_invalid_labels():
    """Labels outside [0, V) that are not ignore_index are treated as ignored
    (their class weight is never read) and counted in the status word; the
    weighted mean and gradients equal the oracle's with those tokens ignored."""
    wl = W.WORKLOADS["odd_tails"]
    x = W.make_inputs(wl)
    bad = x["labels"].copy()
    bad[3] = wl.V
    bad[5] = -7
    bad[6] = 10 ** 12
    xb = dict(x)
    xb["labels"] = bad
    t = G.upload(xb)
    cw = W.make_class_weights(wl.V, wl.seed + 34, 0.1)
    cwt = torch.from_numpy(cw).to(G.dev())
    grads = _scalars(wl.seed + 44)
    g = [torch.from_numpy(a).to(G.dev()) for a in grads]
    out = flce.forward(t["hidden"], t["weight"], t["labels"], reduction="mean", aux=True,
                       class_weight=cwt)
    gh, gw = flce.backward(t["hidden"], t["weight"], t["labels"], out["lse"], out["entropy"],
                           g[0], g[1], reduction="mean", grad_uniform_ce=g[2],
                           grad_z_loss=g[3], class_weight=cwt)
    res = flce.forward_backward(t["hidden"], t["weight"], t["labels"], g[0], g[1],
                                reduction="mean", grad_uniform_ce=g[2], grad_z_loss=g[3],
                                aux=True, class_weight=cwt)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream().cuda_stream
    assert flce.flce_get_status(out["workspace"].data_ptr(), stream) == 3
    assert flce.flce_get_status(res["workspace"].data_ptr(), stream) == 3
    xo = dict(x)
    xo["labels"] = np.where((bad >= 0) & (bad < wl.V), bad, wl.ignore_index)
    fw, dh, dw = _oracle(xo, wl, "mean", 0.0, 0.0, cw, grads)
    _check("invalid labels", out, lambda k: out[f"{k}_mean"], gh, gw, fw, dh, dw, "mean")
    _check("invalid labels fused", res, lambda k: res[f"{k}_mean"], res["grad_hidden"],
           res["grad_weight"], fw, dh, dw, "mean")


def test_class_weights_empty_batch():
    """N = 0 with class weights: means 0, zero weight gradient."""
    d = G.dev()
    h = torch.empty((0, 64), dtype=torch.bfloat16, device=d)
    w = torch.randn((64, 512), device=d).to(torch.bfloat16)
    y = torch.empty(0, dtype=torch.int64, device=d)
    cwt = torch.ones(512, dtype=torch.float32, device=d)
    out = flce.forward(h, w, y, reduction="mean", class_weight=cwt)
    g = torch.ones(1, device=d)
    gh, gw = flce.backward(h, w, y, out["lse"], out["entropy"], g, g, reduction="mean",
                           class_weight=cwt)
    torch.cuda.synchronize()
    assert out["logprob_mean"].item() == 0.0 and out["entropy_mean"].item() == 0.0
    assert gh.shape == (0, 64) and torch.count_nonzero(gw).item() == 0


def test_class_weights_f32_gradients_round_to_bf16():
    """fp32 gradient outputs under class weights: within tolerance of the
    oracle, and the bf16 outputs are exactly their round-to-nearest-even (the
    same fp32 arithmetic)."""
    wl = W.WORKLOADS["dw_split"]
    x = W.make_inputs(wl)
    t = G.upload(x)
    cw = W.make_class_weights(wl.V, wl.seed + 35, 0.1)
    cwt = torch.from_numpy(cw).to(G.dev())
    grads = _scalars(wl.seed + 45)
    g = [torch.from_numpy(a).to(G.dev()) for a in grads]
    out = flce.forward(t["hidden"], t["weight"], t["labels"], reduction="mean", class_weight=cwt)
    res = {}
    for dt in ("f32", "bf16"):
        res[dt] = flce.backward(t["hidden"], t["weight"], t["labels"], out["lse"], out["entropy"],
                                g[0], g[1], reduction="mean", grad_dtype=dt, class_weight=cwt)
    torch.cuda.synchronize()
    gh32, gw32 = res["f32"]
    gh16, gw16 = res["bf16"]
    assert gh32.dtype == torch.float32 and gh16.dtype == torch.bfloat16
    assert torch.equal(gh32.to(torch.bfloat16), gh16) and torch.equal(gw32.to(torch.bfloat16), gw16)
    _, dh, dw = _oracle(x, wl, "mean", 0.0, 0.0, cw, [grads[0], grads[1], None, None])
    assert G.rel_l2(gh32.cpu().numpy(), dh) <= G.GRAD_REL_L2
    assert G.rel_l2(gw32.cpu().numpy(), dw) <= G.GRAD_REL_L2
