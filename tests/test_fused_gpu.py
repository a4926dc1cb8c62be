"""GPU parity of the fused forward + backward (flce_forward_backward: the logit
gradient formed from logits kept during the forward, no recompute) against the
float64 oracle on the same seeded bf16 inputs, at small sizes over every
option and at the full workload sizes against the stored oracle values.

Tolerances as for the other entry points: per-token and reduced outputs within
2e-3 absolute or 1e-3 relative, gradients within 1e-2 relative L2. Exact
checks:
  * the forward outputs equal those of flce_forward_ex bit for bit (the same
    tile statistics, merged in the same order);
  * bf16 gradients equal the fp32 ones rounded to nearest even (the same fp32
    arithmetic in both modes, also when dW is accumulated over token chunks);
  * ignored tokens get zero outputs and zero grad_hidden rows.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import gpu_helpers as G
from linear_cross_entropy_tile_amd import flce, workloads as W

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
OUTS = ("logprob", "entropy", "uniform_ce", "z_loss")

# (workload, reduction, z-loss scale, tokens per chunk; 0 = the default rule)
CASES = [
    ("tiny", "none", 0.0, 0),                  # one chunk, dW written directly
    ("odd_tails", "sum", 0.05, 0),             # ragged N, H, V
    ("mean_ignore", "mean", 0.02, 1024),       # 4 chunks: dW accumulated in fp32
    ("dw_split", "none", 0.1, 256),            # 16 chunks of one token block each
    ("softcap_saturation", "none", 0.01, 256),  # capped logits near +-c, 2 chunks
    ("odd_capped", "mean", 0.02, 256),         # capped logits, ragged N and V, 2 chunks
]


def _grads(N, reduction, seed):
    rng = np.random.default_rng(seed)
    if reduction == "none":
        return [rng.standard_normal(N).astype(np.float32) for _ in OUTS]
    return [np.array([v], dtype=np.float32) for v in rng.standard_normal(4)]


def _fused(t, wl, reduction, lam, grads, grad_dtype, chunk):
    g = [torch.from_numpy(a).to(G.dev()) for a in grads]
    out = flce.forward_backward(t["hidden"], t["weight"], t["labels"], g[0], g[1],
                                ignore_index=wl.ignore_index, softcap=wl.softcap,
                                reduction=reduction, grad_uniform_ce=g[2], grad_z_loss=g[3],
                                z_loss_scale=lam, grad_dtype=grad_dtype, aux=True,
                                chunk_tokens=chunk)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name,reduction,lam,chunk", CASES,
                         ids=[f"{c[0]}-{c[1]}-c{c[3]}" for c in CASES])
def test_fused_parity(name, reduction, lam, chunk):
    wl = W.WORKLOADS[name]
    x = W.make_inputs(wl)
    print(f"[fused] {name} N={wl.N} H={wl.H} V={wl.V} {reduction} lam={lam} chunk={chunk}",
          flush=True)
    t = G.upload(x)
    grads = _grads(wl.N, reduction, wl.seed + 91)
    f32 = _fused(t, wl, reduction, lam, grads, "f32", chunk)
    b16 = _fused(t, wl, reduction, lam, grads, "bf16", chunk)
    assert f32["grad_hidden"].dtype == torch.float32
    assert b16["grad_hidden"].dtype == torch.bfloat16

    hf = W.bf16_bits_to_f32(x["hidden"])
    wf = W.bf16_bits_to_f32(x["weight"])
    fw = oracle.forward(hf, wf, x["labels"], ignore_index=wl.ignore_index, softcap_c=wl.softcap,
                        reduction=reduction, z_loss_scale=lam)
    dh, dw = oracle.backward(hf, wf, x["labels"], ignore_index=wl.ignore_index,
                             softcap_c=wl.softcap, reduction=reduction, grad_logprob=grads[0],
                             grad_entropy=grads[1], grad_uniform_ce=grads[2],
                             grad_z_loss=grads[3], z_loss_scale=lam)
    for k in ("lse",) + OUTS:
        e = G.stat_err(f32[k].cpu().numpy(), fw[k])
        assert e <= 1.0, f"{name} {k}: error {e:.3f} x tolerance"
    if reduction != "none":
        for k in OUTS:
            key = f"{k}_{reduction}"
            e = G.stat_err(f32[key].cpu().numpy(), [fw[key]])
            assert e <= 1.0, f"{name} {key}: error {e:.3f} x tolerance"
    for out in (f32, b16):
        for what, ref in (("grad_hidden", dh), ("grad_weight", dw)):
            e = G.rel_l2(out[what].float().cpu().numpy(), ref)
            assert e <= G.GRAD_REL_L2, f"{name} {what} {out[what].dtype} rel L2 {e:.2e}"
    assert torch.equal(f32["grad_hidden"].to(torch.bfloat16), b16["grad_hidden"])
    assert torch.equal(f32["grad_weight"].to(torch.bfloat16), b16["grad_weight"])

    # The forward outputs are those of the separate forward, bit for bit.
    sep = flce.forward(t["hidden"], t["weight"], t["labels"], ignore_index=wl.ignore_index,
                       softcap=wl.softcap, reduction=reduction, z_loss_scale=lam, aux=True)
    torch.cuda.synchronize()
    for k in ("lse",) + OUTS:
        assert torch.equal(sep[k], f32[k]), f"{name} {k} differs from flce_forward_ex"
    if reduction != "none":
        for k in OUTS:
            assert torch.equal(sep[f"{k}_{reduction}"], f32[f"{k}_{reduction}"])

    ign = torch.from_numpy(x["labels"] == wl.ignore_index).to(G.dev())
    if bool(ign.any()):
        for k in ("lse",) + OUTS:
            assert torch.count_nonzero(f32[k][ign]).item() == 0
        assert torch.count_nonzero(f32["grad_hidden"][ign]).item() == 0


def test_fused_chunking_keeps_results():
    """One chunk, four chunks, and chunks of one token block: identical forward
    outputs; gradients that differ only by fp32 summation order."""
    wl = W.WORKLOADS["mean_ignore"]
    x = W.make_inputs(wl)
    t = G.upload(x)
    grads = _grads(wl.N, "none", wl.seed + 5)
    runs = [_fused(t, wl, "none", 0.0, grads, "f32", c) for c in (0, 1024, 256)]
    for r in runs[1:]:
        for k in ("lse", "logprob", "entropy"):
            assert torch.equal(runs[0][k], r[k])
        for k in ("grad_hidden", "grad_weight"):
            e = G.rel_l2(r[k].cpu().numpy(), runs[0][k].cpu().numpy())
            assert e <= 1e-5, f"{k}: chunked vs one chunk rel L2 {e:.2e}"


def test_fused_all_ignored():
    wl = W.WORKLOADS["all_ignored"]
    x = W.make_inputs(wl)
    t = G.upload(x)
    out = _fused(t, wl, "mean", 0.0, _grads(wl.N, "mean", 3), "bf16", 0)
    for k in ("lse",) + OUTS:
        assert torch.count_nonzero(out[k]).item() == 0
    for k in OUTS:
        assert out[f"{k}_mean"].item() == 0.0
    assert torch.count_nonzero(out["grad_hidden"]).item() == 0
    assert torch.count_nonzero(out["grad_weight"]).item() == 0


def test_fused_matches_recompute_path():
    """The same inputs through flce_forward + flce_backward (recompute) and
    the fused call: forward outputs identical, gradients within the bf16
    rounding of the kept logits."""
    wl = W.WORKLOADS["tiny"].with_(softcap=5.0)
    x = W.make_inputs(wl)
    t = G.upload(x)
    res = G.run(wl, t, keep_grads_on_gpu=True)
    out = flce.forward_backward(t["hidden"], t["weight"], t["labels"], t["grad_logprob"],
                                t["grad_entropy"], ignore_index=wl.ignore_index,
                                softcap=wl.softcap, reduction=wl.reduction)
    torch.cuda.synchronize()
    for k in ("lse", "logprob", "entropy"):
        assert np.array_equal(out[k].cpu().numpy(), res[k])
    for k in ("grad_hidden", "grad_weight"):
        e = G.rel_l2(out[k].float().cpu().numpy(), res[k].float().cpu().numpy())
        assert e <= 5e-3, f"{k}: fused vs recompute rel L2 {e:.2e}"


FULL = ["llama3_head", "gemma2_softcap", "rl_rollout"]


@pytest.mark.parametrize("name", FULL)
def test_fused_full_size(name):
    """At the full sizes, in the configuration the benchmark times, against
    the stored oracle values (every token's statistics; sampled dHidden rows
    and dWeight columns; every row and column through the projections)."""
    path = os.path.join(HERE, "golden", f"{name}.npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated")
    ref = np.load(path)
    wl = W.WORKLOADS[name]
    print(f"[fused full] {name} N={wl.N} H={wl.H} V={wl.V}", flush=True)
    x = W.make_inputs(wl)
    t = G.upload(x)
    out = flce.forward_backward(t["hidden"], t["weight"], t["labels"], t["grad_logprob"],
                                t["grad_entropy"], ignore_index=wl.ignore_index,
                                softcap=wl.softcap, reduction=wl.reduction)
    torch.cuda.synchronize()
    for k in ("lse", "logprob", "entropy"):
        e = G.stat_err(out[k].cpu().numpy(), ref[k])
        assert e <= 1.0, f"{name} {k}: error {e:.3f} x tolerance"
    if wl.reduction == "mean":
        for k in ("logprob", "entropy"):
            e = G.stat_err(out[f"{k}_mean"].cpu().numpy(), ref[f"{k}_mean"])
            assert e <= 1.0, f"{name} {k}_mean: error {e:.3f} x tolerance"
    rows = torch.from_numpy(ref["rows"]).to(G.dev())
    cols = torch.from_numpy(ref["cols"]).to(G.dev())
    gh_rows = out["grad_hidden"].index_select(0, rows).float().cpu().numpy()
    gw_cols = out["grad_weight"].index_select(1, cols).float().cpu().numpy()
    e = G.rel_l2(gh_rows, ref["dhidden_rows"])
    assert e <= G.GRAD_REL_L2, f"{name} grad_hidden rows rel L2 {e:.2e}"
    e = G.rel_l2(gw_cols, ref["dweight_cols"])
    assert e <= G.GRAD_REL_L2, f"{name} grad_weight cols rel L2 {e:.2e}"
    G.check_projections(name, wl, out["grad_hidden"], out["grad_weight"], ref,
                        x["labels"] != wl.ignore_index)
    ign = torch.from_numpy(x["labels"] == wl.ignore_index).to(G.dev())
    if bool(ign.any()):
        assert torch.count_nonzero(out["grad_hidden"][ign]).item() == 0


def test_fused_mostly_ignored_chunks():
    """Most tokens ignored, one token block per chunk: only the first chunks
    hold valid tokens, the chunk holding the last one writes dW and the empty
    chunks exit. Against the oracle and the one-chunk run."""
    wl = W.WORKLOADS["dw_split"]
    x = W.make_inputs(wl)
    rng = np.random.default_rng(7)
    keep = np.sort(rng.choice(wl.N, size=300, replace=False))
    labels = np.full(wl.N, wl.ignore_index, dtype=np.int64)
    labels[keep] = x["labels"][keep]
    x = dict(x, labels=labels)
    t = G.upload(x)
    grads = _grads(wl.N, "sum", 11)
    outs = [_fused(t, wl, "sum", 0.0, grads, "bf16", c) for c in (256, 0)]
    hf = W.bf16_bits_to_f32(x["hidden"])
    wf = W.bf16_bits_to_f32(x["weight"])
    dh, dw = oracle.backward(hf, wf, labels, ignore_index=wl.ignore_index, softcap_c=wl.softcap,
                             reduction="sum", grad_logprob=grads[0], grad_entropy=grads[1],
                             grad_uniform_ce=grads[2], grad_z_loss=grads[3], z_loss_scale=0.0)
    for out in outs:
        for what, ref in (("grad_hidden", dh), ("grad_weight", dw)):
            e = G.rel_l2(out[what].float().cpu().numpy(), ref)
            assert e <= G.GRAD_REL_L2, f"{what} rel L2 {e:.2e}"
    assert torch.equal(outs[0]["lse"], outs[1]["lse"])


def test_fused_full_size_class_weights():
    """The fused call on the Gemma2-shaped head with the seeded class weights
    of the stored variant gemma2_softcap_weighted: weighted means and sampled
    gradient rows / columns against those stored oracle values."""
    name = "gemma2_softcap_weighted"
    path = os.path.join(HERE, "golden", f"{name}.npz")
    if not os.path.exists(path):
        pytest.skip(f"{path} not generated")
    import sys
    sys.path.insert(0, os.path.join(HERE, "golden"))
    import make_golden
    ref = np.load(path)
    wl = W.WORKLOADS[make_golden.WEIGHTED[name][0]]
    print(f"[fused full] {name} N={wl.N} H={wl.H} V={wl.V}", flush=True)
    x = W.make_inputs(wl)
    t = G.upload(x)
    cw = torch.from_numpy(make_golden.class_weights(name)).to(G.dev())
    out = flce.forward_backward(t["hidden"], t["weight"], t["labels"], t["grad_logprob"],
                                t["grad_entropy"], ignore_index=wl.ignore_index,
                                softcap=wl.softcap, reduction=wl.reduction, class_weight=cw)
    torch.cuda.synchronize()
    for k in ("lse", "logprob", "entropy", "logprob_mean", "entropy_mean"):
        e = G.stat_err(out[k].cpu().numpy(), ref[k])
        assert e <= 1.0, f"{name} {k}: error {e:.3f} x tolerance"
    rows = torch.from_numpy(ref["rows"]).to(G.dev())
    cols = torch.from_numpy(ref["cols"]).to(G.dev())
    e = G.rel_l2(out["grad_hidden"].index_select(0, rows).float().cpu().numpy(),
                 ref["dhidden_rows"])
    assert e <= G.GRAD_REL_L2, f"{name} grad_hidden rows rel L2 {e:.2e}"
    e = G.rel_l2(out["grad_weight"].index_select(1, cols).float().cpu().numpy(),
                 ref["dweight_cols"])
    assert e <= G.GRAD_REL_L2, f"{name} grad_weight cols rel L2 {e:.2e}"
