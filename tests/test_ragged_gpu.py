"""Ragged shapes at the tile boundaries, through the recompute entry points
and the fused call, against the float64 oracle: a single token, token counts
one below and one above a 256-token tile, hidden sizes that are not a
multiple of the 32-wide K block or of a 256-row strip, vocabularies of one
8-column group and just past a 256-column tile, with softcap, ignored tokens
and every reduction. Tolerances as in the other parity tests."""
import numpy as np
import pytest
import torch

import oracle
import gpu_helpers as G
from linear_cross_entropy_tile_amd import flce, workloads as W

pytestmark = pytest.mark.gpu

# (N, H, V, softcap, reduction)
SHAPES = [(1, 8, 8, 0.0, "none"), (1, 264, 520, 5.0, "mean"), (255, 264, 520, 0.0, "sum"),
          (257, 136, 264, 3.0, "none"), (513, 8, 2056, 0.0, "mean"), (40, 520, 8, 2.0, "none")]


@pytest.mark.parametrize("N,H,V,cap,red", SHAPES,
                         ids=[f"N{s[0]}-H{s[1]}-V{s[2]}-c{s[3]:g}-{s[4]}" for s in SHAPES])
def test_ragged(N, H, V, cap, red):
    wl = W.Workload("ragged", N, H, V, seed=300 + N + H + V, weight_std=1.0 / np.sqrt(H),
                    softcap=cap, reduction=red, ignore="fraction" if N > 4 else "none",
                    ignore_fraction=0.1,
                    grad_logprob=("normal",) if red == "none" else ("scalar", 0.7),
                    grad_entropy=("normal",) if red == "none" else ("scalar", -0.2))
    print(f"[ragged] N={N} H={H} V={V} cap={cap} {red}", flush=True)
    x = W.make_inputs(wl)
    t = G.upload(x)
    hf = W.bf16_bits_to_f32(x["hidden"])
    wf = W.bf16_bits_to_f32(x["weight"])
    fw = oracle.forward(hf, wf, x["labels"], ignore_index=wl.ignore_index, softcap_c=cap,
                        reduction=red)
    dh, dw = oracle.backward(hf, wf, x["labels"], ignore_index=wl.ignore_index, softcap_c=cap,
                             reduction=red, grad_logprob=x["grad_logprob"],
                             grad_entropy=x["grad_entropy"])
    rec = G.run(wl, t, keep_grads_on_gpu=True)
    fus = flce.forward_backward(t["hidden"], t["weight"], t["labels"], t["grad_logprob"],
                                t["grad_entropy"], ignore_index=wl.ignore_index, softcap=cap,
                                reduction=red, chunk_tokens=256)
    torch.cuda.synchronize()
    for name, lse, lp, ent, gh, gw in (
            ("recompute", rec["lse"], rec["logprob"], rec["entropy"], rec["grad_hidden"],
             rec["grad_weight"]),
            ("fused", fus["lse"].cpu().numpy(), fus["logprob"].cpu().numpy(),
             fus["entropy"].cpu().numpy(), fus["grad_hidden"], fus["grad_weight"])):
        for k, got in (("lse", lse), ("logprob", lp), ("entropy", ent)):
            e = G.stat_err(got, fw[k])
            assert e <= 1.0, f"{name} {k}: error {e:.3f} x tolerance"
        for k, got, ref in (("grad_hidden", gh, dh), ("grad_weight", gw, dw)):
            e = G.rel_l2(got.float().cpu().numpy(), ref)
            assert e <= G.GRAD_REL_L2, f"{name} {k} rel L2 {e:.2e}"
    if red != "none":
        for k in ("logprob", "entropy"):
            e = G.stat_err(rec[f"{k}_{red}"] if f"{k}_{red}" in rec else
                           fus[f"{k}_{red}"].cpu().numpy(), [fw[f"{k}_{red}"]])
            assert e <= 1.0, f"{k}_{red}: error {e:.3f} x tolerance"
