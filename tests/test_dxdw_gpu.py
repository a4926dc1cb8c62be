"""The combined dH + dW launch (bwd_dxdw_kernel), which the backward uses per
vocabulary chunk when the two tile sets have equal K lengths and one grid
needs fewer rounds of CUs than two (the Gemma2-shaped head's full chunks;
covered at full size by tests/test_parity_full_gpu.py).

FLCE_DXDW=1 forces it on every chunk with direct dW stores and FLCE_DXDW=0
turns it off: the gradients must be bit for bit those of the separate
launches (the same tile code runs either way), and within the usual
tolerance of the oracle (1e-2 relative L2), for bf16 and fp32 outputs, with
ignored tokens, several vocabulary chunks and K-split dH.
"""
import numpy as np
import pytest
import torch

import oracle
import gpu_helpers as G
from linear_cross_entropy_tile_amd import flce, workloads as W

pytestmark = pytest.mark.gpu

# (workload, FLCE_D_BUDGET in columns per token or 0 = default, gradient dtype)
# (dW must take direct stores, i.e. no token split, for the combined launch.)
CASES = [("odd_tails", 256, "bf16"),       # four chunks: dH first / middle / last modes
         ("odd_tails", 0, "f32"),          # one chunk, fp32 outputs
         ("tiny", 0, "bf16"),              # K-split dH (four splits) and finalize
         ("mean_ignore", 0, "f32"),        # 10 % ignored tokens, mean reduction
         ("softcap_saturation", 0, "bf16")]  # capped logits, K-split dH


def _grads(t, wl):
    red = wl.reduction
    g = t["grad_logprob"]
    e = t["grad_entropy"]
    return g, e, red


def _backward(t, wl, out, gdt):
    g, e, red = _grads(t, wl)
    gh, gw = flce.backward(t["hidden"], t["weight"], t["labels"], out["lse"], out["entropy"], g, e,
                           ignore_index=wl.ignore_index, softcap=wl.softcap, reduction=red,
                           grad_dtype=gdt)
    torch.cuda.synchronize()
    return gh, gw


@pytest.mark.parametrize("name,cols,gdt", CASES, ids=[f"{c[0]}-{c[1]}-{c[2]}" for c in CASES])
def test_combined_launch_matches_separate(name, cols, gdt, monkeypatch):
    wl = W.WORKLOADS[name]
    x = W.make_inputs(wl)
    print(f"[dxdw] {name} N={wl.N} H={wl.H} V={wl.V} cols={cols} {gdt}", flush=True)
    t = G.upload(x)
    if cols:
        monkeypatch.setenv("FLCE_D_BUDGET", str(2 * max(wl.N, 1) * cols))
    out = flce.forward(t["hidden"], t["weight"], t["labels"], ignore_index=wl.ignore_index,
                       softcap=wl.softcap, reduction=wl.reduction)
    monkeypatch.setenv("FLCE_DXDW", "0")
    gh0, gw0 = _backward(t, wl, out, gdt)
    monkeypatch.setenv("FLCE_DXDW", "1")
    gh1, gw1 = _backward(t, wl, out, gdt)
    assert torch.equal(gh0, gh1), f"{name}: dH differs between combined and separate launches"
    assert torch.equal(gw0, gw1), f"{name}: dW differs between combined and separate launches"
    hf = W.bf16_bits_to_f32(x["hidden"])
    wf = W.bf16_bits_to_f32(x["weight"])
    dh, dw = oracle.backward(hf, wf, x["labels"], ignore_index=wl.ignore_index,
                             softcap_c=wl.softcap, reduction=wl.reduction,
                             grad_logprob=x["grad_logprob"], grad_entropy=x["grad_entropy"])
    assert G.rel_l2(gh1.float().cpu().numpy(), dh) <= G.GRAD_REL_L2
    assert G.rel_l2(gw1.float().cpu().numpy(), dw) <= G.GRAD_REL_L2
