"""GPU parity at the library's size limits, one at a time: the largest
vocabulary (V = 2^22 - 256; 2^21 for the fused call), the most tokens
(N = 2^21: 256 token chunks on the fused path) and the widest hidden size
(H = 2^20), through the recompute entry points the benchmark times and
through the fused forward + backward.

The upstream gradients are kept on a sample of 48 tokens (first and last
included) and set to zero elsewhere, so both gradients depend on the sampled
tokens alone: dHidden is zero on every other row, and dWeight is the sampled
tokens' contribution. The float64 oracle on the sampled tokens then gives
their statistics, their dHidden rows and all of dWeight. Tolerances as in the
other parity tests.
"""
import numpy as np
import pytest
import torch

import oracle
import gpu_helpers as G
from linear_cross_entropy_tile_amd import flce, workloads as W

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("path", ["recompute", "fused"])
@pytest.mark.parametrize("name", ["max_vocab", "max_tokens", "max_hidden"])
def test_size_limits(name, path):
    wl = W.WORKLOADS[name]
    if path == "fused" and wl.V > 1 << 21:
        wl = wl.with_(V=1 << 21)  # the fused call's vocabulary limit
    print(f"[limits] {name} {path} N={wl.N} H={wl.H} V={wl.V}", flush=True)
    x = W.make_inputs(wl)
    rows = W.sample_indices(wl.N, 48, wl.seed + 1)
    keep = np.zeros(wl.N, dtype=bool)
    keep[rows] = True
    for k in ("grad_logprob", "grad_entropy"):
        x[k] = np.where(keep, x[k], 0.0).astype(np.float32)
    t = G.upload(x)
    if path == "recompute":
        got = G.run(wl, t, keep_grads_on_gpu=True)
    else:
        out = flce.forward_backward(t["hidden"], t["weight"], t["labels"], t["grad_logprob"],
                                    t["grad_entropy"], ignore_index=wl.ignore_index,
                                    softcap=wl.softcap, reduction=wl.reduction)
        torch.cuda.synchronize()
        got = {k: out[k].cpu().numpy() for k in ("lse", "logprob", "entropy")}
        got["grad_hidden"], got["grad_weight"] = out["grad_hidden"], out["grad_weight"]
        got["invalid_labels"] = flce.flce_get_status(out["workspace"].data_ptr(),
                                                     torch.cuda.current_stream().cuda_stream)

    hs = W.bf16_bits_to_f32(x["hidden"][rows])
    wf = W.bf16_bits_to_f32(x["weight"])
    ys = x["labels"][rows]
    fw = oracle.forward(hs, wf, ys, ignore_index=wl.ignore_index, softcap_c=wl.softcap)
    dh, dw = oracle.backward(hs, wf, ys, ignore_index=wl.ignore_index, softcap_c=wl.softcap,
                             grad_logprob=x["grad_logprob"][rows],
                             grad_entropy=x["grad_entropy"][rows])
    for k in ("lse", "logprob", "entropy"):
        e = G.stat_err(got[k][rows], fw[k])
        assert e <= 1.0, f"{name} {k}: error {e:.3f} x tolerance"
    sel = torch.from_numpy(rows).to(G.dev())
    e = G.rel_l2(got["grad_hidden"].index_select(0, sel).float().cpu().numpy(), dh)
    assert e <= G.GRAD_REL_L2, f"{name} grad_hidden rows rel L2 {e:.2e}"
    other = torch.from_numpy(~keep).to(G.dev())
    assert torch.count_nonzero(got["grad_hidden"][other]).item() == 0
    e = G.rel_l2(got["grad_weight"].float().cpu().numpy(), dw)
    assert e <= G.GRAD_REL_L2, f"{name} grad_weight rel L2 {e:.2e}"
    assert got["invalid_labels"] == 0
