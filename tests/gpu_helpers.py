"""Shared helpers of the GPU tests: upload seeded inputs, run the library
through its C ABI (via the ctypes binding), and compare with the oracle."""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest
import torch

from linear_cross_entropy_tile_amd import flce, workloads as W

# Tolerances: per-token statistics within 2e-3 absolute or 1e-3 relative;
# gradients within 1e-2 relative L2 error.
STAT_ABS = 2e-3
STAT_REL = 1e-3
GRAD_REL_L2 = 1e-2


def dev():
    return torch.device("cuda:0")


def upload(x: dict) -> dict:
    d = dev()
    out = {
        "hidden": torch.from_numpy(x["hidden"].view(np.int16)).view(torch.bfloat16).to(d),
        "weight": torch.from_numpy(x["weight"].view(np.int16)).view(torch.bfloat16).to(d),
        "labels": torch.from_numpy(x["labels"]).to(d),
    }
    for k in ("grad_logprob", "grad_entropy"):
        out[k] = torch.from_numpy(x[k]).to(d) if x[k] is not None else None
    return out


def run(wl: W.Workload, t: dict, backward: bool = True, keep_grads_on_gpu: bool = False) -> dict:
    """Forward (+ backward) through the library; returns CPU numpy arrays
    (the gradients stay torch GPU tensors with keep_grads_on_gpu)."""
    out = flce.forward(t["hidden"], t["weight"], t["labels"], ignore_index=wl.ignore_index,
                       softcap=wl.softcap, reduction=wl.reduction)
    res = {}
    if backward:
        gh, gw = flce.backward(t["hidden"], t["weight"], t["labels"], out["lse"], out["entropy"],
                               t["grad_logprob"], t["grad_entropy"], ignore_index=wl.ignore_index,
                               softcap=wl.softcap, reduction=wl.reduction)
        torch.cuda.synchronize()
        if keep_grads_on_gpu:
            res["grad_hidden"], res["grad_weight"] = gh, gw
        else:
            res["grad_hidden"] = gh.float().cpu().numpy()
            res["grad_weight"] = gw.float().cpu().numpy()
    torch.cuda.synchronize()
    for k in ("lse", "logprob", "entropy", "logprob_mean", "entropy_mean"):
        if k in out:
            res[k] = out[k].cpu().numpy()
    res["invalid_labels"] = flce.flce_get_status(out["workspace"].data_ptr(),
                                                 torch.cuda.current_stream().cuda_stream)
    return res


def stat_err(got, want):
    """Largest violation ratio of |got - want| <= max(STAT_ABS, STAT_REL |want|)."""
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    tol = np.maximum(STAT_ABS, STAT_REL * np.abs(want))
    return float((np.abs(got - want) / tol).max()) if got.size else 0.0


def rel_l2(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    den = np.linalg.norm(want)
    num = np.linalg.norm(got - want)
    if den == 0.0:
        return float(num)
    return float(num / den)


# ---- full-size gradients through seeded projections ----------------------------

BLOCK = 256
ROW_TOL = 0.1


def _blockwise(got, want, axis, name):
    """Relative L2 error over everything, over each block of 256 along `axis`
    and for each single index along it."""
    e = rel_l2(got, want)
    assert e <= GRAD_REL_L2, f"{name}: rel L2 {e:.2e}"
    n = got.shape[axis]
    for b0 in range(0, n, BLOCK):
        sl = [slice(None)] * 2
        sl[axis] = slice(b0, min(n, b0 + BLOCK))
        e = rel_l2(got[tuple(sl)], want[tuple(sl)])
        assert e <= GRAD_REL_L2, f"{name}: block {b0 // BLOCK} rel L2 {e:.2e}"
    other = 1 - axis
    num = np.linalg.norm(got.astype(np.float64) - want, axis=other)
    den = np.linalg.norm(want.astype(np.float64), axis=other)
    bad = np.nonzero(num > ROW_TOL * np.maximum(den, 1e-30))[0]
    assert bad.size == 0, f"{name}: {bad.size} single rows/columns off, e.g. {bad[:5]}"


def check_projections(name, wl, gh, gw, ref, valid):
    """Every row of dHidden @ R_h and every column of R_w^T @ dWeight against
    the oracle's (R_h, R_w from the same seeds as the stored values)."""
    if "dhidden_proj" not in ref:
        pytest.skip(f"{name}: stored values carry no projections")
    sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden"))
    import make_golden
    rh, rw = make_golden.projections(wl)
    ph = (gh.float() @ torch.from_numpy(rh).to(dev())).cpu().numpy()
    pw = (torch.from_numpy(rw).to(dev()).t().contiguous() @ gw.float()).cpu().numpy()
    want_h = ref["dhidden_proj"].astype(np.float64)
    v = np.asarray(valid)
    assert np.all(want_h[~v] == 0.0) and np.all(ph[~v] == 0.0)
    # Rows of ignored tokens are exactly zero on both sides; the blocks and
    # single rows are taken over the valid tokens in order.
    _blockwise(ph[v], want_h[v], 0, f"{name} grad_hidden @ R_h")
    _blockwise(pw, ref["dweight_proj"].astype(np.float64), 1, f"{name} R_w^T @ grad_weight")
