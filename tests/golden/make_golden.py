"""Writes the stored expected values of the full-size parity tests.

For each full-size workload this runs the float64 CPU oracle (and nothing
else) on the seeded inputs and stores, in tests/golden/<workload>.npz:

  lse, logprob, entropy   [N]   every token's statistics
  logprob_mean, entropy_mean    (reduction "mean" only; class-weighted for
                                 the "_weighted" variant)
  rows, dhidden_rows      sampled rows of dHidden      [len(rows), H]
  cols, dweight_cols      sampled columns of dWeight   [H, len(cols)]

Stored as float32 (the tolerances are 1e-3 relative and looser). The oracle
materialises each block of 128 rows against the full vocabulary once and
derives the statistics, the sampled dHidden rows and the contribution to the
sampled dWeight columns from that block.

Run:  python tests/golden/make_golden.py [workload ...]
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle.flce_oracle as O  # noqa: E402
from linear_cross_entropy_tile_amd import workloads as W  # noqa: E402

FULL = ["llama3_head", "gemma2_softcap", "rl_rollout", "gemma2_softcap_weighted"]
# Variants: stored name -> (workload, seed of the class weights, fraction of
# zero class weights), drawn by workloads.make_class_weights.
WEIGHTED = {"gemma2_softcap_weighted": ("gemma2_softcap", 4242, 0.05)}
N_ROWS = 16
N_COLS = 16


def sample(wl):
    rows = W.sample_indices(wl.N, N_ROWS, wl.seed + 1000)
    cols = W.sample_indices(wl.V, N_COLS, wl.seed + 2000)
    return rows, cols


def class_weights(name: str):
    """The class weights of a stored variant (None for the plain workloads)."""
    if name not in WEIGHTED:
        return None
    base, seed, zf = WEIGHTED[name]
    return W.make_class_weights(W.WORKLOADS[base].V, seed, zf)


def golden(name: str, block: int = 128) -> str:
    wl = W.WORKLOADS[WEIGHTED[name][0] if name in WEIGHTED else name]
    cw = class_weights(name)
    t0 = time.time()
    x = W.make_inputs(wl)
    h = W.bf16_bits_to_f32(x["hidden"])
    w = W.bf16_bits_to_f32(x["weight"]).astype(np.float64)
    labels, valid = O._valid_mask(x["labels"], wl.V, wl.ignore_index)
    gb, eb = O._token_grads(labels, valid, wl.reduction, cw, x["grad_logprob"],
                            x["grad_entropy"])
    rows, cols = sample(wl)
    N, H = wl.N, wl.H
    lse = np.zeros(N)
    lp = np.zeros(N)
    ent = np.zeros(N)
    dh_rows = np.zeros((rows.size, H))
    dw_cols = np.zeros((H, cols.size))
    row_pos = {int(r): i for i, r in enumerate(rows)}
    for r0 in range(0, N, block):
        idx = np.arange(r0, min(N, r0 + block))
        idx = idx[valid[idx]]
        if idx.size == 0:
            continue
        zc = O.logits(h[idx], w, wl.softcap)
        l_, s_, e_, _ = O.row_stats(zc)
        lse[idx] = l_
        ent[idx] = e_
        lp[idx] = zc[np.arange(idx.size), labels[idx]] - l_
        dz = O.dlogits(zc, labels[idx], l_, s_, gb[idx], eb[idx], wl.softcap)
        dw_cols += h[idx].astype(np.float64).T @ dz[:, cols]
        for k, r in enumerate(idx):
            if int(r) in row_pos:
                dh_rows[row_pos[int(r)]] = dz[k] @ w.T
        if (r0 // block) % 16 == 0:
            print(f"  {name}: rows {r0}/{N}  {time.time() - t0:.0f}s", flush=True)
    out = {"lse": lse.astype(np.float32), "logprob": lp.astype(np.float32),
           "entropy": ent.astype(np.float32), "rows": rows, "cols": cols,
           "dhidden_rows": dh_rows.astype(np.float32), "dweight_cols": dw_cols.astype(np.float32)}
    if wl.reduction == "mean":
        om = O._token_weights(labels, valid, wl.reduction, cw)[valid]
        ws = om.sum()
        out["logprob_mean"] = np.array([(om * lp[valid]).sum() / ws if ws else 0.0])
        out["entropy_mean"] = np.array([(om * ent[valid]).sum() / ws if ws else 0.0])
    path = os.path.join(HERE, f"{name}.npz")
    np.savez_compressed(path, **out)
    print(f"wrote {path} in {time.time() - t0:.0f}s", flush=True)
    return path


if __name__ == "__main__":
    for nm in (sys.argv[1:] or FULL):
        golden(nm)
