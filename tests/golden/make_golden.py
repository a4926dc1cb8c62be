"""Writes the stored expected values of the full-size parity tests.

For each full-size workload this runs the float64 CPU oracle (and nothing
else: oracle.forward and oracle.backward, whose results the oracle pins fix)
on the seeded inputs and stores, in tests/golden/<workload>.npz:

  lse, logprob, entropy   [N]   every token's statistics
  logprob_mean, entropy_mean    (reduction "mean" only; class-weighted for
                                 the "_weighted" variant)
  rows, dhidden_rows      sampled rows of dHidden      [len(rows), H]
  cols, dweight_cols      sampled columns of dWeight   [H, len(cols)]
  dhidden_proj            dHidden @ R_h                [N, K_PROJ]
  dweight_proj            R_w^T @ dWeight              [K_PROJ, V]

R_h and R_w are seeded Gaussian [H, K_PROJ] matrices (workloads.
projection_matrix with the seeds of ``projection_seeds``): the projections
carry every row of dHidden and every column of dWeight, so the GPU test checks
all of them, not a sample. The "_weighted" variant stores the sampled rows and
columns only (its contractions are those of the plain workload).

Stored as float32 (the tolerances are 1e-3 relative and looser). The full
float64 dWeight is held in memory: up to 6.2 GB for the RL-rollout head.

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
K_PROJ = 8


def sample(wl):
    rows = W.sample_indices(wl.N, N_ROWS, wl.seed + 1000)
    cols = W.sample_indices(wl.V, N_COLS, wl.seed + 2000)
    return rows, cols


def projection_seeds(wl):
    """Seeds of R_h and R_w for a workload."""
    return wl.seed + 3000, wl.seed + 4000


def projections(wl):
    sh, sw = projection_seeds(wl)
    return W.projection_matrix(wl.H, K_PROJ, sh), W.projection_matrix(wl.H, K_PROJ, sw)


def class_weights(name: str):
    """The class weights of a stored variant (None for the plain workloads)."""
    if name not in WEIGHTED:
        return None
    base, seed, zf = WEIGHTED[name]
    return W.make_class_weights(W.WORKLOADS[base].V, seed, zf)


def expected(wl, x, cw=None, project=True) -> dict:
    """The stored arrays for workload `wl` on inputs `x`, from oracle.forward
    and oracle.backward."""
    h = W.bf16_bits_to_f32(x["hidden"])
    w = W.bf16_bits_to_f32(x["weight"])
    fw = O.forward(h, w, x["labels"], ignore_index=wl.ignore_index, softcap_c=wl.softcap,
                   reduction=wl.reduction, class_weight=cw)
    dh, dw = O.backward(h, w, x["labels"], ignore_index=wl.ignore_index, softcap_c=wl.softcap,
                        reduction=wl.reduction, grad_logprob=x["grad_logprob"],
                        grad_entropy=x["grad_entropy"], class_weight=cw)
    rows, cols = sample(wl)
    out = {"lse": fw["lse"].astype(np.float32), "logprob": fw["logprob"].astype(np.float32),
           "entropy": fw["entropy"].astype(np.float32), "rows": rows, "cols": cols,
           "dhidden_rows": dh[rows].astype(np.float32),
           "dweight_cols": dw[:, cols].astype(np.float32)}
    if wl.reduction == "mean":
        out["logprob_mean"] = np.array([fw["logprob_mean"]])
        out["entropy_mean"] = np.array([fw["entropy_mean"]])
    if project:
        rh, rw = projections(wl)
        out["dhidden_proj"] = (dh @ rh.astype(np.float64)).astype(np.float32)
        out["dweight_proj"] = (rw.astype(np.float64).T @ dw).astype(np.float32)
    return out


def golden(name: str) -> str:
    wl = W.WORKLOADS[WEIGHTED[name][0] if name in WEIGHTED else name]
    t0 = time.time()
    print(f"  {name}: N={wl.N} H={wl.H} V={wl.V}", flush=True)
    out = expected(wl, W.make_inputs(wl), class_weights(name), project=name not in WEIGHTED)
    path = os.path.join(HERE, f"{name}.npz")
    np.savez_compressed(path, **out)
    print(f"wrote {path} in {time.time() - t0:.0f}s", flush=True)
    return path


if __name__ == "__main__":
    for nm in (sys.argv[1:] or FULL):
        golden(nm)
