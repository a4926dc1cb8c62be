"""Seeded synthetic workloads for the fused linear cross-entropy head.

This module only draws inputs: shapes, seeds, value distributions, label
structure and upstream gradients. It holds none of the head's arithmetic, so
the GPU path (tests, benchmark) and the CPU oracle can both draw identical
inputs from it without sharing any computation.

Hidden states and weights are drawn in float32 and rounded to bfloat16 with
round-to-nearest-even; the exact bf16 bit patterns are what every consumer
sees. The random streams come from numpy's PCG64 seeded through a
SeedSequence, so the same workload gives the same bits on every machine with
this numpy.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
import math

import numpy as np

__all__ = ["Workload", "WORKLOADS", "make_inputs", "f32_to_bf16_bits",
           "bf16_bits_to_f32", "sample_indices", "make_class_weights", "projection_matrix"]


@dataclass(frozen=True)
class Workload:
    """One synthetic input recipe.

    grad_logprob / grad_entropy: ("ones",) one per token, ("normal",) N(0,1)
    per token, ("scalar", v) one scalar (mean reduction), ("broadcast", v) the
    value v repeated per token, ("none",) no gradient.
    """
    name: str
    N: int
    H: int
    V: int
    seed: int
    hidden_std: float = 1.0
    weight_std: float = 0.02
    labels: str = "uniform"          # "uniform" | "zipf"
    zipf_s: float = 1.1
    ignore: str = "none"             # "none" | "fraction" | "prompt" | "all"
    ignore_fraction: float = 0.0
    seq_len: int = 0
    prompt_len: int = 0
    ignore_index: int = -100
    softcap: float = 0.0
    reduction: str = "none"
    grad_logprob: tuple = ("ones",)
    grad_entropy: tuple = ("ones",)
    weight_zero: bool = False

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # Tiny CPU-checkable case.
    "tiny": Workload("tiny", 256, 512, 4096, seed=101,
                     weight_std=1.0 / math.sqrt(512.0)),
    # Mid-size head with 10% ignored tokens and mean reduction.
    "mean_ignore": Workload("mean_ignore", 4096, 4096, 32000, seed=102,
                            ignore="fraction", ignore_fraction=0.1,
                            reduction="mean", grad_logprob=("scalar", 1.0),
                            grad_entropy=("scalar", -0.01)),
    # Llama-3-shaped head, Zipf labels, per-token gradients.
    "llama3_head": Workload("llama3_head", 8192, 4096, 128256, seed=103,
                            labels="zipf", zipf_s=1.1,
                            grad_logprob=("normal",), grad_entropy=("normal",)),
    # Gemma2-shaped head with a tanh cap of 30 and mean reduction.
    "gemma2_softcap": Workload("gemma2_softcap", 8192, 2304, 256000, seed=104,
                               weight_std=0.05, softcap=30.0, reduction="mean",
                               grad_logprob=("scalar", 1.0),
                               grad_entropy=("scalar", 1.0)),
    # Long RL rollout batch: 16 sequences of 2048, first 512 of each ignored.
    "rl_rollout": Workload("rl_rollout", 32768, 5120, 152064, seed=105,
                           ignore="prompt", seq_len=2048, prompt_len=512,
                           grad_logprob=("normal",),
                           grad_entropy=("broadcast", -0.001)),
    # Extra parity cases.
    "odd_tails": Workload("odd_tails", 77, 96, 1000, seed=201, weight_std=0.1,
                          ignore="fraction", ignore_fraction=0.1,
                          grad_logprob=("normal",), grad_entropy=("normal",)),
    "softcap_saturation": Workload("softcap_saturation", 512, 2304, 256000,
                                   seed=202, weight_std=0.5, softcap=30.0,
                                   grad_logprob=("normal",),
                                   grad_entropy=("normal",)),
    "all_ignored": Workload("all_ignored", 300, 256, 2048, seed=203,
                            ignore="all", reduction="mean",
                            grad_logprob=("scalar", 1.0),
                            grad_entropy=("scalar", 1.0)),
    "zero_weight": Workload("zero_weight", 200, 256, 3000, seed=204,
                            weight_zero=True, grad_logprob=("normal",),
                            grad_entropy=("normal",)),
    # Few output tiles of dW and many tokens: the token reduction is split.
    "dw_split": Workload("dw_split", 4096, 256, 2048, seed=205, weight_std=0.1,
                         ignore="fraction", ignore_fraction=0.05,
                         grad_logprob=("normal",), grad_entropy=("normal",)),
    # Vocabularies that are not a multiple of 8 (odd; 2 mod 8 with a split dW).
    "odd_vocab": Workload("odd_vocab", 300, 128, 1001, seed=209, weight_std=0.1,
                          ignore="fraction", ignore_fraction=0.1,
                          grad_logprob=("normal",), grad_entropy=("normal",)),
    # Capped logits (std about 1.1 c) with a ragged last tile in every direction.
    "odd_capped": Workload("odd_capped", 300, 192, 1001, seed=211, weight_std=0.4,
                           softcap=5.0, ignore="fraction", ignore_fraction=0.1,
                           grad_logprob=("normal",), grad_entropy=("normal",)),
    "odd_vocab_dw_split": Workload("odd_vocab_dw_split", 2048, 64, 1002, seed=210,
                                   weight_std=0.15, ignore="fraction", ignore_fraction=0.05,
                                   grad_logprob=("normal",), grad_entropy=("normal",)),
    # The library's size limits, one extreme at a time (weight std 1/sqrt(H)
    # keeps the logits of order 1).
    "max_vocab": Workload("max_vocab", 64, 64, (1 << 22) - 256, seed=206, weight_std=0.125,
                          ignore="fraction", ignore_fraction=0.1,
                          grad_logprob=("normal",), grad_entropy=("normal",)),
    "max_tokens": Workload("max_tokens", 1 << 21, 64, 512, seed=207, weight_std=0.125,
                           ignore="fraction", ignore_fraction=0.1,
                           grad_logprob=("normal",), grad_entropy=("normal",)),
    "max_hidden": Workload("max_hidden", 256, 1 << 20, 256, seed=208, weight_std=1.0 / 1024,
                           grad_logprob=("normal",), grad_entropy=("normal",)),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits.

    Inputs here are finite normal draws, so the NaN case is not handled.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact float32 values of bfloat16 bit patterns."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _streams(seed: int):
    ss = np.random.SeedSequence(seed)
    return [np.random.Generator(np.random.PCG64(s)) for s in ss.spawn(5)]


def _normal_bf16(rng, shape, std, chunk_rows=512):
    rows, cols = shape
    out = np.empty(shape, dtype=np.uint16)
    s = np.float32(std)
    for r0 in range(0, rows, chunk_rows):
        r1 = min(rows, r0 + chunk_rows)
        x = rng.standard_normal((r1 - r0, cols), dtype=np.float32)
        x *= s
        out[r0:r1] = f32_to_bf16_bits(x)
    return out


def _labels(wl: Workload, rng_lab, rng_ign):
    N, V = wl.N, wl.V
    if wl.labels == "uniform":
        labels = rng_lab.integers(0, V, size=N, dtype=np.int64)
    elif wl.labels == "zipf":
        # Truncated Zipf over ranks 1..V, explicit normalised pmf, inverse-CDF
        # sampling; token id = rank - 1.
        ranks = np.arange(1, V + 1, dtype=np.float64)
        pmf = ranks ** (-wl.zipf_s)
        cdf = np.cumsum(pmf)
        cdf /= cdf[-1]
        u = rng_lab.random(N)
        labels = np.minimum(np.searchsorted(cdf, u, side="right"), V - 1).astype(np.int64)
    else:
        raise ValueError(wl.labels)
    if wl.ignore == "fraction":
        k = int(round(wl.ignore_fraction * N))
        idx = rng_ign.permutation(N)[:k]
        labels[idx] = wl.ignore_index
    elif wl.ignore == "prompt":
        for s0 in range(0, N, wl.seq_len):
            labels[s0:s0 + wl.prompt_len] = wl.ignore_index
    elif wl.ignore == "all":
        labels[:] = wl.ignore_index
    elif wl.ignore != "none":
        raise ValueError(wl.ignore)
    return labels


def _grad(spec, N, rng):
    kind = spec[0]
    if kind == "ones":
        return np.ones(N, dtype=np.float32)
    if kind == "normal":
        return rng.standard_normal(N, dtype=np.float32)
    if kind == "scalar":
        return np.array([spec[1]], dtype=np.float32)
    if kind == "broadcast":
        return np.full(N, spec[1], dtype=np.float32)
    if kind == "none":
        return None
    raise ValueError(spec)


def make_inputs(wl: Workload) -> dict:
    """Draw the workload's inputs.

    Returns hidden/weight as bf16 bit patterns (uint16, row-major [N,H] and
    [H,V]), labels int64 [N], and the upstream gradients as float32 ([N] under
    "none", [1] under "mean", or None).
    """
    r_hid, r_wt, r_lab, r_ign, r_grad = _streams(wl.seed)
    hidden = _normal_bf16(r_hid, (wl.N, wl.H), wl.hidden_std)
    if wl.weight_zero:
        weight = np.zeros((wl.H, wl.V), dtype=np.uint16)
    else:
        weight = _normal_bf16(r_wt, (wl.H, wl.V), wl.weight_std)
    labels = _labels(wl, r_lab, r_ign)
    g_lp = _grad(wl.grad_logprob, wl.N, r_grad)
    g_ent = _grad(wl.grad_entropy, wl.N, r_grad)
    return {"hidden": hidden, "weight": weight, "labels": labels,
            "grad_logprob": g_lp, "grad_entropy": g_ent}


def sample_indices(n: int, k: int, seed: int) -> np.ndarray:
    """k sorted distinct indices in [0, n), always including the first and
    the last (tails), drawn from their own seeded stream."""
    k = min(k, n)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    pick = set([0, n - 1])
    extra = rng.choice(n, size=k, replace=False)
    for e in extra:
        if len(pick) >= k:
            break
        pick.add(int(e))
    return np.array(sorted(pick), dtype=np.int64)


def make_class_weights(V: int, seed: int, zero_fraction: float = 0.0) -> np.ndarray:
    """Seeded per-class target weights, float32 [V]: uniform in [0.2, 3.0),
    with round(zero_fraction * V) classes (a seeded choice) set to 0."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    cw = rng.uniform(0.2, 3.0, size=V).astype(np.float32)
    k = int(round(zero_fraction * V))
    if k:
        cw[rng.permutation(V)[:k]] = 0.0
    return cw


def projection_matrix(dim: int, k: int, seed: int) -> np.ndarray:
    """Seeded float32 [dim, k] with independent N(0, 1) entries: the random
    directions onto which gradients are projected to compare every row and
    column of them at full size."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    return rng.standard_normal((dim, k)).astype(np.float32)
