"""The seeded input generators: bf16 rounding, determinism, label structure."""
import math

import numpy as np
import torch

from linear_cross_entropy_tile_amd import workloads as W


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 3,
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 65504.0, 1e-30], np.float32)])
    bits = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bits, ref)
    back = W.bf16_bits_to_f32(bits)
    assert np.array_equal(back, torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_deterministic_and_shaped():
    wl = W.WORKLOADS["odd_tails"]
    a = W.make_inputs(wl)
    b = W.make_inputs(wl)
    for k in ("hidden", "weight", "labels", "grad_logprob", "grad_entropy"):
        assert np.array_equal(a[k], b[k])
    assert a["hidden"].shape == (77, 96) and a["weight"].shape == (96, 1000)
    assert a["hidden"].dtype == np.uint16 and a["labels"].dtype == np.int64
    assert (a["labels"] == -100).sum() == round(0.1 * 77)


def test_tiny_stats():
    wl = W.WORKLOADS["tiny"]
    x = W.make_inputs(wl)
    h = W.bf16_bits_to_f32(x["hidden"])
    w = W.bf16_bits_to_f32(x["weight"])
    assert abs(h.std() - 1.0) < 0.01
    assert abs(w.std() - 1 / math.sqrt(512)) < 0.001
    assert x["labels"].min() >= 0 and x["labels"].max() < 4096
    assert np.array_equal(x["grad_logprob"], np.ones(256, np.float32))


def test_mean_ignore_count():
    wl = W.WORKLOADS["mean_ignore"].with_(H=8, V=32000)   # cheap: labels only matter
    x = W.make_inputs(wl)
    assert (x["labels"] == -100).sum() == 410
    assert x["grad_logprob"].shape == (1,) and x["grad_entropy"][0] == np.float32(-0.01)


def test_zipf_labels_and_prompt_mask():
    wl = W.WORKLOADS["llama3_head"].with_(H=8, V=128256)
    x = W.make_inputs(wl)
    y = x["labels"]
    assert y.min() >= 0 and y.max() < 128256
    # rank-1 token frequency of a Zipf(1.1) over 128256 ranks is about 1/H_V(1.1)
    hv = (np.arange(1, 128257, dtype=np.float64) ** -1.1).sum()
    assert abs((y == 0).mean() - 1 / hv) < 0.02
    wl = W.WORKLOADS["rl_rollout"].with_(H=8, V=1000)
    y = W.make_inputs(wl)["labels"]
    m = (y == -100).reshape(16, 2048)
    assert m[:, :512].all() and not m[:, 512:].any()
    assert (y[y != -100] < 1000).all()


def test_sample_indices():
    s = W.sample_indices(1000, 16, 7)
    assert s[0] == 0 and s[-1] == 999 and len(set(s)) == len(s) == 16


def test_class_weights_recipe():
    a = W.make_class_weights(1000, 11, 0.05)
    b = W.make_class_weights(1000, 11, 0.05)
    assert a.dtype == np.float32 and a.shape == (1000,)
    assert np.array_equal(a, b)                      # seeded: same bits
    assert (a == 0).sum() == 50                      # round(0.05 * 1000) zeros
    nz = a[a != 0]
    assert nz.min() >= 0.2 and nz.max() < 3.0
    assert not np.array_equal(a, W.make_class_weights(1000, 12, 0.05))
