"""The script that writes the stored full-size expected values
(tests/golden/make_golden.py) assembles them from oracle.forward and
oracle.backward; here, on small workloads, every array it would store is
checked against the oracle's other pinned entry points: the per-token
statistics and means against oracle.forward, the sampled dHidden rows and
dWeight columns against oracle.dhidden_rows / oracle.dweight_columns, and the
projections against those functions over all rows and columns times the same
seeded matrices."""
import os
import sys

import numpy as np
import pytest

import oracle
from linear_cross_entropy_tile_amd import workloads as W

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden"))
import make_golden as M  # noqa: E402


@pytest.mark.parametrize("name,cw", [("odd_tails", None), ("all_ignored", None),
                                     ("mean_small", None), ("mean_small", "weights")])
def test_golden_assembly(name, cw):
    if name == "mean_small":
        wl = W.WORKLOADS["mean_ignore"].with_(N=300, H=64, V=700, softcap=4.0)
    else:
        wl = W.WORKLOADS[name]
    x = W.make_inputs(wl)
    weights = W.make_class_weights(wl.V, 77, 0.1) if cw else None
    got = M.expected(wl, x, weights)
    h = W.bf16_bits_to_f32(x["hidden"])
    w = W.bf16_bits_to_f32(x["weight"])
    kw = dict(ignore_index=wl.ignore_index, softcap_c=wl.softcap, reduction=wl.reduction,
              grad_logprob=x["grad_logprob"], grad_entropy=x["grad_entropy"],
              class_weight=weights)
    fw = oracle.forward(h, w, x["labels"], ignore_index=wl.ignore_index, softcap_c=wl.softcap,
                        reduction=wl.reduction, class_weight=weights)
    for k in ("lse", "logprob", "entropy"):
        np.testing.assert_allclose(got[k], fw[k], rtol=1e-6, atol=1e-6)
    if wl.reduction == "mean":
        for k in ("logprob_mean", "entropy_mean"):
            np.testing.assert_allclose(got[k][0], fw[k], rtol=1e-9, atol=1e-12)
    rows, cols = M.sample(wl)
    assert np.array_equal(got["rows"], rows) and np.array_equal(got["cols"], cols)
    dh_s = oracle.dhidden_rows(h, w, x["labels"], rows, **kw)
    dw_s = oracle.dweight_columns(h, w, x["labels"], cols, **kw)
    np.testing.assert_allclose(got["dhidden_rows"], dh_s, rtol=1e-5, atol=1e-9)
    np.testing.assert_allclose(got["dweight_cols"], dw_s, rtol=1e-5, atol=1e-9)
    rh, rw = M.projections(wl)
    dh_all = oracle.dhidden_rows(h, w, x["labels"], np.arange(wl.N), **kw)
    dw_all = oracle.dweight_columns(h, w, x["labels"], np.arange(wl.V), **kw)
    scale_h = max(np.abs(dh_all @ rh).max(), 1e-30)
    scale_w = max(np.abs(rw.T @ dw_all).max(), 1e-30)
    np.testing.assert_allclose(got["dhidden_proj"], dh_all @ rh, rtol=1e-5, atol=1e-6 * scale_h)
    np.testing.assert_allclose(got["dweight_proj"], rw.T @ dw_all, rtol=1e-5,
                               atol=1e-6 * scale_w)


def test_projection_matrix_seeded():
    a = W.projection_matrix(64, 8, 5)
    assert a.shape == (64, 8) and a.dtype == np.float32
    assert np.array_equal(a, W.projection_matrix(64, 8, 5))
    assert not np.array_equal(a, W.projection_matrix(64, 8, 6))
    assert abs(float(a.mean())) < 0.2 and 0.8 < float(a.std()) < 1.2
