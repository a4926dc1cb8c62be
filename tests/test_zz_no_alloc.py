"""flce_forward_noalloc, the forward that runs in the library's static
per-device scratch instead of a caller workspace, against flce_forward on the
same inputs through the C ABI: two calls in a row, the second on a smaller
input (the scratch keeps the first call's bytes), each bit for bit equal to
the workspace path; a shape beyond the scratch is refused without touching
the outputs."""
import numpy as np
import pytest
import torch

import gpu_helpers as G
from linear_cross_entropy_tile_amd import flce, workloads as W

pytestmark = pytest.mark.gpu


def _call(fn, t, wl, extra):
    d = G.dev()
    N = wl.N
    f32 = dict(dtype=torch.float32, device=d)
    out = {k: torch.full((N,), float("nan"), **f32) for k in ("lse", "logprob", "entropy")}
    red = flce._REDUCTIONS[wl.reduction]
    lpm = torch.full((1,), float("nan"), **f32)
    entm = torch.full((1,), float("nan"), **f32)
    st = torch.cuda.current_stream().cuda_stream
    fn(t["hidden"].data_ptr(), t["weight"].data_ptr(), t["labels"].data_ptr(), N, wl.H, wl.V,
       wl.ignore_index, wl.softcap, red, out["lse"].data_ptr(), out["logprob"].data_ptr(),
       out["entropy"].data_ptr(), lpm.data_ptr() if red else None,
       entm.data_ptr() if red else None, *extra, st)
    torch.cuda.synchronize()
    res = {k: v.cpu().numpy() for k, v in out.items()}
    if red:
        res["logprob_mean"] = lpm.cpu().numpy()
        res["entropy_mean"] = entm.cpu().numpy()
    return res


def _workspace_path(t, wl):
    red = flce._REDUCTIONS[wl.reduction]
    fbytes, _ = flce.flce_workspace_size(wl.N, wl.H, wl.V, red)
    ws = torch.empty(fbytes, dtype=torch.uint8, device=G.dev())
    return _call(flce.flce_forward, t, wl, (ws.data_ptr(), fbytes))


def _noalloc_path(t, wl):
    return _call(flce.flce_forward_noalloc, t, wl, ())


def test_noalloc_matches_workspace_forward_twice():
    # First call: mean over the valid tokens of a head whose forward workspace
    # fills about half the scratch; second call: a smaller capped head with
    # reduction none, run right after in the same scratch.
    big = W.WORKLOADS["mean_ignore"].with_(N=2048, H=2048, V=32000)
    small = W.WORKLOADS["odd_tails"].with_(softcap=5.0)
    for wl in (big, small):
        fbytes, _ = flce.flce_workspace_size(wl.N, wl.H, wl.V, flce._REDUCTIONS[wl.reduction])
        assert fbytes <= flce.FLCE_NOALLOC_SCRATCH_BYTES
        print(f"[noalloc] {wl.name} N={wl.N} H={wl.H} V={wl.V} forward workspace {fbytes}",
              flush=True)
        t = G.upload(W.make_inputs(wl))
        got = _noalloc_path(t, wl)
        want = _workspace_path(t, wl)
        assert set(got) == set(want)
        for k in want:
            assert np.array_equal(got[k], want[k]), (wl.name, k)
            assert np.all(np.isfinite(got[k])), (wl.name, k)


def test_noalloc_refuses_oversize_untouched():
    wl = W.WORKLOADS["odd_tails"].with_(N=4096, H=4096, V=32000 + 1)
    fbytes, _ = flce.flce_workspace_size(wl.N, wl.H, wl.V, 0)
    assert fbytes > flce.FLCE_NOALLOC_SCRATCH_BYTES
    d = G.dev()
    f32 = dict(dtype=torch.float32, device=d)
    lse = torch.full((wl.N,), 7.0, **f32)
    h = torch.zeros((wl.N, wl.H), dtype=torch.bfloat16, device=d)
    w = torch.zeros((wl.H, wl.V), dtype=torch.bfloat16, device=d)
    y = torch.zeros(wl.N, dtype=torch.int64, device=d)
    st = torch.cuda.current_stream().cuda_stream
    code = flce.lib().flce_forward_noalloc(h.data_ptr(), w.data_ptr(), y.data_ptr(), wl.N, wl.H,
                                           wl.V, -100, 0.0, 0, lse.data_ptr(), lse.data_ptr(),
                                           lse.data_ptr(), None, None, st)
    torch.cuda.synchronize()
    assert code == 10
    assert torch.all(lse == 7.0).item()
