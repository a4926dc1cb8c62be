"""The library enqueues kernels only (no memset, copy, allocation or
synchronisation), so a forward + backward can be captured into a HIP graph.
The captured graph is replayed several times, with unrelated eager work and
synchronisations in between, and every replay must reproduce the eager
results bit for bit (the kernels are deterministic)."""
import numpy as np
import pytest
import torch

import gpu_helpers as G
from linear_cross_entropy_tile_amd import flce, workloads as W

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["odd_tails", "mean_ignore"])
def test_graph_capture_replays(name):
    wl = W.WORKLOADS[name]
    x = W.make_inputs(wl)
    t = G.upload(x)
    dev = G.dev()
    N, H = t["hidden"].shape
    V = t["weight"].shape[1]
    red = flce._REDUCTIONS[wl.reduction]
    fb, bb = flce.flce_workspace_size(N, H, V, red)
    wsf = torch.empty(fb, dtype=torch.uint8, device=dev)
    wsb = torch.empty(bb, dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    lse, lp, ent = (torch.empty(N, **f32) for _ in range(3))
    lpm, entm = torch.empty(1, **f32), torch.empty(1, **f32)
    gh = torch.empty((N, H), dtype=torch.bfloat16, device=dev)
    gw = torch.empty((H, V), dtype=torch.bfloat16, device=dev)
    g, e = t["grad_logprob"], t["grad_entropy"]

    def step():
        s = torch.cuda.current_stream().cuda_stream
        flce.flce_forward(t["hidden"].data_ptr(), t["weight"].data_ptr(), t["labels"].data_ptr(),
                          N, H, V, wl.ignore_index, wl.softcap, red, lse.data_ptr(), lp.data_ptr(),
                          ent.data_ptr(), lpm.data_ptr(), entm.data_ptr(), wsf.data_ptr(), fb, s)
        flce.flce_backward(t["hidden"].data_ptr(), t["weight"].data_ptr(), t["labels"].data_ptr(),
                           N, H, V, wl.ignore_index, wl.softcap, red, lse.data_ptr(),
                           ent.data_ptr(), g.data_ptr(), e.data_ptr(), gh.data_ptr(),
                           gw.data_ptr(), wsb.data_ptr(), bb, s)

    step()
    torch.cuda.synchronize()
    ref = [a.clone() for a in (lse, lp, ent, lpm, entm, gh, gw)]
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    scratch = torch.randn(1 << 20, device=dev)
    for rep in range(4):
        for a in (lse, lp, ent, gh, gw):
            a.zero_()
        scratch.mul_(1.0001)  # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip((lse, lp, ent, lpm, entm, gh, gw), ref):
            assert torch.equal(got, want), f"{name}: replay {rep} differs from the eager result"


def test_graph_capture_fused():
    """The fused forward + backward (several token chunks, fp32 dW
    accumulation) captured and replayed the same way."""
    wl = W.WORKLOADS["mean_ignore"]
    x = W.make_inputs(wl)
    t = G.upload(x)
    dev = G.dev()
    N, H = t["hidden"].shape
    V = t["weight"].shape[1]
    opt = flce.FlceOptions(wl.ignore_index, wl.softcap, flce.FLCE_REDUCTION_MEAN, 0.01,
                           flce.FLCE_GRAD_BF16)
    chunk = 1024
    nbytes = flce.flce_fused_workspace_size(N, H, V, opt, chunk)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    lse, lp, ent = (torch.empty(N, **f32) for _ in range(3))
    red = torch.empty(4, **f32)
    gh = torch.empty((N, H), dtype=torch.bfloat16, device=dev)
    gw = torch.empty((H, V), dtype=torch.bfloat16, device=dev)
    g, e = t["grad_logprob"], t["grad_entropy"]

    def step():
        s = torch.cuda.current_stream().cuda_stream
        flce.flce_forward_backward(t["hidden"].data_ptr(), t["weight"].data_ptr(),
                                   t["labels"].data_ptr(), N, H, V, opt, chunk, g.data_ptr(),
                                   e.data_ptr(), None, None, lse.data_ptr(), lp.data_ptr(),
                                   ent.data_ptr(), None, None, red.data_ptr(), gh.data_ptr(),
                                   gw.data_ptr(), ws.data_ptr(), nbytes, s)

    step()
    torch.cuda.synchronize()
    outs = (lse, lp, ent, red, gh, gw)
    ref = [a.clone() for a in outs]
    step()  # a second eager run is bit for bit the first
    torch.cuda.synchronize()
    for got, want in zip(outs, ref):
        assert torch.equal(got, want), "fused: two eager runs differ"
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    scratch = torch.randn(1 << 20, device=dev)
    for rep in range(4):
        for a in outs:
            a.zero_()
        scratch.mul_(1.0001)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip(outs, ref):
            assert torch.equal(got, want), f"fused: replay {rep} differs from the eager result"
