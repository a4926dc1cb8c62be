"""Re-entrancy across streams: the library keeps no device state between
calls, so two forward + backward calls enqueued on two streams (default
priority) with distinct workspaces and outputs give, bit for bit, what each
gives alone on the current stream."""
import pytest
import torch

import gpu_helpers as G
from linear_cross_entropy_tile_amd import flce, workloads as W

pytestmark = pytest.mark.gpu


def _run(t, wl, ws_f, ws_b):
    out = flce.forward(t["hidden"], t["weight"], t["labels"], ignore_index=wl.ignore_index,
                       softcap=wl.softcap, reduction=wl.reduction, workspace=ws_f)
    gh, gw = flce.backward(t["hidden"], t["weight"], t["labels"], out["lse"], out["entropy"],
                           t["grad_logprob"], t["grad_entropy"], ignore_index=wl.ignore_index,
                           softcap=wl.softcap, reduction=wl.reduction, workspace=ws_b)
    return [out["lse"], out["logprob"], out["entropy"], gh, gw]


def test_two_streams_match_alone():
    wls = [W.WORKLOADS["mean_ignore"], W.WORKLOADS["dw_split"]]
    ts = [G.upload(W.make_inputs(wl)) for wl in wls]
    ws = []
    for wl in wls:
        fb, bb = flce.workspace_bytes(wl.N, wl.H, wl.V, wl.reduction)
        ws.append((torch.empty(fb, dtype=torch.uint8, device=G.dev()),
                   torch.empty(bb, dtype=torch.uint8, device=G.dev())))
    alone = []
    for t, wl, (wf, wb) in zip(ts, wls, ws):
        alone.append([a.clone() for a in _run(t, wl, wf, wb)])
        torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    torch.cuda.synchronize()
    got = [None, None]
    for rep in range(3):
        for i, (t, wl, (wf, wb)) in enumerate(zip(ts, wls, ws)):
            with torch.cuda.stream(streams[i]):
                got[i] = _run(t, wl, wf, wb)
        torch.cuda.synchronize()
        for i in range(2):
            for a, b in zip(got[i], alone[i]):
                assert torch.equal(a, b), f"stream {i}, repetition {rep}: differs from the lone run"
