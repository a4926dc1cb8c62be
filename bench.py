"""Benchmark of the fused linear cross-entropy + entropy head on one MI355X.

One step = flce_forward + flce_backward over one batch (the whole hot path:
logit tiles with the online softmax/entropy epilogue, the tile combine, the
logit-gradient recompute, dHidden and dWeight contractions). Inputs are
seeded synthetic data resident in HBM before the timed region. The default
workload is the Llama-3-shaped head (N=8192 tokens, H=4096, V=128256, Zipf
labels, reduction none, per-token upstream gradients).

Prints one JSON line. Besides the throughput it reports:
  roofline      the dominant kernel's algorithmic TFLOP/s (flops per launch /
                mean launch time from HIP events recorded by the library on its
                launch stream during the timed region) against the bf16 dense
                MFMA peak;
  kernels       the same figures for every kernel kind;
  cpu_baseline  the float64 CPU oracle timed on a bounded token sample;
  memory        peak device memory of the fused step vs the fp32 logits that a
                materialising implementation needs;
  torch_ref     (optional) a materialising torch implementation of the same
                forward + backward on the same GPU, for context.

roofline.traffic is the dominant kernel's HBM bytes per launch as measured
by rocprofv3 counters (FETCH_SIZE and WRITE_SIZE, each scaled by what it reads
for a plain device copy of known size in the same run), taken from
profiles/traffic_<workload>.txt; it is null when that file is missing or was
taken on kernel sources other than the ones built now (a SHA-256 over the
library's sources is stored with the counters). --copy-calibration-mib runs
that plain copy once before warmup, for the counter runs.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CUs x 4096 flop/clk x 2.4 GHz, dense
METRIC = "fwd+bwd tokens/s and % bf16 MFMA peak, N=8192 H=4096 V=128256, 1 GPU"

# Algorithmic flops per valid token of each kernel kind, in units of H*V.
FLOPS_PER_TOKEN_HV = {"fwd_tile": 2, "bwd_dlogits": 2, "bwd_dx": 2, "bwd_dw": 2}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama3_head")
    ap.add_argument("--cpu-tokens", type=int, default=2048,
                    help="tokens of the CPU oracle sample (0 skips the CPU baseline)")
    ap.add_argument("--torch-ref", type=int, default=1,
                    help="also time a materialising torch fwd+bwd (0/1)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB before warmup "
                         "(the reference point of the HBM byte counters)")
    return ap.parse_args()


def kernel_source_hash() -> str:
    """SHA-256 over the library's kernel and boundary sources, in a fixed order."""
    files = sorted(glob.glob(os.path.join(ROOT, "linear_cross_entropy_tile_amd", "csrc", "*")))
    files.append(os.path.join(ROOT, "include", "flce.h"))
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def counted_traffic(workload: str):
    """Per-kernel HBM bytes per launch from profiles/traffic_<workload>.txt, or
    None when absent or taken on other sources. Lines of that file:
      source_sha256 <hex>
      kernel <kind> fetch_bytes <B> write_bytes <B>"""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    sha, per = None, {}
    with open(path) as fh:
        for line in fh:
            f = line.split()
            if len(f) >= 2 and f[0] == "source_sha256":
                sha = f[1]
            elif len(f) >= 6 and f[0] == "kernel" and f[2] == "fetch_bytes" and f[4] == "write_bytes":
                per[f[1]] = float(f[3]) + float(f[5])
    if sha != kernel_source_hash():
        return None
    return per


def cpu_baseline(wl, x, ntok):
    """The float64 oracle, as it stands, on the first `ntok` tokens: forward
    statistics plus those tokens' dHidden rows and dWeight contribution."""
    import oracle
    from linear_cross_entropy_tile_amd import workloads as W
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    n = min(ntok, wl.N)
    h = W.bf16_bits_to_f32(x["hidden"][:n])
    w = W.bf16_bits_to_f32(x["weight"])
    y = x["labels"][:n]
    red = wl.reduction
    g = x["grad_logprob"][:n] if red == "none" else x["grad_logprob"]
    e = x["grad_entropy"][:n] if red == "none" else x["grad_entropy"]
    t0 = time.perf_counter()
    oracle.forward(h, w, y, ignore_index=wl.ignore_index, softcap_c=wl.softcap, reduction=red)
    oracle.backward(h, w, y, ignore_index=wl.ignore_index, softcap_c=wl.softcap, reduction=red,
                    grad_logprob=g, grad_entropy=e)
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {n} of {wl.N} tokens of {wl.name}: float64 oracle forward + "
                      f"backward (their dHidden rows and dWeight contribution), {dt:.1f} s",
            "seconds": dt, "cpu": platform.processor() or platform.machine()}


def torch_reference(t, wl, iters=2):
    """Materialising fwd+bwd in torch (fp32 logits as in the pages' reference
    compute logic), for a context time and peak memory."""
    import torch
    import torch.nn.functional as F
    h = t["hidden"]
    w = t["weight"]
    y = t["labels"]
    g = t["grad_logprob"]
    e = t["grad_entropy"]

    def step():
        hh = h.detach().float().requires_grad_(True)
        ww = w.detach().float().requires_grad_(True)
        z = hh @ ww
        if wl.softcap > 0:
            z = wl.softcap * torch.tanh(z / wl.softcap)
        lse = torch.logsumexp(z, dim=-1)
        p = torch.softmax(z, dim=-1)
        ent = lse - (p * z).sum(-1)
        lp = -F.cross_entropy(z, y, ignore_index=wl.ignore_index, reduction="none")
        valid = (y != wl.ignore_index).float()
        loss = (g * lp).sum() + (e * ent * valid).sum()
        loss.backward()
        return hh.grad, ww.grad

    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    step()
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - base
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(iters):
        step()
    b.record()
    torch.cuda.synchronize()
    return {"ms_per_step": a.elapsed_time(b) / iters, "peak_bytes_above_inputs": int(peak),
            "what": "torch eager, fp32 logits materialised, autograd backward"}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path "
              "(use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    from linear_cross_entropy_tile_amd import flce, workloads as W

    wl = W.WORKLOADS[args.workload]
    x = W.make_inputs(wl)
    dev = torch.device("cuda:0")
    t = {
        "hidden": torch.from_numpy(x["hidden"].view(np.int16)).view(torch.bfloat16).to(dev),
        "weight": torch.from_numpy(x["weight"].view(np.int16)).view(torch.bfloat16).to(dev),
        "labels": torch.from_numpy(x["labels"]).to(dev),
        "grad_logprob": torch.from_numpy(x["grad_logprob"]).to(dev),
        "grad_entropy": torch.from_numpy(x["grad_entropy"]).to(dev),
    }
    N, H, V = wl.N, wl.H, wl.V
    n_valid = int((x["labels"] != wl.ignore_index).sum())
    red = flce.FLCE_REDUCTION_MEAN if wl.reduction == "mean" else flce.FLCE_REDUCTION_NONE
    fbytes, bbytes = flce.flce_workspace_size(N, H, V, red)
    f32 = dict(dtype=torch.float32, device=dev)
    lse = torch.empty(N, **f32)
    lp = torch.empty(N, **f32)
    ent = torch.empty(N, **f32)
    lpm = torch.empty(1, **f32)
    entm = torch.empty(1, **f32)
    gh = torch.empty((N, H), dtype=torch.bfloat16, device=dev)
    gw = torch.empty((H, V), dtype=torch.bfloat16, device=dev)
    wsf = torch.empty(fbytes, dtype=torch.uint8, device=dev)
    wsb = torch.empty(bbytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream().cuda_stream
    P = {k: v.data_ptr() for k, v in t.items()}

    def step():
        flce.flce_forward(P["hidden"], P["weight"], P["labels"], N, H, V, wl.ignore_index,
                          wl.softcap, red, lse.data_ptr(), lp.data_ptr(), ent.data_ptr(),
                          lpm.data_ptr(), entm.data_ptr(), wsf.data_ptr(), fbytes, stream)
        flce.flce_backward(P["hidden"], P["weight"], P["labels"], N, H, V, wl.ignore_index,
                           wl.softcap, red, lse.data_ptr(), ent.data_ptr(), P["grad_logprob"],
                           P["grad_entropy"], gh.data_ptr(), gw.data_ptr(), wsb.data_ptr(),
                           bbytes, stream)

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 19   # bf16 elements
        src = torch.ones(n, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        print(f"[bench] calibration copy of {args.copy_calibration_mib} MiB done", flush=True)

    # Peak memory of one fused step, everything allocated by torch.
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    step()
    torch.cuda.synchronize()
    fused_peak = torch.cuda.max_memory_allocated()
    print(f"[bench] {wl.name} N={N} H={H} V={V}: warmup {args.warmup}", flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    print(f"[bench] timing {args.steps} steps", flush=True)
    flce.flce_profile_reset()
    flce.flce_profile_enable(True)
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(args.steps):
        step()
    b.record()
    torch.cuda.synchronize()
    flce.flce_profile_enable(False)
    ms = a.elapsed_time(b) / args.steps
    table = flce.profile_table()

    kernels = {}
    for name, (n, tot) in table.items():
        per = tot / n
        row = {"launches_per_step": n / args.steps, "ms_per_launch": per,
               "ms_per_step": tot / args.steps}
        if name in FLOPS_PER_TOKEN_HV:
            flops = FLOPS_PER_TOKEN_HV[name] * n_valid * H * V * args.steps / n
            row["tflops"] = flops / (per * 1e-3) / 1e12
            row["mfma_frac"] = row["tflops"] / PEAK_BF16_TFLOPS
        kernels[name] = row
    dom = max(kernels, key=lambda k: kernels[k]["ms_per_step"])
    dk = kernels[dom]
    traffic = counted_traffic(wl.name)
    step_tflops = 8.0 * n_valid * H * V / (ms * 1e-3) / 1e12

    out = {
        "metric": METRIC,
        "value": N / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "N": N, "H": H, "V": V, "n_valid": n_valid,
                   "labels": wl.labels, "softcap": wl.softcap, "reduction": wl.reduction,
                   "parallelism": "single GPU"},
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": dk.get("tflops"),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": dk.get("mfma_frac"),
                     "traffic": (traffic or {}).get(dom)},
        "step_tflops": step_tflops,
        "step_mfma_frac": step_tflops / PEAK_BF16_TFLOPS,
        "kernels": kernels,
        "memory": {"fused_step_peak_bytes": int(fused_peak),
                   "fp32_logits_bytes": 4 * N * V,
                   "workspace_bytes": {"forward": fbytes, "backward": bbytes}},
    }
    if args.torch_ref:
        try:
            print("[bench] torch materialising reference", flush=True)
            out["torch_ref"] = torch_reference(t, wl)
        except Exception as exc:  # context only; never fatal
            out["torch_ref"] = {"error": str(exc)[:200]}
    if args.cpu_tokens > 0:
        print(f"[bench] cpu oracle on {args.cpu_tokens} tokens", flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, x, args.cpu_tokens)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
