"""Benchmark of the fused linear cross-entropy + entropy head on one MI355X.

One step = flce_forward + flce_backward over one batch (the whole hot path:
logit tiles with the online softmax/entropy epilogue, the tile combine, the
logit-gradient recompute, dHidden and dWeight contractions). Inputs are
seeded synthetic data resident in HBM before the timed region. The default
workload is the Llama-3-shaped head (N=8192 tokens, H=4096, V=128256, Zipf
labels, reduction none, per-token upstream gradients).

--path fused times flce_forward_backward instead (the gradient formed from
logits kept during the forward, for upstream gradients known in advance; no
recompute GEMM) with its default token chunks (kept-logit images within
1 GiB). With the default path the fused one is also timed on the same inputs
and reported under alt_paths.fused, and with every logit of the batch kept in
one chunk under alt_paths.fused_one_chunk (--alt-fused 0 skips both).

Prints one JSON line. Besides the throughput it reports:
  roofline      the dominant kernel's algorithmic TFLOP/s (flops per launch /
                mean launch time from HIP events recorded by the library on its
                launch stream during the timed region) against the bf16 dense
                MFMA peak;
  kernels       the same figures for every kernel kind;
  fwd_ms, bwd_ms  flce_forward and flce_backward timed on their own;
  cpu_baseline  the float64 CPU oracle timed on a bounded token sample;
  mfma_sustained  the bf16 MFMA rate the device sustains in the kernels' wave
                tile with no memory traffic, on pseudo-random and on zero
                operands, and with the tile's LDS fragment reads and its
                L2 -> LDS DMA added (flce_probe_mfma_rate modes 0-3);
                roofline.frac_of_sustained is the roofline kernel's rate
                against the random-operand figure, frac_of_lds_dma_probe
                against the figure with the tile's data movement;
  memory        peak device memory of one step vs the fp32 logits that a
                materialising implementation needs;
  torch_ref     (optional) a materialising torch implementation of the same
                forward + backward on the same GPU, for context.

roofline.traffic is the dominant kernel's fabric bytes per launch: what its
L2 caches fetched from and wrote to the memory fabric (MALL hits and HBM
alike; the counters do not separate them), from the rocprofv3 counters
FETCH_SIZE and WRITE_SIZE, each scaled by what it reads for a plain device
copy of known size in the same run, taken from profiles/traffic_<workload>.txt;
it is null when that file is missing or was taken on kernel sources other
than the ones built now (a SHA-256 over the library's sources is stored with
the counters). --copy-calibration-mib runs that plain copy once before warmup,
for the counter runs.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import platform
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # 256 CUs x 4096 flop/clk x 2.4 GHz, dense
METRIC = "fwd+bwd tokens/s and % bf16 MFMA peak, N=8192 H=4096 V=128256, 1 GPU"

# Algorithmic flops per valid token of each kernel kind, in units of H*V.
FLOPS_PER_TOKEN_HV = {"fwd_tile": 2, "bwd_dlogits": 2, "bwd_dx": 2, "bwd_dw": 2, "fused_tile": 2}
# Algorithmic HBM bytes per valid token of the memory-bound kernels, in units
# of V: the fused path's gradient pass reads each kept bf16 logit and writes
# the two bf16 gradient images.
BYTES_PER_TOKEN_V = {"fused_dlogits": 6}
PEAK_HBM_GBPS = 8000.0


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
    ap.add_argument("--path", choices=("recompute", "fused"), default="recompute",
                    help="recompute: flce_forward + flce_backward; fused: flce_forward_backward")
    ap.add_argument("--alt-fused", type=int, default=1,
                    help="with --path recompute, also time the fused path (0/1)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB before warmup "
                         "(the reference point of the HBM byte counters)")
    return ap.parse_args()


def _code_only(text: str) -> str:
    """C/C++ source without comments and with whitespace collapsed: editing a
    comment does not change a kernel."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    """SHA-256 over the code (comments and blank space dropped) of the
    library's kernel and boundary sources, in a fixed order."""
    files = sorted(glob.glob(os.path.join(ROOT, "linear_cross_entropy_tile_amd", "csrc", "*")))
    files.append(os.path.join(ROOT, "include", "flce.h"))
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()


TRAFFIC_WHAT = ("fabric bytes per launch (L2 fetches + writes to MALL or HBM, rocprofv3 "
                "FETCH_SIZE + WRITE_SIZE scaled by a device-copy calibration)")


def counted_traffic(workload: str, path: str = "recompute"):
    """Per-kernel fabric bytes (L2 misses to MALL or HBM, and L2 write-backs)
    per launch from profiles/traffic_<workload>.txt
    (traffic_<workload>_fused.txt for the fused path), or None when absent or
    taken on other sources. Lines of that file:
      source_sha256 <hex>
      kernel <kind> fetch_bytes <B> write_bytes <B>"""
    suffix = "" if path == "recompute" else "_" + path
    fname = os.path.join(ROOT, "profiles", f"traffic_{workload}{suffix}.txt")
    if not os.path.exists(fname):
        return None
    sha, per = None, {}
    with open(fname) as fh:
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


def kernel_rows(table, steps, n_valid, H, V):
    """Per kernel kind: launches and ms per step, and the algorithmic rate."""
    kernels = {}
    for name, (n, tot) in table.items():
        per = tot / n
        row = {"launches_per_step": n / steps, "ms_per_launch": per, "ms_per_step": tot / steps}
        if name in FLOPS_PER_TOKEN_HV:
            flops = FLOPS_PER_TOKEN_HV[name] * n_valid * H * V * steps / n
            row["tflops"] = flops / (per * 1e-3) / 1e12
            row["mfma_frac"] = row["tflops"] / PEAK_BF16_TFLOPS
        if name in BYTES_PER_TOKEN_V:
            nbytes = BYTES_PER_TOKEN_V[name] * n_valid * V * steps / n
            row["gbps"] = nbytes / (per * 1e-3) / 1e9
            row["hbm_frac"] = row["gbps"] / PEAK_HBM_GBPS
        kernels[name] = row
    # Chunks whose dH and dW tiles share one launch (bwd_dxdw) leave bwd_dx and
    # bwd_dw with only part of the vocabulary: the three kinds are then rated
    # together, 4 flop per valid token x H x V over their summed time.
    group = [k for k in ("bwd_dx", "bwd_dw", "bwd_dxdw") if k in table]
    if "bwd_dxdw" in table:
        gms = sum(table[k][1] for k in group)
        rate = 4 * n_valid * H * V * steps / (gms * 1e-3) / 1e12
        for k in group:
            kernels[k]["tflops"] = rate
            kernels[k]["mfma_frac"] = rate / PEAK_BF16_TFLOPS
            kernels[k]["rated_with"] = "+".join(group)
    return kernels


def timed(step, steps, warmup):
    """Mean ms per step over `steps` after `warmup` steps, and the library's
    per-kernel event timings of the timed steps."""
    import torch
    from linear_cross_entropy_tile_amd import flce
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    flce.flce_profile_reset()
    flce.flce_profile_enable(True)
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(steps):
        step()
    b.record()
    torch.cuda.synchronize()
    flce.flce_profile_enable(False)
    return a.elapsed_time(b) / steps, flce.profile_table()


def peak_of(step):
    """Peak device memory (torch allocator) of one step."""
    import torch
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    step()
    torch.cuda.synchronize()
    return int(torch.cuda.max_memory_allocated())


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path "
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
    stream = torch.cuda.current_stream().cuda_stream
    P = {k: v.data_ptr() for k, v in t.items()}
    # The recompute path's workspaces, allocated on first use and released
    # before the fused path is measured (each path's peak counts its own).
    rws = {}

    def rws_ptr(key, nbytes):
        if key not in rws:
            rws[key] = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        return rws[key].data_ptr()

    def fwd_only():
        flce.flce_forward(P["hidden"], P["weight"], P["labels"], N, H, V, wl.ignore_index,
                          wl.softcap, red, lse.data_ptr(), lp.data_ptr(), ent.data_ptr(),
                          lpm.data_ptr(), entm.data_ptr(), rws_ptr("f", fbytes), fbytes, stream)

    def bwd_only():
        flce.flce_backward(P["hidden"], P["weight"], P["labels"], N, H, V, wl.ignore_index,
                           wl.softcap, red, lse.data_ptr(), ent.data_ptr(), P["grad_logprob"],
                           P["grad_entropy"], gh.data_ptr(), gw.data_ptr(), rws_ptr("b", bbytes),
                           bbytes, stream)

    def step_recompute():
        fwd_only()
        bwd_only()

    opt = flce.FlceOptions(wl.ignore_index, wl.softcap, red, 0.0, flce.FLCE_GRAD_BF16)
    reduced = torch.empty(4, **f32)
    fused_ws = {}

    def make_step_fused(chunk_tokens):
        """flce_forward_backward with `chunk_tokens` (0: the library's
        default); its workspace is allocated on the first call and freed
        before another chunking allocates its own."""
        def step_fused():
            if fused_ws.get("chunk") != chunk_tokens:
                fused_ws.clear()
                torch.cuda.empty_cache()
                fused_ws["chunk"] = chunk_tokens
                fused_ws["bytes"] = flce.flce_fused_workspace_size(N, H, V, opt, chunk_tokens)
                fused_ws["buf"] = torch.empty(fused_ws["bytes"], dtype=torch.uint8, device=dev)
            flce.flce_forward_backward(P["hidden"], P["weight"], P["labels"], N, H, V, opt,
                                       chunk_tokens, P["grad_logprob"], P["grad_entropy"], None,
                                       None, lse.data_ptr(), lp.data_ptr(), ent.data_ptr(), None,
                                       None, reduced.data_ptr(), gh.data_ptr(), gw.data_ptr(),
                                       fused_ws["buf"].data_ptr(), fused_ws["bytes"], stream)
        return step_fused

    step_fused = make_step_fused(0)
    step = step_fused if args.path == "fused" else step_recompute

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 19   # bf16 elements
        src = torch.ones(n, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        print(f"[bench] calibration copy of {args.copy_calibration_mib} MiB done", flush=True)

    # Peak memory of one step, everything allocated by torch.
    step_peak = peak_of(step)
    print(f"[bench] {wl.name} N={N} H={H} V={V} path={args.path}: warmup {args.warmup}, "
          f"timing {args.steps} steps", flush=True)
    ms, table = timed(step, args.steps, args.warmup)
    kernels = kernel_rows(table, args.steps, n_valid, H, V)
    dom = max((k for k in kernels if "tflops" in kernels[k]),
              key=lambda k: kernels[k]["ms_per_step"])
    dk = kernels[dom]
    traffic = counted_traffic(wl.name, args.path)
    # Algorithmic flops of the step: 8 N H V with the recompute (forward,
    # recompute, dH, dW), 6 N H V on the fused path, which skips the recompute.
    step_flops_hv = 8.0 if args.path == "recompute" else 6.0
    step_tflops = step_flops_hv * n_valid * H * V / (ms * 1e-3) / 1e12

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
                   "path": args.path, "parallelism": "single GPU"},
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": dk.get("tflops"),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": dk.get("mfma_frac"),
                     "traffic": (traffic or {}).get(dom), "traffic_what": TRAFFIC_WHAT},
        "step_tflops": step_tflops,
        "step_mfma_frac": step_tflops / PEAK_BF16_TFLOPS,
        "kernels": kernels,
        "memory": {"step_peak_bytes": int(step_peak),
                   "fp32_logits_bytes": 4 * N * V,
                   "workspace_bytes": ({"forward": fbytes, "backward": bbytes}
                                       if args.path == "recompute"
                                       else {"fused": fused_ws.get("bytes")})},
    }
    # The rate the matrix cores sustain here on varying data (context for
    # the roofline fraction against the published peak).
    if args.path == "recompute":
        # The step's two halves timed on their own (same stream, events).
        out["fwd_ms"], _ = timed(fwd_only, args.steps, 1)
        out["bwd_ms"], _ = timed(bwd_only, args.steps, 1)
    # Context measurements below never keep the line from being printed.
    try:
        probe_ws = torch.empty(256 * 512 * 4 + (2 << 20), dtype=torch.uint8, device=dev)
        probe = lambda mode, steps: flce.flce_probe_mfma_rate(mode, steps, probe_ws.data_ptr(),
                                                              probe_ws.numel(), stream)
        probe(flce.PROBE_REGISTERS, 20000)  # warm-up: let the clock settle under this load
        sustained = {
            "random_tflops": probe(flce.PROBE_REGISTERS, 120000),
            "zero_tflops": probe(flce.PROBE_ZEROS, 120000),
            "lds_tflops": probe(flce.PROBE_LDS, 120000),
            "lds_dma_tflops": probe(flce.PROBE_LDS_DMA, 120000),
            "what": "4 x 2 v_mfma_f32_32x32x16_bf16 wave tile, 2 waves per SIMD, one block per "
                    "CU: operands in registers, uniform in [-2, 2) (random) or zero; random "
                    "with the fragments read from LDS (lds); and with the 32 KiB-per-K-block "
                    "global->LDS DMA of a 256 x 256 tile from L2 added (lds_dma)",
        }
        out["mfma_sustained"] = sustained
        if out["roofline"]["achieved"]:
            out["roofline"]["frac_of_sustained"] = (out["roofline"]["achieved"]
                                                    / sustained["random_tflops"])
            out["roofline"]["frac_of_lds_dma_probe"] = (out["roofline"]["achieved"]
                                                        / sustained["lds_dma_tflops"])
    except Exception as exc:
        out["mfma_sustained"] = {"error": str(exc)[:200]}
    if args.path == "recompute" and args.alt_fused:
        rws.clear()
        torch.cuda.empty_cache()
        out["alt_paths"] = {}
        vt = -(-V // 256) * 256
        for key, chunk in (("fused", 0), ("fused_one_chunk", N)):
            try:
                print(f"[bench] fused path (gradient in the forward), {key}", flush=True)
                sf = make_step_fused(chunk)
                fpeak = peak_of(sf)
                fms, ftable = timed(sf, args.steps, args.warmup)
                fk = kernel_rows(ftable, args.steps, n_valid, H, V)
                fdom = max((k for k in fk if "tflops" in fk[k]),
                           key=lambda k: fk[k]["ms_per_step"])
                ntok = fk["fused_tile"]["launches_per_step"] if "fused_tile" in fk else None
                out["alt_paths"][key] = {
                    "value": N / (fms * 1e-3), "unit": "tokens/s", "ms_per_step": fms,
                    "executed_tflops": 6.0 * n_valid * H * V / (fms * 1e-3) / 1e12,
                    "chunk_tokens": chunk if chunk else "default",
                    "token_chunks_run": ntok,
                    "peak_bytes": fpeak, "workspace_bytes": fused_ws["bytes"],
                    "kept_logit_image_bytes": 4 * vt * 256 * (
                        -(-chunk // 256) if chunk
                        else min(-(-N // 256), max(1, (1 << 30) // (4 * 256 * vt)))),
                    "roofline": {"kernel": fdom, "bound": "mfma",
                                 "achieved": fk[fdom]["tflops"], "peak": PEAK_BF16_TFLOPS,
                                 "unit": "TFLOP/s", "frac": fk[fdom]["mfma_frac"],
                                 "traffic": ((counted_traffic(wl.name, "fused") or {}).get(fdom)
                                             if key == "fused" else None)},
                    "kernels": fk}
            except Exception as exc:
                out["alt_paths"][key] = {"error": str(exc)[:200]}
        fused_ws.clear()
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
