"""The C ABI on the CPU: libflce.so loads, exports every function that
include/flce.h declares, and rejects bad arguments on the host with the
documented status codes (no device work is involved on these paths)."""
import ctypes
import os
import re
import subprocess

import pytest

from linear_cross_entropy_tile_amd import flce

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flce.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(flce_[a-z_]+)\s*\(", text)))


def _exported():
    out = subprocess.run(["nm", "-D", "--defined-only", flce.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    return {ln.split()[-1] for ln in out.splitlines() if " T " in ln}


def test_library_loads():
    assert flce.flce_version() >= 100


def test_exports_match_header():
    decl = _declared()
    assert len(decl) >= 10, decl
    exp = _exported()
    missing = [d for d in decl if d not in exp]
    assert not missing, f"declared but not exported: {missing}"
    extra = sorted(e for e in exp if e.startswith("flce_") and e not in decl)
    assert not extra, f"exported but not declared: {extra}"
    assert set(flce._SIG) == set(decl), "binding and header disagree"


def test_status_strings():
    for code in range(11):
        assert flce.flce_status_string(code)
    assert "unknown" in flce.flce_status_string(99)


# Host-side validation: none of these calls reaches the device. Pointer values
# are dummies (16-byte aligned) that are never dereferenced.
A = 0x1000
BIG = 1 << 40


def _fwd(**kw):
    args = dict(hidden=A, weight=A, labels=A, N=4, H=8, V=8, ii=-100, cap=0.0, red=0,
                lse=A, lp=A, ent=A, lpm=None, entm=None, ws=A, wsb=BIG, st=None)
    args.update(kw)
    return flce.lib().flce_forward(args["hidden"], args["weight"], args["labels"], args["N"],
                                   args["H"], args["V"], args["ii"], args["cap"], args["red"],
                                   args["lse"], args["lp"], args["ent"], args["lpm"],
                                   args["entm"], args["ws"], args["wsb"], args["st"])


def _bwd(**kw):
    args = dict(hidden=A, weight=A, labels=A, N=4, H=8, V=8, ii=-100, cap=0.0, red=0,
                lse=A, ent=A, g=A, e=A, gh=A, gw=A, ws=A, wsb=BIG, st=None)
    args.update(kw)
    return flce.lib().flce_backward(args["hidden"], args["weight"], args["labels"], args["N"],
                                    args["H"], args["V"], args["ii"], args["cap"], args["red"],
                                    args["lse"], args["ent"], args["g"], args["e"], args["gh"],
                                    args["gw"], args["ws"], args["wsb"], args["st"])


@pytest.mark.parametrize("kw,code", [
    (dict(hidden=None), 1), (dict(weight=None), 1), (dict(labels=None), 1), (dict(lse=None), 1),
    (dict(ws=None), 1), (dict(red=1), 1), (dict(red=2), 1),    # mean / sum need the outputs
    (dict(N=-1), 2), (dict(N=(1 << 21) + 1), 2), (dict(H=0), 2), (dict(V=0), 2),
    (dict(H=(1 << 20) + 8), 2),
    (dict(V=(1 << 22) + 8), 2),
    (dict(red=3), 3), (dict(red=-1), 3),
    (dict(H=12), 4), (dict(hidden=A + 2), 4), (dict(weight=A + 8), 4),
    (dict(ws=A + 4), 4),
    (dict(wsb=16), 5),
    (dict(cap=float("nan")), 6), (dict(cap=float("inf")), 6),
])
def test_forward_rejects(kw, code):
    assert _fwd(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(weight=None), 1), (dict(gw=None), 1), (dict(gh=None), 1), (dict(lse=None), 1),
    (dict(ent=None), 1), (dict(ws=None), 1),
    (dict(N=-3), 2), (dict(H=-8), 2),
    (dict(red=7), 3),
    (dict(gh=A + 2), 4), (dict(gw=A + 2), 4), (dict(H=12), 4),
    (dict(wsb=100), 5),
    (dict(cap=float("-inf")), 6),
])
def test_backward_rejects(kw, code):
    assert _bwd(**kw) == code


def _fwd_noalloc(**kw):
    args = dict(hidden=A, weight=A, labels=A, N=4, H=8, V=8, ii=-100, cap=0.0, red=0,
                lse=A, lp=A, ent=A, lpm=None, entm=None, st=None)
    args.update(kw)
    return flce.lib().flce_forward_noalloc(args["hidden"], args["weight"], args["labels"],
                                           args["N"], args["H"], args["V"], args["ii"],
                                           args["cap"], args["red"], args["lse"], args["lp"],
                                           args["ent"], args["lpm"], args["entm"], args["st"])


@pytest.mark.parametrize("kw,code", [
    (dict(N=-1), 2), (dict(H=12), 4), (dict(red=7), 3), (dict(cap=float("inf")), 6),
    # forward workspace beyond the static scratch: 16 * N * ceil(V/256) + 2 N H bytes
    (dict(N=8192, H=4096, V=128256), 10), (dict(N=1 << 20, H=64, V=512), 10),
    (dict(N=4096, H=4096, V=128256 + 1), 10),   # the padded weight copy alone is 1 GB
])
def test_forward_noalloc_rejects(kw, code):
    """The static-scratch forward refuses bad arguments and shapes that do not
    fit its scratch on the host, before it looks up the device array."""
    assert _fwd_noalloc(**kw) == code


def test_workspace_size():
    f, b = flce.flce_workspace_size(8192, 4096, 128256, 0)
    # 16 B per (token, 256-wide vocabulary tile) of forward partials.
    assert f >= 16 * 8192 * 501
    # bounded logit-gradient slice + fp32 dHidden accumulator; far below N*V*2.
    assert b < 2 * 8192 * 128256 and b >= 8192 * 4096 * 4
    f1, b1 = flce.flce_workspace_size(0, 64, 64, 1)
    assert f1 >= 256 and b1 >= 256
    with pytest.raises(flce.FlceError):
        flce.flce_workspace_size(4, 7, 8, 0)


def test_profile_hooks_host_only():
    flce.flce_profile_reset()
    assert flce.flce_profile_kinds() >= 8
    name, n, ms = flce.flce_profile_read(1)
    assert name == "fwd_tile" and n == 0 and ms == 0.0
    with pytest.raises(flce.FlceError):
        flce.flce_profile_read(99)


def _opt(**kw):
    o = dict(ignore_index=-100, softcap=0.0, reduction=0, z_loss_scale=0.0, grad_dtype=0,
             class_weight=None, entropy_per_token=0)
    o.update(kw)
    return flce.FlceOptions(o["ignore_index"], o["softcap"], o["reduction"], o["z_loss_scale"],
                            o["grad_dtype"], o["class_weight"], o["entropy_per_token"])


def _fwd_ex(opt=None, **kw):
    args = dict(hidden=A, weight=A, labels=A, N=4, H=8, V=8, lse=A, lp=A, ent=A, uce=None,
                zl=None, red=None, ws=A, wsb=BIG, st=None)
    args.update(kw)
    o = ctypes.byref(opt) if opt is not None else None
    return flce.lib().flce_forward_ex(args["hidden"], args["weight"], args["labels"], args["N"],
                                      args["H"], args["V"], o, args["lse"], args["lp"],
                                      args["ent"], args["uce"], args["zl"], args["red"],
                                      args["ws"], args["wsb"], args["st"])


def _bwd_ex(opt=None, **kw):
    args = dict(hidden=A, weight=A, labels=A, N=4, H=8, V=8, lse=A, ent=A, g=A, e=A, gu=None,
                gz=None, gh=A, gw=A, ws=A, wsb=BIG, st=None)
    args.update(kw)
    o = ctypes.byref(opt) if opt is not None else None
    return flce.lib().flce_backward_ex(args["hidden"], args["weight"], args["labels"], args["N"],
                                       args["H"], args["V"], o, args["lse"], args["ent"],
                                       args["g"], args["e"], args["gu"], args["gz"], args["gh"],
                                       args["gw"], args["ws"], args["wsb"], args["st"])


@pytest.mark.parametrize("okw,kw,code", [
    (None, {}, 1),                                          # no options
    (dict(reduction=1), {}, 1), (dict(reduction=2), {}, 1),  # reduced outputs required
    (dict(reduction=5), {}, 3),
    (dict(softcap=float("nan")), {}, 6),
    (dict(z_loss_scale=-0.5), {}, 9), (dict(z_loss_scale=float("inf")), {}, 9),
    (dict(grad_dtype=3), {}, 9),
    (dict(class_weight=A), {}, 9),                          # class weights under "none"
    (dict(reduction=2, class_weight=A + 2), dict(red=A), 4),  # class weights not 4-byte aligned
    (dict(), dict(N=-2), 2), (dict(), dict(H=12), 4), (dict(), dict(wsb=8), 5),
])
def test_forward_ex_rejects(okw, kw, code):
    assert _fwd_ex(_opt(**okw) if okw is not None else None, **kw) == code


@pytest.mark.parametrize("okw,kw,code", [
    (None, {}, 1),
    (dict(reduction=-3), {}, 3),
    (dict(z_loss_scale=float("nan")), {}, 9), (dict(grad_dtype=-1), {}, 9),
    (dict(grad_dtype=1), dict(V=(1 << 21) + 8), 2),           # fp32 gradients: V <= 2^21
    (dict(class_weight=A), {}, 9), (dict(reduction=1, class_weight=A + 1), {}, 4),
    (dict(reduction=1, entropy_per_token=2), {}, 9), (dict(entropy_per_token=-1), {}, 9),
    (dict(), dict(gw=None), 1), (dict(), dict(gh=A + 4), 4), (dict(), dict(wsb=8), 5),
])
def test_backward_ex_rejects(okw, kw, code):
    assert _bwd_ex(_opt(**okw) if okw is not None else None, **kw) == code


def test_options_layout():
    # flce_options_t: int64, float, int, float, int, pointer, int -> 40 bytes
    # with natural alignment (4 bytes of padding before the pointer and at
    # the end).
    assert ctypes.sizeof(flce.FlceOptions) == 40
    assert flce.FlceOptions.reduction.offset == 12 and flce.FlceOptions.grad_dtype.offset == 20
    assert flce.FlceOptions.class_weight.offset == 24
    assert flce.FlceOptions.entropy_per_token.offset == 32
    assert flce.flce_version() == 212


def test_binding_shape_checks():
    """The torch wrappers refuse tensors whose extents disagree before any
    launch (the kernels read every tensor by N, H and V): hidden [N,H],
    weight [H,V], labels [N], and the saved lse / entropy [N]."""
    import torch
    h = torch.zeros(6, 8)
    w = torch.zeros(8, 5)
    y = torch.zeros(6, dtype=torch.int64)
    v = torch.zeros(6)
    flce.check_shapes(h, w, y, ("lse", v), ("entropy", v))
    with pytest.raises(ValueError):
        flce.check_shapes(h, torch.zeros(7, 5), y)
    with pytest.raises(ValueError):
        flce.check_shapes(h, w, torch.zeros(5, dtype=torch.int64))
    with pytest.raises(ValueError):
        flce.check_shapes(h, w, y, ("lse", torch.zeros(5)))
    with pytest.raises(ValueError):
        flce.check_shapes(h, w, y, ("lse", v), ("entropy", torch.zeros(7)))
    with pytest.raises(ValueError):
        flce.check_shapes(h, torch.zeros(8), y)


def test_entropy_reduction_argument():
    assert flce._entropy_per_token("mean", None) == 0
    assert flce._entropy_per_token("mean", "mean") == 0
    assert flce._entropy_per_token("none", "none") == 0
    assert flce._entropy_per_token("sum", "none") == 1
    with pytest.raises(ValueError):
        flce._entropy_per_token("none", "mean")


def test_workspace_size_any_vocabulary():
    # A vocabulary that is not a multiple of 8 adds the padded weight copy
    # and the padded dW buffer (fp32 room) to the backward and fused
    # workspaces, the weight copy to the forward one.
    H = 64
    f0, b0 = flce.flce_workspace_size(300, H, 1000, 0)
    f1, b1 = flce.flce_workspace_size(300, H, 1001, 0)
    assert f1 >= f0 + 2 * H * 1008 and b1 >= b0 + 6 * H * 1008
    u0 = flce.flce_fused_workspace_size(300, H, 1000, _opt())
    u1 = flce.flce_fused_workspace_size(300, H, 1001, _opt())
    assert u1 >= u0 + 6 * H * 1008


def test_workspace_size_sum():
    f0, b0 = flce.flce_workspace_size(4096, 4096, 32000, 0)
    f2, b2 = flce.flce_workspace_size(4096, 4096, 32000, 2)
    assert f2 > f0 and b2 == b0


def _fwd_shard(opt, **kw):
    args = dict(hidden=A, weight=A, labels=A, N=4, H=8, Vs=8, v0=0, VT=16, state=A, zl=A, ws=A,
                wsb=BIG, st=None)
    args.update(kw)
    return flce.lib().flce_forward_shard(args["hidden"], args["weight"], args["labels"], args["N"],
                                         args["H"], args["Vs"], args["v0"], args["VT"],
                                         ctypes.byref(opt), args["state"], args["zl"], args["ws"],
                                         args["wsb"], args["st"])


@pytest.mark.parametrize("kw,code", [
    (dict(v0=-8), 2), (dict(v0=12), 2), (dict(VT=4), 2),    # slice outside [0, V_total)
    (dict(state=None), 1), (dict(zl=None), 1), (dict(state=A + 4), 4), (dict(H=12), 4),
])
def test_forward_shard_rejects(kw, code):
    assert _fwd_shard(_opt(), **kw) == code


def test_merge_rejects_and_size():
    L = flce.lib()
    o = _opt(reduction=1)
    assert L.flce_merge_shards(A, A, 0, A, 4, 16, ctypes.byref(o), A, A, A, None, None, A, A, BIG,
                               None) == 2
    assert L.flce_merge_shards(A, A, 2, A, 4, 16, ctypes.byref(o), A, A, A, None, None, None, A,
                               BIG, None) == 1
    assert L.flce_merge_shards(A, A, 2, A, 4, 16, ctypes.byref(o), A, A, A, None, None, A, A, 8,
                               None) == 5
    assert flce.flce_merge_workspace_size(8192) >= 8192 * 8


def _fused(opt=None, **kw):
    args = dict(hidden=A, weight=A, labels=A, N=4, H=8, V=8, chunk=0, g=A, e=A, gu=None, gz=None,
                lse=A, lp=A, ent=A, uce=None, zl=None, red=None, gh=A, gw=A, ws=A, wsb=BIG,
                st=None)
    args.update(kw)
    o = ctypes.byref(opt) if opt is not None else None
    return flce.lib().flce_forward_backward(
        args["hidden"], args["weight"], args["labels"], args["N"], args["H"], args["V"], o,
        args["chunk"], args["g"], args["e"], args["gu"], args["gz"], args["lse"], args["lp"],
        args["ent"], args["uce"], args["zl"], args["red"], args["gh"], args["gw"], args["ws"],
        args["wsb"], args["st"])


@pytest.mark.parametrize("okw,kw,code", [
    (None, {}, 1),                                           # no options
    (dict(reduction=1), {}, 1), (dict(reduction=2), {}, 1),  # reduced outputs required
    (dict(reduction=4), {}, 3), (dict(softcap=float("inf")), {}, 6),
    (dict(z_loss_scale=-1.0), {}, 9), (dict(grad_dtype=2), {}, 9),
    (dict(), dict(N=-1), 2), (dict(), dict(V=(1 << 21) + 8), 2),  # V <= 2^21
    (dict(), dict(chunk=-256), 2), (dict(), dict(H=12), 4),
    (dict(), dict(lse=None), 1), (dict(), dict(gw=None), 1), (dict(), dict(ws=None), 1),
    (dict(), dict(gh=A + 8), 4), (dict(), dict(wsb=8), 5),
])
def test_forward_backward_rejects(okw, kw, code):
    assert _fused(_opt(**okw) if okw is not None else None, **kw) == code


def test_fused_workspace_size():
    o = _opt()
    one = flce.flce_fused_workspace_size(8192, 4096, 128256, o, 8192)
    four = flce.flce_fused_workspace_size(8192, 4096, 128256, o, 2048)
    vt = -(-128256 // 256) * 256
    # One chunk: both bf16 images of all 8192 x vt logits, the re-laid-out
    # weight, and the forward's partial states.
    assert one >= 4 * 8192 * vt + 2 * 4096 * vt + 16 * 8192 * (vt // 256)
    # Four chunks: images of 2048 tokens plus the fp32 dW accumulator.
    assert four >= 4 * 2048 * vt + 4 * 4096 * 128256
    assert four < one
    # fp32 gradients accumulate dW in grad_weight itself.
    assert flce.flce_fused_workspace_size(8192, 4096, 128256, _opt(grad_dtype=1), 2048) < four
    # The default chunk is the largest whose two bf16 images fit in 1 GiB:
    # 2048 tokens at V = 128256 (4 * 2048 * 128256 bytes), 8192 at V = 32000
    # (one chunk for N = 4096), and at least 256 tokens.
    assert flce.flce_fused_workspace_size(8192, 4096, 128256, o, 0) == four
    assert (flce.flce_fused_workspace_size(32768, 4096, 128256, o, 0)
            == flce.flce_fused_workspace_size(32768, 4096, 128256, o, 2048))
    assert (flce.flce_fused_workspace_size(4096, 4096, 32000, o, 0)
            == flce.flce_fused_workspace_size(4096, 4096, 32000, o, 4096))
    assert (flce.flce_fused_workspace_size(4096, 64, (1 << 21), o, 0)
            == flce.flce_fused_workspace_size(4096, 64, (1 << 21), o, 256))
    for N, V in ((8192, 128256), (8192, 256000), (32768, 152064), (4096, 32000)):
        vt = -(-V // 256) * 256
        d = flce.flce_fused_workspace_size(N, 4096, V, o, 0)
        images = d - flce.flce_fused_workspace_size(N, 4096, V, o, 256) + 4 * 256 * vt
        assert images <= (1 << 30) + 4 * 256 * vt
    with pytest.raises(flce.FlceError):
        flce.flce_fused_workspace_size(8, 8, (1 << 21) + 8, o, 0)


def test_probe_mfma_rejects():
    L = flce.lib()
    t = ctypes.c_double(0.0)
    assert L.flce_probe_mfma_rate(0, 1000, None, A, BIG, None) == 1
    assert L.flce_probe_mfma_rate(0, 1000, ctypes.byref(t), None, BIG, None) == 1
    assert L.flce_probe_mfma_rate(0, 2, ctypes.byref(t), A, BIG, None) == 2
    assert L.flce_probe_mfma_rate(0, (1 << 24) + 4, ctypes.byref(t), A, BIG, None) == 2
    assert L.flce_probe_mfma_rate(0, 1000, ctypes.byref(t), A, 1024, None) == 5
