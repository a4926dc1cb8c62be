"""ctypes binding for libflce.so (declared in include/flce.h).

Two layers, both argument marshalling only:

* ``flce_workspace_size``, ``flce_forward``, ``flce_backward``,
  ``flce_forward_ex``, ``flce_backward_ex``, ``flce_get_status``, ... : one
  Python function per C entry point, same name, same arguments (device
  pointers and streams as integers, the options as ``FlceOptions``). A non-OK
  status raises ``FlceError``.
* ``forward`` / ``backward`` / ``forward_backward`` (the fused call, for
  upstream gradients known before the forward): take torch CUDA tensors,
  check dtypes and layouts, allocate outputs and the workspace with torch (so
  torch's caching allocator owns all memory), and call the C entry points on
  torch's current stream. No arithmetic of the head happens here.

The library is loaded on first use. There is no fallback: if libflce.so is
missing or the device is not a GPU, calls raise.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "FlceError", "lib", "LIB_PATH",
    "FLCE_REDUCTION_NONE", "FLCE_REDUCTION_MEAN", "FLCE_REDUCTION_SUM",
    "FLCE_GRAD_BF16", "FLCE_GRAD_F32", "FlceOptions",
    "flce_workspace_size", "flce_forward", "flce_backward", "flce_forward_ex",
    "flce_backward_ex", "flce_fused_workspace_size", "flce_forward_backward", "flce_get_status",
    "flce_forward_noalloc", "FLCE_NOALLOC_SCRATCH_BYTES",
    "flce_status_string", "flce_version", "flce_profile_enable", "flce_profile_reset",
    "flce_profile_kinds", "flce_profile_read", "profile_table", "flce_probe_mfma_rate",
    "forward", "backward", "forward_backward", "workspace_bytes", "check_shapes",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libflce.so")

FLCE_REDUCTION_NONE = 0
FLCE_REDUCTION_MEAN = 1
FLCE_REDUCTION_SUM = 2
_REDUCTIONS = {"none": FLCE_REDUCTION_NONE, "mean": FLCE_REDUCTION_MEAN,
               "sum": FLCE_REDUCTION_SUM}
FLCE_GRAD_BF16 = 0
FLCE_GRAD_F32 = 1
_GRAD_DTYPES = {"bf16": FLCE_GRAD_BF16, "f32": FLCE_GRAD_F32}

STATUS_NAMES = {
    0: "FLCE_OK", 1: "FLCE_ERR_NULL_POINTER", 2: "FLCE_ERR_BAD_SHAPE",
    3: "FLCE_ERR_BAD_REDUCTION", 4: "FLCE_ERR_MISALIGNED",
    5: "FLCE_ERR_WORKSPACE_TOO_SMALL", 6: "FLCE_ERR_BAD_SOFTCAP", 7: "FLCE_ERR_HIP",
    8: "FLCE_ERR_INVALID_LABEL", 9: "FLCE_ERR_BAD_OPTION", 10: "FLCE_ERR_TOO_LARGE",
}
FLCE_NOALLOC_SCRATCH_BYTES = 64 << 20


class FlceOptions(ctypes.Structure):
    """flce_options_t."""
    _fields_ = [("ignore_index", ctypes.c_int64), ("softcap", ctypes.c_float),
                ("reduction", ctypes.c_int), ("z_loss_scale", ctypes.c_float),
                ("grad_dtype", ctypes.c_int), ("class_weight", ctypes.c_void_p),
                ("entropy_per_token", ctypes.c_int)]

# Every exported symbol with its (restype, argtypes).
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SIG = {
    "flce_workspace_size": (ctypes.c_int, [_I64, _I64, _I64, ctypes.c_int,
                                           ctypes.POINTER(ctypes.c_size_t),
                                           ctypes.POINTER(ctypes.c_size_t)]),
    "flce_forward": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, _I64, ctypes.c_float,
                                    ctypes.c_int, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "flce_backward": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, _I64, ctypes.c_float,
                                     ctypes.c_int, _P, _P, _P, _P, _P, _P, _P,
                                     ctypes.c_size_t, _P]),
    "flce_forward_noalloc": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, _I64, ctypes.c_float,
                                            ctypes.c_int, _P, _P, _P, _P, _P, _P]),
    "flce_forward_ex": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, ctypes.POINTER(FlceOptions),
                                       _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "flce_backward_ex": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, ctypes.POINTER(FlceOptions),
                                        _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "flce_fused_workspace_size": (ctypes.c_int, [_I64, _I64, _I64, ctypes.POINTER(FlceOptions),
                                                 _I64, ctypes.POINTER(ctypes.c_size_t)]),
    "flce_forward_backward": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64,
                                             ctypes.POINTER(FlceOptions), _I64, _P, _P, _P, _P,
                                             _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t,
                                             _P]),
    "flce_forward_shard": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, _I64, _I64,
                                          ctypes.POINTER(FlceOptions), _P, _P, _P,
                                          ctypes.c_size_t, _P]),
    "flce_merge_workspace_size": (ctypes.c_int, [_I64, ctypes.POINTER(ctypes.c_size_t)]),
    "flce_merge_shards": (ctypes.c_int, [_P, _P, _I64, _P, _I64, _I64, ctypes.POINTER(FlceOptions),
                                         _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "flce_backward_shard": (ctypes.c_int, [_P, _P, _P, _I64, _I64, _I64, _I64, _I64,
                                           ctypes.POINTER(FlceOptions), _P, _P, _P, _P, _P, _P,
                                           _P, _P, _P, ctypes.c_size_t, _P]),
    "flce_get_status": (ctypes.c_int, [_P, ctypes.POINTER(_I64), _P]),
    "flce_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "flce_version": (ctypes.c_int, []),
    "flce_profile_enable": (ctypes.c_int, [ctypes.c_int]),
    "flce_profile_reset": (ctypes.c_int, []),
    "flce_profile_kinds": (ctypes.c_int, []),
    "flce_profile_read": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(ctypes.c_char_p),
                                         ctypes.POINTER(_I64), ctypes.POINTER(ctypes.c_double)]),
    "flce_probe_mfma_rate": (ctypes.c_int, [ctypes.c_int, _I64, ctypes.POINTER(ctypes.c_double),
                                            _P, ctypes.c_size_t, _P]),
}


class FlceError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        name = STATUS_NAMES.get(status, str(status))
        try:
            text = lib().flce_status_string(status).decode()
        except Exception:  # pragma: no cover - library itself unavailable
            text = ""
        super().__init__(f"{where}: {name} ({text})")


_LIB = None


def lib():
    """The loaded libflce.so (loads it on first call)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "or python -m linear_cross_entropy_tile_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIG.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _LIB = L
    return _LIB


def _check(status: int, where: str) -> None:
    if status != 0:
        raise FlceError(status, where)


# ---------------------------------------------------------------- C entry points

def flce_workspace_size(N: int, H: int, V: int, reduction: int):
    f = ctypes.c_size_t(0)
    b = ctypes.c_size_t(0)
    _check(lib().flce_workspace_size(N, H, V, reduction, ctypes.byref(f), ctypes.byref(b)),
           "flce_workspace_size")
    return f.value, b.value


def flce_forward(hidden, weight, labels, N, H, V, ignore_index, softcap, reduction,
                 lse, logprob, entropy, logprob_mean, entropy_mean, workspace,
                 workspace_bytes, stream):
    _check(lib().flce_forward(hidden, weight, labels, N, H, V, ignore_index, softcap, reduction,
                              lse, logprob, entropy, logprob_mean, entropy_mean, workspace,
                              workspace_bytes, stream), "flce_forward")


def flce_forward_noalloc(hidden, weight, labels, N, H, V, ignore_index, softcap, reduction,
                         lse, logprob, entropy, logprob_mean, entropy_mean, stream):
    _check(lib().flce_forward_noalloc(hidden, weight, labels, N, H, V, ignore_index, softcap,
                                      reduction, lse, logprob, entropy, logprob_mean,
                                      entropy_mean, stream), "flce_forward_noalloc")


def flce_backward(hidden, weight, labels, N, H, V, ignore_index, softcap, reduction,
                  lse, entropy, grad_logprob, grad_entropy, grad_hidden, grad_weight,
                  workspace, workspace_bytes, stream):
    _check(lib().flce_backward(hidden, weight, labels, N, H, V, ignore_index, softcap,
                               reduction, lse, entropy, grad_logprob, grad_entropy,
                               grad_hidden, grad_weight, workspace, workspace_bytes, stream),
           "flce_backward")


def flce_forward_ex(hidden, weight, labels, N, H, V, opt, lse, logprob, entropy, uniform_ce,
                    z_loss, reduced, workspace, workspace_bytes, stream):
    _check(lib().flce_forward_ex(hidden, weight, labels, N, H, V, ctypes.byref(opt), lse,
                                 logprob, entropy, uniform_ce, z_loss, reduced, workspace,
                                 workspace_bytes, stream), "flce_forward_ex")


def flce_backward_ex(hidden, weight, labels, N, H, V, opt, lse, entropy, grad_logprob,
                     grad_entropy, grad_uniform_ce, grad_z_loss, grad_hidden, grad_weight,
                     workspace, workspace_bytes, stream):
    _check(lib().flce_backward_ex(hidden, weight, labels, N, H, V, ctypes.byref(opt), lse,
                                  entropy, grad_logprob, grad_entropy, grad_uniform_ce,
                                  grad_z_loss, grad_hidden, grad_weight, workspace,
                                  workspace_bytes, stream), "flce_backward_ex")


def flce_fused_workspace_size(N: int, H: int, V: int, opt, chunk_tokens: int = 0) -> int:
    b = ctypes.c_size_t(0)
    _check(lib().flce_fused_workspace_size(N, H, V, ctypes.byref(opt), chunk_tokens,
                                           ctypes.byref(b)), "flce_fused_workspace_size")
    return b.value


def flce_forward_backward(hidden, weight, labels, N, H, V, opt, chunk_tokens, grad_logprob,
                          grad_entropy, grad_uniform_ce, grad_z_loss, lse, logprob, entropy,
                          uniform_ce, z_loss, reduced, grad_hidden, grad_weight, workspace,
                          workspace_bytes, stream):
    _check(lib().flce_forward_backward(hidden, weight, labels, N, H, V, ctypes.byref(opt),
                                       chunk_tokens, grad_logprob, grad_entropy, grad_uniform_ce,
                                       grad_z_loss, lse, logprob, entropy, uniform_ce, z_loss,
                                       reduced, grad_hidden, grad_weight, workspace,
                                       workspace_bytes, stream), "flce_forward_backward")


def flce_forward_shard(hidden, weight_shard, labels, N, H, Vs, v_begin, V_total, opt, state,
                       label_logit, workspace, workspace_bytes, stream):
    _check(lib().flce_forward_shard(hidden, weight_shard, labels, N, H, Vs, v_begin, V_total,
                                    ctypes.byref(opt), state, label_logit, workspace,
                                    workspace_bytes, stream), "flce_forward_shard")


def flce_merge_workspace_size(N: int) -> int:
    b = ctypes.c_size_t(0)
    _check(lib().flce_merge_workspace_size(N, ctypes.byref(b)), "flce_merge_workspace_size")
    return b.value


def flce_merge_shards(states, label_logits, S, labels, N, V_total, opt, lse, logprob, entropy,
                      uniform_ce, z_loss, reduced, workspace, workspace_bytes, stream):
    _check(lib().flce_merge_shards(states, label_logits, S, labels, N, V_total, ctypes.byref(opt),
                                   lse, logprob, entropy, uniform_ce, z_loss, reduced, workspace,
                                   workspace_bytes, stream), "flce_merge_shards")


def flce_backward_shard(hidden, weight_shard, labels, N, H, Vs, v_begin, V_total, opt, lse,
                        entropy, grad_logprob, grad_entropy, grad_uniform_ce, grad_z_loss,
                        grad_hidden_partial, grad_weight_shard, workspace, workspace_bytes,
                        stream):
    _check(lib().flce_backward_shard(hidden, weight_shard, labels, N, H, Vs, v_begin, V_total,
                                     ctypes.byref(opt), lse, entropy, grad_logprob, grad_entropy,
                                     grad_uniform_ce, grad_z_loss, grad_hidden_partial,
                                     grad_weight_shard, workspace, workspace_bytes, stream),
           "flce_backward_shard")


def flce_get_status(workspace, stream) -> int:
    """Number of invalid labels the last call on this workspace saw (syncs)."""
    n = _I64(0)
    st = lib().flce_get_status(workspace, ctypes.byref(n), stream)
    if st not in (0, 8):
        _check(st, "flce_get_status")
    return n.value


def flce_status_string(status: int) -> str:
    return lib().flce_status_string(status).decode()


def flce_version() -> int:
    return lib().flce_version()


def flce_profile_enable(enable: bool) -> None:
    _check(lib().flce_profile_enable(1 if enable else 0), "flce_profile_enable")


def flce_profile_reset() -> None:
    _check(lib().flce_profile_reset(), "flce_profile_reset")


def flce_profile_kinds() -> int:
    return lib().flce_profile_kinds()


def flce_profile_read(kind: int):
    name = ctypes.c_char_p()
    n = _I64(0)
    ms = ctypes.c_double(0.0)
    _check(lib().flce_profile_read(kind, ctypes.byref(name), ctypes.byref(n), ctypes.byref(ms)),
           "flce_profile_read")
    return name.value.decode(), n.value, ms.value


PROBE_REGISTERS, PROBE_ZEROS, PROBE_LDS, PROBE_LDS_DMA = 0, 1, 2, 3


def flce_probe_mfma_rate(mode, steps: int, workspace, workspace_bytes, stream) -> float:
    """Sustained bf16 MFMA TFLOP/s of the GEMM wave tile (synchronises the
    stream). mode: PROBE_REGISTERS (or False), PROBE_ZEROS (or True),
    PROBE_LDS, PROBE_LDS_DMA; see include/flce.h."""
    t = ctypes.c_double(0.0)
    _check(lib().flce_probe_mfma_rate(int(mode), steps, ctypes.byref(t), workspace,
                                      workspace_bytes, stream), "flce_probe_mfma_rate")
    return t.value


def profile_table() -> dict:
    """{kernel kind: (launches, total ms)} for kinds launched at least once."""
    out = {}
    for k in range(flce_profile_kinds()):
        name, n, ms = flce_profile_read(k)
        if n:
            out[name] = (n, ms)
    return out


# ---------------------------------------------------------------- torch marshalling

def _torch():
    import torch
    return torch


def _stream():
    return _torch().cuda.current_stream().cuda_stream


def _require(t, dtype, ndim, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {ndim}-d tensor")


def check_shapes(hidden, weight, labels, *per_token) -> None:
    """Raises ValueError unless hidden [N,H], weight [H,V], labels [N] and
    each (name, tensor) pair of ``per_token`` ([N] each; None skipped) agree
    in size: the kernels read them by those extents."""
    N, H = hidden.shape
    if weight.dim() != 2 or weight.shape[0] != H or labels.shape[0] != N:
        raise ValueError("shape mismatch among hidden [N,H], weight [H,V], labels [N]")
    for name, t in per_token:
        if t is not None and (t.dim() != 1 or t.shape[0] != N):
            raise ValueError(f"{name} must have N = {N} elements")


def _entropy_per_token(reduction: str, entropy_reduction) -> int:
    if entropy_reduction is None or entropy_reduction == reduction:
        return 0
    if entropy_reduction != "none":
        raise ValueError("entropy_reduction must be None, 'none' or the reduction itself")
    return 1


def workspace_bytes(N: int, H: int, V: int, reduction: str = "none"):
    return flce_workspace_size(N, H, V, _REDUCTIONS[reduction])


_OUT_NAMES = ("logprob", "entropy", "uniform_ce", "z_loss")


def _ptr(t):
    return t.data_ptr() if t is not None else None


def _check_class_weight(cw, V):
    if cw is not None:
        _require(cw, _torch().float32, 1, "class_weight")
        if cw.shape[0] != V:
            raise ValueError("class_weight must have one weight per class (V)")


def forward(hidden, weight, labels, ignore_index: int = -100, softcap: float = 0.0,
            reduction: str = "none", z_loss_scale: float = 0.0, aux: bool = False,
            class_weight=None, workspace=None) -> dict:
    """lse, logprob, entropy [N] (fp32); with ``aux`` also uniform_ce and
    z_loss [N]; under "mean" / "sum" the reductions as ``<name>_mean`` /
    ``<name>_sum`` (fp32 [1]).

    hidden: bf16 [N,H]; weight: bf16 [H,V]; labels: int64 [N];
    class_weight: optional fp32 [V] target weights of the "mean" / "sum"
    reductions. Without aux, z-loss, "sum" and class weights this calls
    flce_forward, else flce_forward_ex.
    """
    torch = _torch()
    _require(hidden, torch.bfloat16, 2, "hidden")
    _require(weight, torch.bfloat16, 2, "weight")
    _require(labels, torch.int64, 1, "labels")
    check_shapes(hidden, weight, labels)
    N, H = hidden.shape
    V = weight.shape[1]
    red = _REDUCTIONS[reduction]
    fbytes, _ = flce_workspace_size(N, H, V, red)
    if workspace is None or workspace.numel() < fbytes:
        workspace = torch.empty(max(fbytes, 256), dtype=torch.uint8, device=hidden.device)
    dev = hidden.device
    f32 = dict(dtype=torch.float32, device=dev)
    lse = torch.empty(N, **f32)
    lp = torch.empty(N, **f32)
    ent = torch.empty(N, **f32)
    out = {"lse": lse, "logprob": lp, "entropy": ent, "workspace": workspace}
    _check_class_weight(class_weight, V)
    extended = aux or z_loss_scale != 0.0 or red == FLCE_REDUCTION_SUM or class_weight is not None
    if not extended:
        lpm = entm = None
        if red == FLCE_REDUCTION_MEAN:
            lpm = torch.empty(1, **f32)
            entm = torch.empty(1, **f32)
            out["logprob_mean"] = lpm
            out["entropy_mean"] = entm
        flce_forward(hidden.data_ptr(), weight.data_ptr(), labels.data_ptr(), N, H, V,
                     int(ignore_index), float(softcap), red, lse.data_ptr(), lp.data_ptr(),
                     ent.data_ptr(), _ptr(lpm), _ptr(entm), workspace.data_ptr(),
                     workspace.numel(), _stream())
        return out
    uce = torch.empty(N, **f32) if aux else None
    zl = torch.empty(N, **f32) if aux else None
    reduced = torch.empty(4, **f32) if red != FLCE_REDUCTION_NONE else None
    opt = FlceOptions(int(ignore_index), float(softcap), red, float(z_loss_scale), FLCE_GRAD_BF16,
                      _ptr(class_weight))
    flce_forward_ex(hidden.data_ptr(), weight.data_ptr(), labels.data_ptr(), N, H, V, opt,
                    lse.data_ptr(), lp.data_ptr(), ent.data_ptr(), _ptr(uce), _ptr(zl),
                    _ptr(reduced), workspace.data_ptr(), workspace.numel(), _stream())
    if aux:
        out["uniform_ce"] = uce
        out["z_loss"] = zl
    if reduced is not None:
        for k, name in enumerate(_OUT_NAMES):
            out[f"{name}_{reduction}"] = reduced[k:k + 1]
    return out


def _check_grads(grads, N, red, reduction, ept):
    torch = _torch()
    for g, name in grads:
        if g is not None:
            _require(g, torch.float32, 1, name)
            want = N if (red == FLCE_REDUCTION_NONE or (ept and name == "grad_entropy")) else 1
            if g.shape[0] != want:
                raise ValueError(f"{name} must have {want} element(s) under '{reduction}'")


def backward(hidden, weight, labels, lse, entropy, grad_logprob=None, grad_entropy=None,
             ignore_index: int = -100, softcap: float = 0.0, reduction: str = "none",
             grad_uniform_ce=None, grad_z_loss=None, z_loss_scale: float = 0.0,
             grad_dtype: str = "bf16", class_weight=None, entropy_reduction=None,
             workspace=None):
    """(grad_hidden [N,H], grad_weight [H,V]), bf16 or fp32 (``grad_dtype``).

    Upstream gradients: fp32 [N] under "none", fp32 [1] under "mean" and
    "sum", or None for zero; with ``entropy_reduction="none"`` under "mean" /
    "sum" the entropy's gradient is per token [N] (the entropy taken
    unreduced beside the reduced logprob; options field entropy_per_token).
    class_weight as for ``forward``. Without the auxiliary gradients, z-loss,
    "sum", class weights, a per-token entropy and fp32 outputs this calls
    flce_backward, else flce_backward_ex.
    """
    torch = _torch()
    _require(hidden, torch.bfloat16, 2, "hidden")
    _require(weight, torch.bfloat16, 2, "weight")
    _require(labels, torch.int64, 1, "labels")
    _require(lse, torch.float32, 1, "lse")
    _require(entropy, torch.float32, 1, "entropy")
    check_shapes(hidden, weight, labels, ("lse", lse), ("entropy", entropy))
    N, H = hidden.shape
    V = weight.shape[1]
    red = _REDUCTIONS[reduction]
    gdt = _GRAD_DTYPES[grad_dtype]
    ept = _entropy_per_token(reduction, entropy_reduction)
    grads = ((grad_logprob, "grad_logprob"), (grad_entropy, "grad_entropy"),
             (grad_uniform_ce, "grad_uniform_ce"), (grad_z_loss, "grad_z_loss"))
    _check_grads(grads, N, red, reduction, ept)
    _, bbytes = flce_workspace_size(N, H, V, red)
    if workspace is None or workspace.numel() < bbytes:
        workspace = torch.empty(max(bbytes, 256), dtype=torch.uint8, device=hidden.device)
    odt = torch.float32 if gdt == FLCE_GRAD_F32 else torch.bfloat16
    gh = torch.empty((N, H), dtype=odt, device=hidden.device)
    gw = torch.empty((H, V), dtype=odt, device=hidden.device)
    _check_class_weight(class_weight, V)
    extended = (grad_uniform_ce is not None or grad_z_loss is not None or z_loss_scale != 0.0
                or red == FLCE_REDUCTION_SUM or gdt != FLCE_GRAD_BF16 or class_weight is not None
                or ept)
    if not extended:
        flce_backward(hidden.data_ptr(), weight.data_ptr(), labels.data_ptr(), N, H, V,
                      int(ignore_index), float(softcap), red, lse.data_ptr(), entropy.data_ptr(),
                      _ptr(grad_logprob), _ptr(grad_entropy), gh.data_ptr(), gw.data_ptr(),
                      workspace.data_ptr(), workspace.numel(), _stream())
        return gh, gw
    opt = FlceOptions(int(ignore_index), float(softcap), red, float(z_loss_scale), gdt,
                      _ptr(class_weight), ept)
    flce_backward_ex(hidden.data_ptr(), weight.data_ptr(), labels.data_ptr(), N, H, V, opt,
                     lse.data_ptr(), entropy.data_ptr(), _ptr(grad_logprob), _ptr(grad_entropy),
                     _ptr(grad_uniform_ce), _ptr(grad_z_loss), gh.data_ptr(), gw.data_ptr(),
                     workspace.data_ptr(), workspace.numel(), _stream())
    return gh, gw


def forward_backward(hidden, weight, labels, grad_logprob=None, grad_entropy=None,
                     ignore_index: int = -100, softcap: float = 0.0, reduction: str = "none",
                     grad_uniform_ce=None, grad_z_loss=None, z_loss_scale: float = 0.0,
                     grad_dtype: str = "bf16", aux: bool = False, chunk_tokens: int = 0,
                     class_weight=None, entropy_reduction=None, workspace=None) -> dict:
    """The fused forward + backward (flce_forward_backward): the outputs of
    ``forward`` and, under "grad_hidden" / "grad_weight", the gradients of
    ``backward`` for upstream gradients known before the call (fp32 [N] under
    "none", [1] under "mean" and "sum", None for zero; entropy_reduction as
    for ``backward``).
    """
    torch = _torch()
    _require(hidden, torch.bfloat16, 2, "hidden")
    _require(weight, torch.bfloat16, 2, "weight")
    _require(labels, torch.int64, 1, "labels")
    check_shapes(hidden, weight, labels)
    N, H = hidden.shape
    V = weight.shape[1]
    red = _REDUCTIONS[reduction]
    gdt = _GRAD_DTYPES[grad_dtype]
    ept = _entropy_per_token(reduction, entropy_reduction)
    grads = ((grad_logprob, "grad_logprob"), (grad_entropy, "grad_entropy"),
             (grad_uniform_ce, "grad_uniform_ce"), (grad_z_loss, "grad_z_loss"))
    _check_grads(grads, N, red, reduction, ept)
    _check_class_weight(class_weight, V)
    opt = FlceOptions(int(ignore_index), float(softcap), red, float(z_loss_scale), gdt,
                      _ptr(class_weight), ept)
    nbytes = flce_fused_workspace_size(N, H, V, opt, int(chunk_tokens))
    if workspace is None or workspace.numel() < nbytes:
        workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=hidden.device)
    dev = hidden.device
    f32 = dict(dtype=torch.float32, device=dev)
    odt = torch.float32 if gdt == FLCE_GRAD_F32 else torch.bfloat16
    out = {"lse": torch.empty(N, **f32), "logprob": torch.empty(N, **f32),
           "entropy": torch.empty(N, **f32), "workspace": workspace,
           "grad_hidden": torch.empty((N, H), dtype=odt, device=dev),
           "grad_weight": torch.empty((H, V), dtype=odt, device=dev)}
    uce = torch.empty(N, **f32) if aux else None
    zl = torch.empty(N, **f32) if aux else None
    reduced = torch.empty(4, **f32) if red != FLCE_REDUCTION_NONE else None
    flce_forward_backward(hidden.data_ptr(), weight.data_ptr(), labels.data_ptr(), N, H, V, opt,
                          int(chunk_tokens), _ptr(grad_logprob), _ptr(grad_entropy),
                          _ptr(grad_uniform_ce), _ptr(grad_z_loss), out["lse"].data_ptr(),
                          out["logprob"].data_ptr(), out["entropy"].data_ptr(), _ptr(uce),
                          _ptr(zl), _ptr(reduced), out["grad_hidden"].data_ptr(),
                          out["grad_weight"].data_ptr(), workspace.data_ptr(), workspace.numel(),
                          _stream())
    if aux:
        out["uniform_ce"] = uce
        out["z_loss"] = zl
    if reduced is not None:
        for k, name in enumerate(_OUT_NAMES):
            out[f"{name}_{reduction}"] = reduced[k:k + 1]
    return out
