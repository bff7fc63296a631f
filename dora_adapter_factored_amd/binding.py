"""Thin Python binding of libdora_mi355x.so (ctypes).

Argument marshalling only: every step of the computation runs in the HIP
library.  torch provides device memory (outputs, workspace) and the current
stream.  Each function checks what the C ABI cannot see (device, dtype,
contiguity, shapes), passes raw pointers, and raises on a non-OK status.
There is no fallback path: without the built library every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdora_mi355x.so")

DORA_OK, DORA_ERR_INVALID_ARG, DORA_ERR_UNSUPPORTED, DORA_ERR_WORKSPACE, DORA_ERR_HIP = range(5)
_DTYPE_CODE = {torch.float32: 0, torch.bfloat16: 1, torch.float16: 2}

_lib = None
_lib_lock = threading.Lock()

# C entry points and their signatures, as declared in include/dora.h.
_i64, _f32, _vp, _sz = ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
class NormMember(ctypes.Structure):
    """DoraNormMember of include/dora.h."""
    _fields_ = [("W0", ctypes.c_void_p), ("A", ctypes.c_void_p), ("B", ctypes.c_void_p), ("m", ctypes.c_void_p),
                ("wnorm", ctypes.c_void_p), ("g", ctypes.c_void_p), ("d_out", ctypes.c_int64), ("d_in", ctypes.c_int64),
                ("s", ctypes.c_float)]


MAX_NORM_GROUP = 8

_SIGNATURES = {
    "dora_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "dora_last_error_detail": (ctypes.c_char_p, []),
    "dora_version": (ctypes.c_int, []),
    "dora_factored_norm_workspace_size": (ctypes.c_int, [_i64, _i64, _i64, ctypes.c_int, ctypes.POINTER(_sz)]),
    "dora_factored_norm": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, ctypes.c_int, _f32, _f32,
                                          _vp, _vp, _vp, _sz, _vp]),
    "dora_factored_norm_noalloc": (ctypes.c_int, [_vp, _vp, _vp, _vp, _i64, _i64, _i64, ctypes.c_int, _f32, _f32,
                                                  _vp, _vp, _vp]),
    "dora_compose": (ctypes.c_int, [_vp, _vp, _vp, _f32, _i64, _i64, ctypes.c_int, ctypes.c_int, _vp, _vp]),
    "dora_compose_backward_workspace_size": (ctypes.c_int, [_i64, _i64, ctypes.POINTER(_sz)]),
    "dora_compose_backward": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _f32, _f32, _i64, _i64, ctypes.c_int,
                                             ctypes.c_int, _vp, _vp, _vp, _vp, _sz, _vp]),
    "dora_factored_norm_group_workspace_size": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(_i64),
                                                               ctypes.POINTER(_i64), _i64, ctypes.c_int,
                                                               ctypes.POINTER(_sz)]),
    "dora_factored_norm_group": (ctypes.c_int, [ctypes.c_int, ctypes.POINTER(NormMember), _i64, ctypes.c_int,
                                                _f32, _vp, _sz, _vp]),
    "dora_merge_workspace_size": (ctypes.c_int, [_i64, _i64, ctypes.c_int, ctypes.POINTER(_sz)]),
    "dora_merge": (ctypes.c_int, [_vp, _vp, _vp, _vp, _f32, _i64, _i64, _i64, ctypes.c_int, _vp, _vp, _sz, _vp]),
    "dora_compose_dual": (ctypes.c_int, [_vp, _vp, _vp, _f32, _i64, _i64, ctypes.c_int, ctypes.c_int, _vp, _vp,
                                         _vp]),
    "dora_compose_backward_inner": (ctypes.c_int, [_vp, _vp, _vp, _vp, _f32, _f32, _i64, _i64, ctypes.c_int,
                                                   ctypes.c_int, _vp, _vp, _vp, _vp, _sz, _vp]),
}
EXPORTED = tuple(_SIGNATURES)


class DoraError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load()
        msg = lib.dora_status_string(status).decode()
        detail = lib.dora_last_error_detail().decode()
        super().__init__(f"{where}: {msg}" + (f" ({detail})" if detail else ""))
        self.status = status


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load the shared library (once).  Raises ImportError if it is not built."""
    global _lib
    if _lib is None:
        with _lib_lock:
            if _lib is None:
                if not os.path.exists(_LIB_PATH):
                    raise ImportError(f"{_LIB_PATH} is not built; run `python -m dora_adapter_factored_amd.build`")
                lib = ctypes.CDLL(_LIB_PATH)
                for name, (res, args) in _SIGNATURES.items():
                    fn = getattr(lib, name)
                    fn.restype = res
                    fn.argtypes = args
                _lib = lib
    return _lib


def _check(status: int, where: str):
    if status != DORA_OK:
        raise DoraError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, name: str, device, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def default_eps(dtype: torch.dtype) -> float:
    """Clamp of the magnitude division: the machine epsilon of the input dtype."""
    return float(torch.finfo(dtype).eps)


# ------------------------------------------------------------ workspaces
_ws_cache: dict = {}


def workspace(nbytes: int, device) -> torch.Tensor | None:
    """A cached uint8 device buffer of at least nbytes for (device, current stream).

    Calls on one stream are ordered, so reusing the buffer across them is safe.
    """
    if nbytes == 0:
        return None
    key = (device, torch.cuda.current_stream(device).cuda_stream)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return buf


def norm_workspace_size(d_out: int, d_in: int, r: int, dtype: torch.dtype) -> int:
    n = ctypes.c_size_t(0)
    _check(load().dora_factored_norm_workspace_size(d_out, d_in, r, _DTYPE_CODE[dtype], ctypes.byref(n)),
           "dora_factored_norm_workspace_size")
    return n.value


def compose_backward_workspace_size(T: int, d_out: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().dora_compose_backward_workspace_size(T, d_out, ctypes.byref(n)),
           "dora_compose_backward_workspace_size")
    return n.value


def norm_group_workspace_size(d_outs, d_ins, r: int, dtype: torch.dtype) -> int:
    """Workspace of a grouped norm whose member j is [d_outs[j], d_ins[j]]."""
    if len(d_outs) != len(d_ins):
        raise ValueError("d_outs and d_ins must have one entry per member")
    n = ctypes.c_size_t(0)
    outs = (_i64 * len(d_outs))(*[int(d) for d in d_outs])
    ins = (_i64 * len(d_ins))(*[int(d) for d in d_ins])
    _check(load().dora_factored_norm_group_workspace_size(len(d_outs), outs, ins, r, _DTYPE_CODE[dtype],
                                                           ctypes.byref(n)),
           "dora_factored_norm_group_workspace_size")
    return n.value


def merge_workspace_size(d_in: int, r: int, dtype: torch.dtype) -> int:
    n = ctypes.c_size_t(0)
    _check(load().dora_merge_workspace_size(d_in, r, _DTYPE_CODE[dtype], ctypes.byref(n)),
           "dora_merge_workspace_size")
    return n.value


# ------------------------------------------------------------ entry points
def factored_norm(W0, A, B, s: float, m=None, eps: float | None = None, *, wnorm=None, g=None, ws=None):
    """wnorm = ||W0_i + s (BA)_i|| (factored, never forming BA) and g = m / max(wnorm, eps).

    W0 [d_out, d_in], A [r, d_in], B [d_out, r] share a dtype (bf16 or fp32);
    m is fp32 [d_out] or None.  Returns (wnorm, g) with g None when m is None.
    """
    lib = load()
    dev = W0.device
    d_out, d_in = W0.shape
    r = A.shape[0]
    _need(W0, "W0", dev)
    _need(A, "A", dev, W0.dtype, (r, d_in))
    _need(B, "B", dev, W0.dtype, (d_out, r))
    if m is not None:
        _need(m, "m", dev, torch.float32, (d_out,))
    if W0.dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported dtype {W0.dtype}")
    eps = default_eps(W0.dtype) if eps is None else float(eps)
    if wnorm is None:
        wnorm = torch.empty(d_out, dtype=torch.float32, device=dev)
    _need(wnorm, "wnorm", dev, torch.float32, (d_out,))
    if m is not None and g is None:
        g = torch.empty(d_out, dtype=torch.float32, device=dev)
    if g is not None:
        _need(g, "g", dev, torch.float32, (d_out,))
    if ws is None:
        ws = workspace(norm_workspace_size(d_out, d_in, r, W0.dtype), dev)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.dora_factored_norm(_ptr(W0), _ptr(A), _ptr(B), _ptr(m), d_out, d_in, r, _DTYPE_CODE[W0.dtype],
                                  float(s), eps, _ptr(wnorm), _ptr(g), _ptr(ws), nbytes, _stream(dev)),
           "dora_factored_norm")
    return wnorm, (g if m is not None else None)


def factored_norm_noalloc(W0, A, B, s: float, m=None, eps: float | None = None, *, wnorm=None, g=None):
    """factored_norm through dora_factored_norm_noalloc: no workspace, the
    library's static per-GPU scratch instead (same kernels, bitwise the same
    result).  Outputs are allocated here unless given."""
    lib = load()
    dev = W0.device
    d_out, d_in = W0.shape
    r = A.shape[0]
    _need(W0, "W0", dev)
    _need(A, "A", dev, W0.dtype, (r, d_in))
    _need(B, "B", dev, W0.dtype, (d_out, r))
    if m is not None:
        _need(m, "m", dev, torch.float32, (d_out,))
    if W0.dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported dtype {W0.dtype}")
    eps = default_eps(W0.dtype) if eps is None else float(eps)
    if wnorm is None:
        wnorm = torch.empty(d_out, dtype=torch.float32, device=dev)
    _need(wnorm, "wnorm", dev, torch.float32, (d_out,))
    if m is not None and g is None:
        g = torch.empty(d_out, dtype=torch.float32, device=dev)
    if g is not None:
        _need(g, "g", dev, torch.float32, (d_out,))
    with torch.cuda.device(dev):
        _check(lib.dora_factored_norm_noalloc(_ptr(W0), _ptr(A), _ptr(B), _ptr(m), d_out, d_in, r,
                                              _DTYPE_CODE[W0.dtype], float(s), eps, _ptr(wnorm), _ptr(g),
                                              _stream(dev)),
               "dora_factored_norm_noalloc")
    return wnorm, (g if m is not None else None)


def factored_norm_group(members, eps: float | None = None, *, outs=None, ws=None):
    """Factored norms of several projections sharing r and the dtype in one call.

    members: sequence of (W0, A, B, s, m) with m fp32 [d_out] or None; each
    member has its own [d_out, d_in].  Returns a list of (wnorm, g) per
    member, g None where m is None; each equals factored_norm's result for
    that member bitwise.
    """
    lib = load()
    n = len(members)
    if not 1 <= n <= MAX_NORM_GROUP:
        raise ValueError(f"a group holds 1..{MAX_NORM_GROUP} members (got {n})")
    W0_0, A_0 = members[0][0], members[0][1]
    dev, dt = W0_0.device, W0_0.dtype
    r = A_0.shape[0]
    if dt not in _DTYPE_CODE:
        raise ValueError(f"unsupported dtype {dt}")
    eps = default_eps(dt) if eps is None else float(eps)
    arr = (NormMember * n)()
    results = []
    for j, (W0, A, B, s, m) in enumerate(members):
        d_out, d_in = W0.shape
        _need(W0, f"W0[{j}]", dev, dt, (d_out, d_in))
        _need(A, f"A[{j}]", dev, dt, (r, d_in))
        _need(B, f"B[{j}]", dev, dt, (d_out, r))
        if m is not None:
            _need(m, f"m[{j}]", dev, torch.float32, (d_out,))
        if outs is not None:
            wnorm, g = outs[j]
        else:
            wnorm = torch.empty(d_out, dtype=torch.float32, device=dev)
            g = torch.empty(d_out, dtype=torch.float32, device=dev) if m is not None else None
        _need(wnorm, f"wnorm[{j}]", dev, torch.float32, (d_out,))
        if m is not None:
            _need(g, f"g[{j}]", dev, torch.float32, (d_out,))
        arr[j] = NormMember(_ptr(W0), _ptr(A), _ptr(B), _ptr(m), _ptr(wnorm), _ptr(g) if m is not None else None,
                            d_out, d_in, float(s))
        results.append((wnorm, g if m is not None else None))
    if ws is None:
        ws = workspace(norm_group_workspace_size([mb[0].shape[0] for mb in members],
                                                 [mb[0].shape[1] for mb in members], r, dt), dev)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.dora_factored_norm_group(n, arr, r, _DTYPE_CODE[dt], eps, _ptr(ws), nbytes, _stream(dev)),
           "dora_factored_norm_group")
    return results


def merge(W0, A, B, g, s: float, *, out=None, ws=None):
    """W = diag(g) (W0 + s B A), the adapter folded into one weight for serving.

    g is fp32 [d_out] (the g of factored_norm).  out=W0 merges in place.
    """
    lib = load()
    dev = W0.device
    d_out, d_in = W0.shape
    r = A.shape[0]
    _need(W0, "W0", dev)
    _need(A, "A", dev, W0.dtype, (r, d_in))
    _need(B, "B", dev, W0.dtype, (d_out, r))
    _need(g, "g", dev, torch.float32, (d_out,))
    if W0.dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported dtype {W0.dtype}")
    if out is None:
        out = torch.empty_like(W0)
    _need(out, "out", dev, W0.dtype, (d_out, d_in))
    if ws is None:
        ws = workspace(merge_workspace_size(d_in, r, W0.dtype), dev)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.dora_merge(_ptr(W0), _ptr(A), _ptr(B), _ptr(g), float(s), d_out, d_in, r, _DTYPE_CODE[W0.dtype],
                          _ptr(out), _ptr(ws), nbytes, _stream(dev)),
           "dora_merge")
    return out


def compose(base_out, lora_out, g, s: float, delta_only: bool = False, *, out=None):
    """y = base + ((g-1)*base + (g*s)*lora) (or the delta alone), one fused pass."""
    lib = load()
    dev = base_out.device
    T, d_out = base_out.shape
    _need(base_out, "base_out", dev)
    _need(lora_out, "lora_out", dev, base_out.dtype, (T, d_out))
    _need(g, "g", dev, torch.float32, (d_out,))
    if base_out.dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported dtype {base_out.dtype}")
    if out is None:
        out = torch.empty_like(base_out)
    _need(out, "out", dev, base_out.dtype, (T, d_out))
    _check(lib.dora_compose(_ptr(base_out), _ptr(lora_out), _ptr(g), float(s), T, d_out,
                            _DTYPE_CODE[base_out.dtype], int(bool(delta_only)), _ptr(out), _stream(dev)),
           "dora_compose")
    return out


def compose_backward(dy, base_out, lora_out, g, wnorm, s: float, eps: float | None = None,
                     delta_only: bool = False, *, need_d_base=True, need_d_lora=True, need_d_m=True,
                     d_base=None, d_lora=None, d_m=None, ws=None):
    """(d_base, d_lora, d_m) of compose with the norm detached; unrequested ones are None."""
    lib = load()
    dev = dy.device
    T, d_out = dy.shape
    _need(dy, "dy", dev)
    if dy.dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported dtype {dy.dtype}")
    _need(g, "g", dev, torch.float32, (d_out,))
    if need_d_m:
        _need(base_out, "base_out", dev, dy.dtype, (T, d_out))
        _need(lora_out, "lora_out", dev, dy.dtype, (T, d_out))
        _need(wnorm, "wnorm", dev, torch.float32, (d_out,))
    eps = default_eps(dy.dtype) if eps is None else float(eps)
    if need_d_base and d_base is None:
        d_base = torch.empty_like(dy)
    if need_d_lora and d_lora is None:
        d_lora = torch.empty_like(dy)
    if need_d_m and d_m is None:
        d_m = torch.empty(d_out, dtype=torch.float32, device=dev)
    for t, name in ((d_base, "d_base"), (d_lora, "d_lora")):
        if t is not None:
            _need(t, name, dev, dy.dtype, (T, d_out))
    if d_m is not None:
        _need(d_m, "d_m", dev, torch.float32, (d_out,))
    if need_d_m and ws is None:
        ws = workspace(compose_backward_workspace_size(T, d_out), dev)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.dora_compose_backward(_ptr(dy), _ptr(base_out) if need_d_m else None,
                                     _ptr(lora_out) if need_d_m else None, _ptr(g),
                                     _ptr(wnorm) if need_d_m else None, float(s), eps, T, d_out,
                                     _DTYPE_CODE[dy.dtype], int(bool(delta_only)),
                                     _ptr(d_base) if need_d_base else None,
                                     _ptr(d_lora) if need_d_lora else None,
                                     _ptr(d_m) if need_d_m else None, _ptr(ws), nbytes, _stream(dev)),
           "dora_compose_backward")
    return (d_base if need_d_base else None, d_lora if need_d_lora else None, d_m if need_d_m else None)


def compose_dual(base_out, lora_out, g, s: float, delta_only: bool = False, *, out=None, inner=None):
    """(y, inner): the compose output and inner = base + s*lora from one pass."""
    lib = load()
    dev = base_out.device
    T, d_out = base_out.shape
    _need(base_out, "base_out", dev)
    _need(lora_out, "lora_out", dev, base_out.dtype, (T, d_out))
    _need(g, "g", dev, torch.float32, (d_out,))
    if base_out.dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported dtype {base_out.dtype}")
    if out is None:
        out = torch.empty_like(base_out)
    if inner is None:
        inner = torch.empty_like(base_out)
    _need(out, "out", dev, base_out.dtype, (T, d_out))
    _need(inner, "inner", dev, base_out.dtype, (T, d_out))
    _check(lib.dora_compose_dual(_ptr(base_out), _ptr(lora_out), _ptr(g), float(s), T, d_out,
                                 _DTYPE_CODE[base_out.dtype], int(bool(delta_only)), _ptr(out), _ptr(inner),
                                 _stream(dev)),
           "dora_compose_dual")
    return out, inner


def compose_backward_inner(dy, inner, g, wnorm, s: float, eps: float | None = None, delta_only: bool = False, *,
                           need_d_base=True, need_d_lora=True, need_d_m=True, d_base=None, d_lora=None, d_m=None,
                           ws=None):
    """(d_base, d_lora, d_m) from (dy, inner) with the norm detached; unrequested ones are None."""
    lib = load()
    dev = dy.device
    T, d_out = dy.shape
    _need(dy, "dy", dev)
    if dy.dtype not in _DTYPE_CODE:
        raise ValueError(f"unsupported dtype {dy.dtype}")
    _need(g, "g", dev, torch.float32, (d_out,))
    if need_d_m:
        _need(inner, "inner", dev, dy.dtype, (T, d_out))
        _need(wnorm, "wnorm", dev, torch.float32, (d_out,))
    eps = default_eps(dy.dtype) if eps is None else float(eps)
    if need_d_base and d_base is None:
        d_base = torch.empty_like(dy)
    if need_d_lora and d_lora is None:
        d_lora = torch.empty_like(dy)
    if need_d_m and d_m is None:
        d_m = torch.empty(d_out, dtype=torch.float32, device=dev)
    for t, name in ((d_base, "d_base"), (d_lora, "d_lora")):
        if t is not None:
            _need(t, name, dev, dy.dtype, (T, d_out))
    if d_m is not None:
        _need(d_m, "d_m", dev, torch.float32, (d_out,))
    if need_d_m and ws is None:
        ws = workspace(compose_backward_workspace_size(T, d_out), dev)
    nbytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib.dora_compose_backward_inner(_ptr(dy), _ptr(inner) if need_d_m else None, _ptr(g),
                                           _ptr(wnorm) if need_d_m else None, float(s), eps, T, d_out,
                                           _DTYPE_CODE[dy.dtype], int(bool(delta_only)),
                                           _ptr(d_base) if need_d_base else None,
                                           _ptr(d_lora) if need_d_lora else None,
                                           _ptr(d_m) if need_d_m else None, _ptr(ws), nbytes, _stream(dev)),
           "dora_compose_backward_inner")
    return (d_base if need_d_base else None, d_lora if need_d_lora else None, d_m if need_d_m else None)


class DoRACompose(torch.autograd.Function):
    """Autograd wiring of the fused compose: inputs (base_out, lora_out, m) with
    the norm wnorm detached; g = m / max(wnorm, eps) comes from factored_norm.

    forward(ctx, base_out, lora_out, m, g, wnorm, s, eps, delta_only)
    """

    @staticmethod
    def forward(ctx, base_out, lora_out, m, g, wnorm, s, eps, delta_only=False):
        ctx.save_for_backward(base_out, lora_out, g, wnorm)
        ctx.s, ctx.eps, ctx.delta_only = float(s), float(eps), bool(delta_only)
        ctx.need = (ctx.needs_input_grad[0], ctx.needs_input_grad[1], ctx.needs_input_grad[2])
        return compose(base_out, lora_out, g, s, delta_only)

    @staticmethod
    def backward(ctx, dy):
        base_out, lora_out, g, wnorm = ctx.saved_tensors
        nb, nl, nm = ctx.need
        d_base, d_lora, d_m = compose_backward(dy.contiguous(), base_out, lora_out, g, wnorm, ctx.s, ctx.eps,
                                               ctx.delta_only, need_d_base=nb, need_d_lora=nl, need_d_m=nm)
        return d_base, d_lora, d_m, None, None, None, None, None


class DoRAComposeInner(torch.autograd.Function):
    """Training-tier autograd wiring: the forward writes y and inner = base +
    s*lora in one pass and saves only inner (one activation instead of two);
    the backward reads (dy, inner).  Same inputs and norm treatment as
    DoRACompose.

    forward(ctx, base_out, lora_out, m, g, wnorm, s, eps, delta_only)
    """

    @staticmethod
    def forward(ctx, base_out, lora_out, m, g, wnorm, s, eps, delta_only=False):
        y, inner = compose_dual(base_out, lora_out, g, s, delta_only)
        ctx.save_for_backward(inner, g, wnorm)
        ctx.s, ctx.eps, ctx.delta_only = float(s), float(eps), bool(delta_only)
        ctx.need = (ctx.needs_input_grad[0], ctx.needs_input_grad[1], ctx.needs_input_grad[2])
        return y

    @staticmethod
    def backward(ctx, dy):
        inner, g, wnorm = ctx.saved_tensors
        nb, nl, nm = ctx.need
        d_base, d_lora, d_m = compose_backward_inner(dy.contiguous(), inner, g, wnorm, ctx.s, ctx.eps,
                                                     ctx.delta_only, need_d_base=nb, need_d_lora=nl, need_d_m=nm)
        return d_base, d_lora, d_m, None, None, None, None, None
