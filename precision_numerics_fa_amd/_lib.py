"""ctypes marshalling for libfa.so (argument checks and pointer passing only)."""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libfa.so"
_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float
_S = ctypes.c_size_t

_SIGNATURES = {
    "fa_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_fwd_diag": (_I, [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_bwd_workspace_bytes": (_S, [_I, _I, _I, _I, _I]),
    "fa_bwd": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _S, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_bwd_noalloc": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_bwd_dot": (_I, [_P, _P, _P, _I, _I, _I, _I, _P]),
    "fa_bwd_dkdv": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P]),
    "fa_bwd_dq": (_I, [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P]),
    "fa_bwd_grads": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _P]),
    "fa_fwd_ex": (_I, [_I, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_bwd_ex": (_I, [_I, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _S, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_fwd_split_workspace_bytes": (_S, [_I, _I, _I, _I, _I]),
    "fa_fwd_split": (_I, [_P, _P, _P, _P, _P, _I, _P, _S, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fa_base_ld": (_I, [_I]),
    "fa_base_workspace_bytes": (_S, [_I, _I, _I, _I, _I]),
    "fa_base_fwd": (_I, [_P, _P, _P, _P, _P, _P, _S, _I, _I, _I, _I, _I, _F, _P]),
    "fa_base_scores": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _F, _P]),
    "fa_base_softmax": (_I, [_P, _P, _P, _I, _I, _I, _I, _P]),
    "fa_base_pv": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _P]),
    "fa_mfma_probe": (ctypes.c_longlong, [_P, _I, _I, _P]),
    "fa_hbm_probe": (_I, [_P, _S, _P, _P]),
    "fa_issue_probe": (_I, [_I, _I, _P, _I, _I, _P]),
    "fa_status_string": (ctypes.c_char_p, [_I]),
    "fa_stabilize_params": (None, [ctypes.POINTER(_F)] * 3),
    "fa_stabilize_params_ex": (_I, [_I] + [ctypes.POINTER(_F)] * 3),
    "fa_fwd_tile": (None, [_I, ctypes.POINTER(_I), ctypes.POINTER(_I)]),
    "fa_version": (_I, []),
}


FA_BF16 = 0
FA_F16 = 1


class FAError(RuntimeError):
    """A C ABI call returned a non-zero status."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed with status {status}: {status_string(status)}")


def lib_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def load():
    """Load libfa.so (once) and declare the ABI signatures."""
    global _lib
    if _lib is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it with `python -m precision_numerics_fa_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load().fa_status_string(int(status)).decode()


def version() -> int:
    return int(load().fa_version())


def stabilize_params(dtype: int = 0) -> Tuple[float, float, float]:
    """(delta_min, delta_max, fold) of the shift rule for an element type
    (FA_BF16 = 0, FA_F16 = 1)."""
    a, b, c = _F(), _F(), _F()
    if dtype == 0:
        load().fa_stabilize_params(ctypes.byref(a), ctypes.byref(b), ctypes.byref(c))
    else:
        _call("fa_stabilize_params_ex", int(dtype), ctypes.byref(a), ctypes.byref(b), ctypes.byref(c))
    return a.value, b.value, c.value


def fwd_tile(d: int) -> Tuple[int, int]:
    q, k = _I(), _I()
    load().fa_fwd_tile(int(d), ctypes.byref(q), ctypes.byref(k))
    return q.value, k.value


def workspace_bytes(B: int, H: int, N: int, d: int, causal: bool) -> int:
    return int(load().fa_bwd_workspace_bytes(B, H, N, d, int(bool(causal))))


# ---------------------------------------------------------------- tensor plumbing

def _torch():
    import torch
    return torch


def _stream():
    torch = _torch()
    return _P(torch.cuda.current_stream().cuda_stream)


def _check(name, t, dtype, shape, device):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _ptr(t):
    return _P(t.data_ptr())


def _call(fn: str, *args):
    st = getattr(load(), fn)(*args)
    if st != 0:
        raise FAError(fn, st)


def _shape(q):
    if q.dim() != 4:
        raise ValueError("q must have shape (B, H, N, d)")
    return tuple(int(x) for x in q.shape)


def _scale(scale: Optional[float], d: int) -> float:
    s = 1.0 / math.sqrt(d) if scale is None else float(scale)
    return s


def fwd(q, k, v, causal: bool = False, scale: Optional[float] = None, stabilize: bool = False,
        out=None, lse=None):
    """Forward pass.  Returns (O bf16 (B,H,N,d), LSE fp32 (B,H,N))."""
    torch = _torch()
    B, H, N, d = _shape(q)
    dev = q.device
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check(n, t, torch.bfloat16, (B, H, N, d), dev)
    o = torch.empty_like(q) if out is None else out
    l = torch.empty((B, H, N), dtype=torch.float32, device=dev) if lse is None else lse
    _check("out", o, torch.bfloat16, (B, H, N, d), dev)
    _check("lse", l, torch.float32, (B, H, N), dev)
    _call("fa_fwd", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(l), B, H, N, d, int(bool(causal)),
          _scale(scale, d), int(bool(stabilize)), _stream())
    return o, l


def fwd_diag(q, k, v, causal: bool = False, scale: Optional[float] = None, stabilize: bool = False):
    """Forward pass that also returns, per row, whether the stabilised shift
    was applied at some key block (uint8 (B,H,N))."""
    torch = _torch()
    B, H, N, d = _shape(q)
    dev = q.device
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check(n, t, torch.bfloat16, (B, H, N, d), dev)
    o = torch.empty_like(q)
    l = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    flags = torch.empty((B, H, N), dtype=torch.uint8, device=dev)
    _call("fa_fwd_diag", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(l), _ptr(flags), B, H, N, d,
          int(bool(causal)), _scale(scale, d), int(bool(stabilize)), _stream())
    return o, l, flags


def fwd_split_workspace_bytes(B: int, H: int, N: int, d: int, splits: int) -> int:
    return int(load().fa_fwd_split_workspace_bytes(B, H, N, d, int(splits)))


def fwd_split(q, k, v, splits: int, causal: bool = False, scale: Optional[float] = None,
              stabilize: bool = False, workspace=None, out=None, lse=None):
    """Forward pass split over `splits` key ranges per query block (bf16).
    Returns (O, LSE) as fwd does."""
    torch = _torch()
    B, H, N, d = _shape(q)
    dev = q.device
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check(n, t, torch.bfloat16, (B, H, N, d), dev)
    need = fwd_split_workspace_bytes(B, H, N, d, splits)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    o = torch.empty_like(q) if out is None else out
    l = torch.empty((B, H, N), dtype=torch.float32, device=dev) if lse is None else lse
    _check("out", o, torch.bfloat16, (B, H, N, d), dev)
    _check("lse", l, torch.float32, (B, H, N), dev)
    _call("fa_fwd_split", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(l), int(splits), _ptr(workspace),
          workspace.numel() * workspace.element_size(), B, H, N, d, int(bool(causal)), _scale(scale, d),
          int(bool(stabilize)), _stream())
    return o, l


def bwd(q, k, v, o, do, lse, causal: bool = False, scale: Optional[float] = None,
        stabilize: bool = False, workspace=None):
    """Backward pass.  Returns (dQ, dK, dV), bf16 (B,H,N,d)."""
    torch = _torch()
    B, H, N, d = _shape(q)
    dev = q.device
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check(n, t, torch.bfloat16, (B, H, N, d), dev)
    _check("lse", lse, torch.float32, (B, H, N), dev)
    nbytes = workspace_bytes(B, H, N, d, causal)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    _call("fa_bwd", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
          _ptr(workspace), workspace.numel() * workspace.element_size(), B, H, N, d, int(bool(causal)),
          _scale(scale, d), int(bool(stabilize)), _stream())
    return dq, dk, dv


# Rows of D (B*H*N) the allocation-free backward's fixed scratch holds.
NOALLOC_MAX_ROWS = 4194304


def bwd_noalloc(q, k, v, o, do, lse, causal: bool = False, scale: Optional[float] = None,
                stabilize: bool = False, dq=None, dk=None, dv=None):
    """Backward pass through fa_bwd_noalloc: no workspace, D in the library's
    fixed per-device scratch (B*H*N <= NOALLOC_MAX_ROWS).  Calls that may
    overlap on one GPU race on that scratch.  Returns (dQ, dK, dV); pass
    preallocated dq, dk, dv to make the call allocate nothing at all."""
    torch = _torch()
    B, H, N, d = _shape(q)
    dev = q.device
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check(n, t, torch.bfloat16, (B, H, N, d), dev)
    _check("lse", lse, torch.float32, (B, H, N), dev)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for n, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        _check(n, t, torch.bfloat16, (B, H, N, d), dev)
    _call("fa_bwd_noalloc", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk),
          _ptr(dv), B, H, N, d, int(bool(causal)), _scale(scale, d), int(bool(stabilize)), _stream())
    return dq, dk, dv


def bwd_dot(o, do, dvec=None):
    """D = rowsum(dO * O) in fp32, (B,H,N)."""
    torch = _torch()
    B, H, N, d = _shape(o)
    _check("do", do, torch.bfloat16, (B, H, N, d), o.device)
    _check("o", o, torch.bfloat16, (B, H, N, d), o.device)
    dvec = torch.empty((B, H, N), dtype=torch.float32, device=o.device) if dvec is None else dvec
    _check("dvec", dvec, torch.float32, (B, H, N), o.device)
    _call("fa_bwd_dot", _ptr(o), _ptr(do), _ptr(dvec), B, H, N, d, _stream())
    return dvec


def bwd_dkdv(q, k, v, do, lse, dvec, causal: bool = False, scale: Optional[float] = None, dk=None, dv=None):
    torch = _torch()
    B, H, N, d = _shape(q)
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for n, t in (("q", q), ("k", k), ("v", v), ("do", do), ("dk", dk), ("dv", dv)):
        _check(n, t, torch.bfloat16, (B, H, N, d), q.device)
    _check("lse", lse, torch.float32, (B, H, N), q.device)
    _check("dvec", dvec, torch.float32, (B, H, N), q.device)
    _call("fa_bwd_dkdv", _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse), _ptr(dvec), _ptr(dk), _ptr(dv),
          B, H, N, d, int(bool(causal)), _scale(scale, d), _stream())
    return dk, dv


def bwd_grads(q, k, v, do, lse, dvec, causal: bool = False, scale: Optional[float] = None,
              dq=None, dk=None, dv=None):
    """dQ, dK, dV in one launch (what bwd runs after bwd_dot)."""
    torch = _torch()
    B, H, N, d = _shape(q)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for n, t in (("q", q), ("k", k), ("v", v), ("do", do), ("dq", dq), ("dk", dk), ("dv", dv)):
        _check(n, t, torch.bfloat16, (B, H, N, d), q.device)
    _check("lse", lse, torch.float32, (B, H, N), q.device)
    _check("dvec", dvec, torch.float32, (B, H, N), q.device)
    _call("fa_bwd_grads", _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse), _ptr(dvec), _ptr(dq), _ptr(dk),
          _ptr(dv), B, H, N, d, int(bool(causal)), _scale(scale, d), _stream())
    return dq, dk, dv


def bwd_dq(q, k, v, do, lse, dvec, causal: bool = False, scale: Optional[float] = None, dq=None):
    torch = _torch()
    B, H, N, d = _shape(q)
    dq = torch.empty_like(q) if dq is None else dq
    for n, t in (("q", q), ("k", k), ("v", v), ("do", do), ("dq", dq)):
        _check(n, t, torch.bfloat16, (B, H, N, d), q.device)
    _check("lse", lse, torch.float32, (B, H, N), q.device)
    _check("dvec", dvec, torch.float32, (B, H, N), q.device)
    _call("fa_bwd_dq", _ptr(q), _ptr(k), _ptr(v), _ptr(do), _ptr(lse), _ptr(dvec), _ptr(dq),
          B, H, N, d, int(bool(causal)), _scale(scale, d), _stream())
    return dq


# ---------------------------------------------------------------- element type chosen by the tensors

def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float16:
        return FA_F16
    raise TypeError(f"q must be torch.bfloat16 or torch.float16, got {t.dtype}")


def fwd_ex(q, k, v, causal: bool = False, scale: Optional[float] = None, stabilize: bool = False,
           diag: bool = False):
    """Forward pass in the element type of q (bfloat16 or float16).

    Returns (O, LSE), plus the per-row shift report (uint8 (B,H,N)) when
    ``diag``."""
    torch = _torch()
    B, H, N, d = _shape(q)
    dev = q.device
    code = _dtype_code(q)
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check(n, t, q.dtype, (B, H, N, d), dev)
    o = torch.empty_like(q)
    l = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    flags = torch.empty((B, H, N), dtype=torch.uint8, device=dev) if diag else None
    _call("fa_fwd_ex", code, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(l), _ptr(flags) if diag else None,
          B, H, N, d, int(bool(causal)), _scale(scale, d), int(bool(stabilize)), _stream())
    return (o, l, flags) if diag else (o, l)


def bwd_ex(q, k, v, o, do, lse, causal: bool = False, scale: Optional[float] = None,
           stabilize: bool = False, workspace=None):
    """Backward pass in the element type of q.  Returns (dQ, dK, dV)."""
    torch = _torch()
    B, H, N, d = _shape(q)
    dev = q.device
    code = _dtype_code(q)
    for n, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check(n, t, q.dtype, (B, H, N, d), dev)
    _check("lse", lse, torch.float32, (B, H, N), dev)
    nbytes = workspace_bytes(B, H, N, d, causal)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    _call("fa_bwd_ex", code, _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(do), _ptr(lse), _ptr(dq), _ptr(dk),
          _ptr(dv), _ptr(workspace), workspace.numel() * workspace.element_size(), B, H, N, d,
          int(bool(causal)), _scale(scale, d), int(bool(stabilize)), _stream())
    return dq, dk, dv


# ---------------------------------------------------------------- baseline attention

def base_ld(N: int) -> int:
    """Row stride (elements) of the baseline's S and P matrices."""
    return int(load().fa_base_ld(int(N)))


def base_workspace_bytes(B: int, H: int, N: int, d: int, causal: bool) -> int:
    return int(load().fa_base_workspace_bytes(B, H, N, d, int(bool(causal))))


def base_fwd(q, k, v, causal: bool = False, scale: Optional[float] = None, workspace=None):
    """The unfused FP32-accumulating baseline attention.  Returns (O bf16, LSE fp32)."""
    torch = _torch()
    B, H, N, d = _shape(q)
    dev = q.device
    for n, t in (("q", q), ("k", k), ("v", v)):
        _check(n, t, torch.bfloat16, (B, H, N, d), dev)
    if workspace is None:
        workspace = torch.empty(base_workspace_bytes(B, H, N, d, causal), dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    l = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    _call("fa_base_fwd", _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(l), _ptr(workspace),
          workspace.numel() * workspace.element_size(), B, H, N, d, int(bool(causal)), _scale(scale, d), _stream())
    return o, l


def base_scores(q, k, causal: bool = False, scale: Optional[float] = None, s=None):
    """S = fl32(fl32(Q K^T) * scale), fp32 (B, H, N, base_ld(N)); entries the
    baseline never reads (causal: past the diagonal block; columns >= N) are
    left as they were."""
    torch = _torch()
    B, H, N, d = _shape(q)
    _check("k", k, torch.bfloat16, (B, H, N, d), q.device)
    _check("q", q, torch.bfloat16, (B, H, N, d), q.device)
    s = torch.empty((B, H, N, base_ld(N)), dtype=torch.float32, device=q.device) if s is None else s
    _check("s", s, torch.float32, (B, H, N, base_ld(N)), q.device)
    _call("fa_base_scores", _ptr(q), _ptr(k), _ptr(s), B, H, N, d, int(bool(causal)), _scale(scale, d), _stream())
    return s


def base_softmax(s, causal: bool = False, p=None, lse=None):
    """P (bf16, same shape as S) and LSE (fp32 (B, H, N)) from the baseline's S."""
    torch = _torch()
    if s.dim() != 4:
        raise ValueError("s must have shape (B, H, N, ld)")
    B, H, N, ld = (int(x) for x in s.shape)
    if ld != base_ld(N):
        raise ValueError(f"s has row stride {ld}, expected {base_ld(N)}")
    _check("s", s, torch.float32, (B, H, N, ld), s.device)
    p = torch.empty((B, H, N, ld), dtype=torch.bfloat16, device=s.device) if p is None else p
    lse = torch.empty((B, H, N), dtype=torch.float32, device=s.device) if lse is None else lse
    _check("p", p, torch.bfloat16, (B, H, N, ld), s.device)
    _check("lse", lse, torch.float32, (B, H, N), s.device)
    _call("fa_base_softmax", _ptr(s), _ptr(p), _ptr(lse), B, H, N, int(bool(causal)), _stream())
    return p, lse


def base_pv(p, v, causal: bool = False, out=None):
    """O = bf16(P V) of the baseline."""
    torch = _torch()
    B, H, N, d = _shape(v)
    _check("v", v, torch.bfloat16, (B, H, N, d), v.device)
    _check("p", p, torch.bfloat16, (B, H, N, base_ld(N)), v.device)
    o = torch.empty_like(v) if out is None else out
    _check("out", o, torch.bfloat16, (B, H, N, d), v.device)
    _call("fa_base_pv", _ptr(p), _ptr(v), _ptr(o), B, H, N, d, int(bool(causal)), _stream())
    return o


# ---------------------------------------------------------------- measured ceiling

def mfma_probe(blocks: int = 2048, iters: int = 2000, out=None):
    """Enqueue the bf16 MFMA throughput probe; returns (FLOP of the launch, out)."""
    torch = _torch()
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda") if out is None else out
    if out.numel() < blocks * 256 or out.dtype != torch.float32:
        raise ValueError("out must hold blocks*256 float32 values")
    flop = int(load().fa_mfma_probe(_ptr(out), int(blocks), int(iters), _stream()))
    if flop < 0:
        raise FAError("fa_mfma_probe", flop)
    return flop, out


HBM_PROBE_THREADS = 4096 * 256


def hbm_probe(src, sink=None):
    """Enqueue the HBM read probe over the bytes of src (a contiguous device
    tensor whose size is a multiple of 16 bytes).  Returns the sink tensor
    (one folded int32 per probe thread)."""
    torch = _torch()
    if not src.is_contiguous():
        raise ValueError("src must be contiguous")
    sink = torch.empty(HBM_PROBE_THREADS, dtype=torch.int32, device=src.device) if sink is None else sink
    if sink.numel() < HBM_PROBE_THREADS or sink.element_size() != 4:
        raise ValueError(f"sink must hold {HBM_PROBE_THREADS} 32-bit values")
    _call("fa_hbm_probe", _ptr(src), src.numel() * src.element_size(), _ptr(sink), _stream())
    return sink


ISSUE_PROBE_KINDS = ("mfma", "v_fma_f32", "v_max3_f32", "v_med3_f32", "v_exp_f32", "v_cvt_pk_bf16_f32",
                     "mfma+fma", "mfma|fma", "ds_read_b128", "mfma(lds a)",
                     "ds_read_b64_tr_b16", "mfma(lds a, transposing reads)", "mfma+exp", "mfma+softmax mix",
                     "mfma+max3", "mfma+cvt_pk_bf16", "mfma+max")


def issue_probe(kind: int, waves_per_simd: int, blocks: int = 1024, iters: int = 2048, out=None):
    """Enqueue the instruction-issue probe (see fa.h); returns out."""
    torch = _torch()
    out = torch.empty(blocks * 512, dtype=torch.float32, device="cuda") if out is None else out
    if out.numel() < blocks * 512 or out.dtype != torch.float32:
        raise ValueError("out must hold blocks*512 float32 values")
    _call("fa_issue_probe", int(kind), int(waves_per_simd), _ptr(out), int(blocks), int(iters), _stream())
    return out


# ---------------------------------------------------------------- autograd

def attention(q, k, v, causal: bool = False, scale: Optional[float] = None, stabilize: bool = False):
    """softmax(scale * q k^T) v as a differentiable torch op: the forward is
    fa_fwd_ex and the backward fa_bwd_ex (bfloat16 or float16 tensors,
    (B, H, N, d), contiguous).  Only the marshalling is Python."""
    return _attention_fn().apply(q, k, v, bool(causal), scale, bool(stabilize))


_ATTN = None


def _attention_fn():
    global _ATTN
    if _ATTN is None:
        torch = _torch()

        class _Attention(torch.autograd.Function):
            @staticmethod
            def forward(ctx, q, k, v, causal, scale, stabilize):
                q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
                o, lse = fwd_ex(q, k, v, causal=causal, scale=scale, stabilize=stabilize)
                ctx.save_for_backward(q, k, v, o, lse)
                ctx.causal, ctx.scale, ctx.stabilize = causal, scale, stabilize
                return o

            @staticmethod
            def backward(ctx, do):
                q, k, v, o, lse = ctx.saved_tensors
                dq, dk, dv = bwd_ex(q, k, v, o, do.contiguous(), lse, causal=ctx.causal, scale=ctx.scale,
                                    stabilize=ctx.stabilize)
                return dq, dk, dv, None, None, None

        _ATTN = _Attention
    return _ATTN
