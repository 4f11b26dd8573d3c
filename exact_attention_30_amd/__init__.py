"""exact_attention_30_amd — fused exact attention for AMD Instinct MI355X.

Python binding of the C ABI declared in include/fa.h (libfa.so, built from
csrc/ by ``exact_attention_30_amd.build``).  This module only marshals
arguments: it checks torch tensors, allocates outputs with torch (device
memory) and passes raw pointers and the current HIP stream to the library.
Every step of the computation runs in the library's HIP kernels; there is no
fallback.  Importing works without a GPU; the first call loads libfa.so and
raises if it is missing.

    o, lse = fwd(q, k, v, scale=None, causal=True)
    dq, dk, dv = bwd(q, k, v, o, dout, lse, scale=None, causal=True)

q, o, dout: [B, Hq, T, D]; k, v: [B, Hkv, T, D]; contiguous, on the same GPU,
all bfloat16 or all float32; lse: [B, Hq, T] float32.  `scale` defaults to
1/sqrt(D).
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = ["fwd", "bwd", "bwd_preprocess", "bwd_dkdv", "bwd_dq", "bwd_workspace_bytes",
           "FAError", "library", "LIB_PATH", "version"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_BF16, FA_FP32 = 0, 1
_DTYPES = {torch.bfloat16: FA_BF16, torch.float32: FA_FP32}

# names and argument lists of every entry point in include/fa.h
_vp, _fp, _i, _f = ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_float
SIGNATURES = {
    "fa_fwd": ([_vp, _vp, _vp, _vp, _fp, _i, _i, _i, _i, _i, _f, _i, _i, _vp], ctypes.c_int),
    "fa_bwd_workspace_bytes": ([_i, _i, _i, _i, _i, _i], ctypes.c_size_t),
    "fa_bwd": ([_vp, _vp, _vp, _vp, _vp, _fp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i,
                _i, _vp], ctypes.c_int),
    "fa_bwd_preprocess": ([_vp, _vp, _fp, _i, _i, _i, _i, _i, _vp], ctypes.c_int),
    "fa_bwd_dkdv": ([_vp, _vp, _vp, _vp, _fp, _fp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i, _i,
                     _vp], ctypes.c_int),
    "fa_bwd_dq": ([_vp, _vp, _vp, _vp, _fp, _fp, _vp, _i, _i, _i, _i, _i, _f, _i, _i, _vp],
                  ctypes.c_int),
    "fa_status_string": ([_i], ctypes.c_char_p),
    "fa_version": ([], ctypes.c_char_p),
}

_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {library().fa_status_string(status).decode()} (status {status})")


def library() -> ctypes.CDLL:
    """The loaded libfa.so (loaded on first use; raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m exact_attention_30_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _lib = lib
    return _lib


def version() -> str:
    return library().fa_version().decode()


def _check(status: int, where: str):
    if status != 0:
        raise FAError(status, where)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _dims(q, k, v):
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q must be [B,Hq,T,D]; k and v [B,Hkv,T,D]")
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    if k.shape[0] != B or k.shape[2] != T or k.shape[3] != D:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)}")
    return B, Hq, Hkv, T, D


def _dtype_code(*ts) -> int:
    dt = ts[0].dtype
    if dt not in _DTYPES:
        raise TypeError(f"unsupported dtype {dt}: use bfloat16 or float32")
    for t in ts:
        if t.dtype != dt:
            raise TypeError("q, k, v (and o, dout) must share one dtype")
        if not t.is_cuda or t.device != ts[0].device:
            raise ValueError("all tensors must be on the same GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")
    return _DTYPES[dt]


def _scale(scale, D) -> float:
    return 1.0 / math.sqrt(D) if scale is None else float(scale)


def fwd(q, k, v, scale=None, causal: bool = True, out=None, lse=None):
    """Forward pass; returns (o, lse).  `out`/`lse` may be preallocated."""
    B, Hq, Hkv, T, D = _dims(q, k, v)
    dt = _dtype_code(q, k, v)
    o = torch.empty_like(q) if out is None else out
    l = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device) if lse is None else lse
    _check(library().fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), l.data_ptr(),
                            B, Hq, Hkv, T, D, _scale(scale, D), int(bool(causal)), dt,
                            _stream(q)), "fa_fwd")
    return o, l


def bwd_workspace_bytes(B, Hq, Hkv, T, D, dtype=torch.bfloat16) -> int:
    return int(library().fa_bwd_workspace_bytes(B, Hq, Hkv, T, D, _DTYPES[dtype]))


def bwd(q, k, v, o, dout, lse, scale=None, causal: bool = True, workspace=None, grads=None):
    """Backward pass; returns (dq, dk, dv).  `grads` = (dq, dk, dv) may be
    preallocated; `workspace` is a uint8 device tensor of at least
    bwd_workspace_bytes(...) bytes."""
    B, Hq, Hkv, T, D = _dims(q, k, v)
    dt = _dtype_code(q, k, v, o, dout)
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, T):
        raise ValueError("lse must be float32 [B,Hq,T]")
    dq, dk, dv = grads if grads is not None else (torch.empty_like(q), torch.empty_like(k),
                                                  torch.empty_like(v))
    ws_bytes = bwd_workspace_bytes(B, Hq, Hkv, T, D, q.dtype)
    ws = workspace if workspace is not None else torch.empty(max(ws_bytes, 16), dtype=torch.uint8,
                                                             device=q.device)
    if ws.numel() * ws.element_size() < ws_bytes:
        raise ValueError("workspace too small")
    _check(library().fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                            dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                            dv.data_ptr(), ws.data_ptr(), B, Hq, Hkv, T, D, _scale(scale, D),
                            int(bool(causal)), dt, _stream(q)), "fa_bwd")
    return dq, dk, dv


def bwd_preprocess(o, dout, delta=None):
    """delta = rowsum(dout * o) as float32 [B, Hq, T]."""
    B, Hq, T, D = o.shape
    dt = _dtype_code(o, dout)
    d = torch.empty((B, Hq, T), dtype=torch.float32, device=o.device) if delta is None else delta
    _check(library().fa_bwd_preprocess(o.data_ptr(), dout.data_ptr(), d.data_ptr(), B, Hq, T, D,
                                       dt, _stream(o)), "fa_bwd_preprocess")
    return d


def bwd_dkdv(q, k, v, dout, lse, delta, scale=None, causal: bool = True, dk=None, dv=None):
    B, Hq, Hkv, T, D = _dims(q, k, v)
    dt = _dtype_code(q, k, v, dout)
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _check(library().fa_bwd_dkdv(q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(),
                                 lse.data_ptr(), delta.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                 B, Hq, Hkv, T, D, _scale(scale, D), int(bool(causal)), dt,
                                 _stream(q)), "fa_bwd_dkdv")
    return dk, dv


def bwd_dq(q, k, v, dout, lse, delta, scale=None, causal: bool = True, dq=None):
    B, Hq, Hkv, T, D = _dims(q, k, v)
    dt = _dtype_code(q, k, v, dout)
    dq = torch.empty_like(q) if dq is None else dq
    _check(library().fa_bwd_dq(q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(),
                               lse.data_ptr(), delta.data_ptr(), dq.data_ptr(), B, Hq, Hkv, T, D,
                               _scale(scale, D), int(bool(causal)), dt, _stream(q)), "fa_bwd_dq")
    return dq
