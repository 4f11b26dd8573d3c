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

q, o, dout: [B, Hq, Tq, D]; k, v: [B, Hkv, Tk, D]; contiguous, on the same GPU,
all bfloat16 or all float32; lse: [B, Hq, Tq] float32.  `scale` defaults to
1/sqrt(D).  With causal=True, query row i sees keys j <= i + q_offset;
q_offset defaults to Tk - Tq (the last query row on the last key; 0 when
Tq == Tk).
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = ["fwd", "bwd", "bwd_noalloc", "NOALLOC_SCRATCH_BYTES", "bwd_preprocess", "bwd_dkdv", "bwd_dq", "bwd_workspace_bytes",
           "dkdv_split_bytes", "dq_split_bytes", "fwd_split_bytes", "FAError", "library",
           "LIB_PATH", "version"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libfa.so")

FA_BF16, FA_FP32, FA_BF16_F32OUT = 0, 1, 2
# FA_NOALLOC_SCRATCH_BYTES of include/fa.h: the static scratch of fa_bwd_noalloc
NOALLOC_SCRATCH_BYTES = 64 << 20
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
    "fa_fwd_kv": ([_vp, _vp, _vp, _vp, _fp, _i, _i, _i, _i, _i, _i, _f, _i, _i, _i, _vp],
                  ctypes.c_int),
    "fa_bwd_kv": ([_vp, _vp, _vp, _vp, _vp, _fp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f,
                   _i, _i, _i, _vp], ctypes.c_int),
    "fa_bwd_dkdv_kv": ([_vp, _vp, _vp, _vp, _fp, _fp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i,
                        _i, _i, _vp], ctypes.c_int),
    "fa_bwd_dq_kv": ([_vp, _vp, _vp, _vp, _fp, _fp, _vp, _i, _i, _i, _i, _i, _i, _f, _i, _i, _i,
                      _vp], ctypes.c_int),
    "fa_bwd_kv_workspace_bytes": ([_i, _i, _i, _i, _i, _i, _i], ctypes.c_size_t),
    "fa_bwd_dkdv_split_bytes": ([_i, _i, _i, _i, _i, _i, _i], ctypes.c_size_t),
    "fa_bwd_dkdv_split": ([_vp, _vp, _vp, _vp, _fp, _fp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f,
                           _i, _i, _i, _vp], ctypes.c_int),
    "fa_bwd_dq_split_bytes": ([_i, _i, _i, _i, _i, _i, _i], ctypes.c_size_t),
    "fa_bwd_dq_split": ([_vp, _vp, _vp, _vp, _fp, _fp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i,
                         _i, _i, _vp], ctypes.c_int),
    "fa_bwd_dq_delta": ([_vp, _vp, _vp, _vp, _vp, _fp, _fp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f,
                         _i, _i, _i, _vp], ctypes.c_int),
    "fa_fwd_split_bytes": ([_i, _i, _i, _i, _i, _i, _i], ctypes.c_size_t),
    "fa_block_rows": ([_i, _i, _i, _i, _i, _i], _i),
    "fa_bwd_atomic_workspace_bytes": ([_i, _i, _i, _i, _i], ctypes.c_size_t),
    "fa_bwd_atomic": ([_vp, _vp, _vp, _vp, _vp, _fp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _i,
                       _i, _vp], ctypes.c_int),
    "fa_fwd_split": ([_vp, _vp, _vp, _vp, _fp, _vp, _i, _i, _i, _i, _i, _i, _f, _i, _i, _i, _vp],
                     ctypes.c_int),
    "fa_fwd_fp8_workspace_bytes": ([_i, _i, _i, _i], ctypes.c_size_t),
    "fa_fwd_fp8": ([_vp, _vp, _vp, _f, _f, _f, _vp, _fp, _vp, _i, _i, _i, _i, _i, _i, _f, _i, _i,
                    _vp], ctypes.c_int),
    "fa_fp8_transpose_v": ([_vp, _vp, _i, _i, _i, _i, _vp], ctypes.c_int),
    "fa_fwd_fp8_vt": ([_vp, _vp, _vp, _f, _f, _f, _vp, _fp, _i, _i, _i, _i, _i, _i, _f, _i, _i,
                       _vp], ctypes.c_int),
    "fa_bwd_noalloc": ([_vp, _vp, _vp, _vp, _vp, _fp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _i,
                        _i, _i, _vp], ctypes.c_int),
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
    """(B, Hq, Hkv, Tq, Tk, D) of q [B,Hq,Tq,D] and k, v [B,Hkv,Tk,D]."""
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q must be [B,Hq,Tq,D]; k and v [B,Hkv,Tk,D]")
    B, Hq, Tq, D = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != D:
        raise ValueError(f"shape mismatch q{tuple(q.shape)} k{tuple(k.shape)}")
    return B, Hq, Hkv, Tq, Tk, D


def _expect(t, shape, name, dtype=None):
    """Raise ValueError unless tensor t has the given shape (and dtype): the
    kernels read and write exactly that many elements."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _offset(Tq, Tk, q_offset) -> int:
    return Tk - Tq if q_offset is None else int(q_offset)


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


def _out_code(in_dtype, out_dtype) -> int:
    """fa_dtype of a call whose inputs have in_dtype and whose results have
    out_dtype: the same type, or float32 results of bfloat16 inputs
    (FA_BF16_F32OUT: the bf16 kernels' results stored unrounded)."""
    if out_dtype == in_dtype and in_dtype in _DTYPES:
        return _DTYPES[in_dtype]
    if in_dtype == torch.bfloat16 and out_dtype == torch.float32:
        return FA_BF16_F32OUT
    raise TypeError(f"results of {out_dtype} for inputs of {in_dtype}: use the inputs' dtype, "
                    "or float32 for bfloat16 inputs")


def _result_dtype(q, given, out_dtype):
    """dtype of the results: that of the preallocated tensor `given`, else
    out_dtype, else q's."""
    if given is not None:
        if out_dtype is not None and given.dtype != out_dtype:
            raise TypeError(f"preallocated result is {given.dtype}, out_dtype {out_dtype}")
        return given.dtype
    return q.dtype if out_dtype is None else out_dtype


def _same_device(ref, *ts):
    """Every given tensor is a contiguous tensor on ref's GPU."""
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda or t.device != ref.device:
            raise ValueError("all tensors must be on the same GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _scale(scale, D) -> float:
    return 1.0 / math.sqrt(D) if scale is None else float(scale)


def fwd_split_bytes(B, Hq, Hkv, Tq, Tk, D, dtype=torch.bfloat16) -> int:
    """Bytes of the chunk-partial buffer fwd uses to split key ranges (0: these
    shapes do not split)."""
    return int(library().fa_fwd_split_bytes(B, Hq, Hkv, Tq, Tk, D, _DTYPES[dtype]))


STAGES = {"fwd": 0, "dq": 1, "dkdv": 2}


def block_rows(stage, B, H, T, D, dtype=torch.bfloat16) -> int:
    """Rows of one workgroup's block for these shapes (the tile table):
    stage "fwd" or "dq" (query rows; H = Hq, T = Tq) or "dkdv" (keys;
    H = Hkv, T = Tk); 0 for shapes the kernels reject."""
    return int(library().fa_block_rows(STAGES[stage], B, H, T, D, _DTYPES[dtype]))


def fwd(q, k, v, scale=None, causal: bool = True, out=None, lse=None, q_offset=None,
        partial=None, out_dtype=None):
    """Forward pass; returns (o, lse).  `out`/`lse` may be preallocated.
    With bfloat16 inputs, out_dtype=torch.float32 (or a float32 `out`) stores
    O unrounded (FA_BF16_F32OUT).
    Calls fa_fwd when Tq == Tk and the offset is 0, else fa_fwd_kv; with
    `partial` (a device tensor of at least fwd_split_bytes(...) bytes) calls
    fa_fwd_split, which splits key ranges when the shapes call for it."""
    B, Hq, Hkv, Tq, Tk, D = _dims(q, k, v)
    odt = _result_dtype(q, out, out_dtype)
    _expect(out, q.shape, "out", odt)
    _expect(lse, (B, Hq, Tq), "lse", torch.float32)
    dt = _out_code(q.dtype, odt)
    _dtype_code(q, k, v)
    _same_device(q, out, lse, partial)
    off = _offset(Tq, Tk, q_offset)
    o = torch.empty(q.shape, dtype=odt, device=q.device) if out is None else out
    l = torch.empty((B, Hq, Tq), dtype=torch.float32, device=q.device) if lse is None else lse
    lib = library()
    if partial is not None:
        need = fwd_split_bytes(B, Hq, Hkv, Tq, Tk, D, q.dtype)
        if partial.numel() * partial.element_size() < need:
            raise ValueError("partial buffer too small")
        _check(lib.fa_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                l.data_ptr(), partial.data_ptr() if need else None, B, Hq, Hkv, Tq,
                                Tk, D, _scale(scale, D), int(bool(causal)), off, dt, _stream(q)),
               "fa_fwd_split")
    elif Tq == Tk and (off == 0 or not causal):
        _check(lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), l.data_ptr(),
                          B, Hq, Hkv, Tq, D, _scale(scale, D), int(bool(causal)), dt,
                          _stream(q)), "fa_fwd")
    else:
        _check(lib.fa_fwd_kv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), l.data_ptr(),
                             B, Hq, Hkv, Tq, Tk, D, _scale(scale, D), int(bool(causal)), off, dt,
                             _stream(q)), "fa_fwd_kv")
    return o, l


def fwd_fp8_workspace_bytes(B, Hkv, Tk, D) -> int:
    """Workspace bytes of fwd_fp8 (V transposed tile by tile)."""
    return int(library().fa_fwd_fp8_workspace_bytes(B, Hkv, Tk, D))


def _fp8_check(*ts):
    for t in ts:
        if t.dtype != torch.float8_e4m3fn:
            raise TypeError("the fp8 calls take torch.float8_e4m3fn tensors")
        if not t.is_cuda or t.device != ts[0].device or not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous tensors on one GPU")


def fp8_transpose_v(v, vt=None):
    """V (float8_e4m3fn [B,Hkv,Tk,D]) transposed as fwd_fp8_vt reads it, into a
    uint8 device tensor of fwd_fp8_workspace_bytes(...) bytes (fa_fp8_transpose_v)."""
    _fp8_check(v)
    B, Hkv, Tk, D = v.shape
    need = fwd_fp8_workspace_bytes(B, Hkv, Tk, D)
    if vt is None:
        vt = torch.empty(max(need, 16), dtype=torch.uint8, device=v.device)
    elif vt.numel() * vt.element_size() < need:
        raise ValueError("vt too small")
    _check(library().fa_fp8_transpose_v(v.data_ptr(), vt.data_ptr(), B, Hkv, Tk, D, _stream(v)),
           "fa_fp8_transpose_v")
    return vt


def fwd_fp8_vt(q, k, vt, v_shape, q_descale, k_descale, v_descale, scale=None,
               causal: bool = True, out=None, lse=None, q_offset=None):
    """fwd_fp8 with V already transposed by fp8_transpose_v (fa_fwd_fp8_vt);
    v_shape is the shape of the V it came from."""
    B, Hq, Tq, D = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    if tuple(k.shape) != tuple(v_shape) or k.shape[0] != B or k.shape[3] != D:
        raise ValueError("shape mismatch")
    _expect(out, q.shape, "out", torch.bfloat16)
    _expect(lse, (B, Hq, Tq), "lse", torch.float32)
    _fp8_check(q, k)
    _same_device(q, vt, out, lse)
    need = fwd_fp8_workspace_bytes(B, Hkv, Tk, D)
    if vt.numel() * vt.element_size() < need:
        raise ValueError("vt too small")
    off = _offset(Tq, Tk, q_offset)
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device) if out is None else out
    l = torch.empty((B, Hq, Tq), dtype=torch.float32, device=q.device) if lse is None else lse
    _check(library().fa_fwd_fp8_vt(q.data_ptr(), k.data_ptr(), vt.data_ptr(), float(q_descale),
                                   float(k_descale), float(v_descale), o.data_ptr(), l.data_ptr(),
                                   B, Hq, Hkv, Tq, Tk, D, _scale(scale, D), int(bool(causal)), off,
                                   _stream(q)), "fa_fwd_fp8_vt")
    return o, l


def fwd_fp8(q, k, v, q_descale, k_descale, v_descale, scale=None, causal: bool = True,
            out=None, lse=None, q_offset=None, workspace=None):
    """FP8 forward: q, k, v are torch.float8_e4m3fn codes whose real values are
    the codes times q_descale, k_descale, v_descale.  Returns (o bf16, lse
    float32); calls fa_fwd_fp8.  `workspace` (uint8 device tensor of at least
    fwd_fp8_workspace_bytes(...) bytes) is allocated when not given."""
    B, Hq, Hkv, Tq, Tk, D = _dims(q, k, v)
    _expect(out, q.shape, "out", torch.bfloat16)
    _expect(lse, (B, Hq, Tq), "lse", torch.float32)
    _fp8_check(q, k, v)
    _same_device(q, out, lse, workspace)
    off = _offset(Tq, Tk, q_offset)
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device) if out is None else out
    l = torch.empty((B, Hq, Tq), dtype=torch.float32, device=q.device) if lse is None else lse
    need = fwd_fp8_workspace_bytes(B, Hkv, Tk, D)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    elif workspace.numel() * workspace.element_size() < need:
        raise ValueError("workspace too small")
    _check(library().fa_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), float(q_descale),
                                float(k_descale), float(v_descale), o.data_ptr(), l.data_ptr(),
                                workspace.data_ptr(), B, Hq, Hkv, Tq, Tk, D, _scale(scale, D),
                                int(bool(causal)), off, _stream(q)), "fa_fwd_fp8")
    return o, l


def bwd_workspace_bytes(B, Hq, Hkv, T, D, dtype=torch.bfloat16, Tk=None) -> int:
    """Workspace bytes of bwd for T query rows (against Tk keys, default T)."""
    Tk = T if Tk is None else Tk
    return int(library().fa_bwd_kv_workspace_bytes(B, Hq, Hkv, T, Tk, D, _DTYPES[dtype]))


def dq_split_bytes(B, Hq, Hkv, Tq, Tk, D, dtype=torch.bfloat16) -> int:
    """Bytes of the partial-sum buffer bwd_dq uses to split its key range
    (0: these shapes do not split)."""
    return int(library().fa_bwd_dq_split_bytes(B, Hq, Hkv, Tq, Tk, D, _DTYPES[dtype]))


def dkdv_split_bytes(B, Hq, Hkv, Tq, Tk, D, dtype=torch.bfloat16) -> int:
    """Bytes of the partial-sum buffer bwd_dkdv uses to split its query side
    (0: these shapes do not split)."""
    return int(library().fa_bwd_dkdv_split_bytes(B, Hq, Hkv, Tq, Tk, D, _DTYPES[dtype]))


def bwd(q, k, v, o, dout, lse, scale=None, causal: bool = True, workspace=None, grads=None,
        q_offset=None):
    """Backward pass; returns (dq, dk, dv), of o's dtype (float32 o with
    bfloat16 inputs: FA_BF16_F32OUT, gradients stored unrounded).  `grads` = (dq, dk, dv) may be
    preallocated; `workspace` is a uint8 device tensor of at least
    bwd_workspace_bytes(...) bytes.  Calls fa_bwd when Tq == Tk and the
    offset is 0, else fa_bwd_kv (same q_offset as the forward)."""
    B, Hq, Hkv, Tq, Tk, D = _dims(q, k, v)
    _expect(o, q.shape, "o")
    _expect(dout, q.shape, "dout")
    _expect(lse, (B, Hq, Tq), "lse", torch.float32)
    if grads is not None:
        for t, like, name in zip(grads, (q, k, v), ("dq", "dk", "dv")):
            _expect(t, like.shape, name, o.dtype)
    dt = _out_code(q.dtype, o.dtype)  # float32 o with bf16 inputs: float32 gradients
    _dtype_code(q, k, v, dout)
    _same_device(q, o, *(grads or ()))
    _same_device(q, lse, workspace)
    off = _offset(Tq, Tk, q_offset)
    dq, dk, dv = grads if grads is not None else (torch.empty_like(q, dtype=o.dtype),
                                                  torch.empty_like(k, dtype=o.dtype),
                                                  torch.empty_like(v, dtype=o.dtype))
    ws_bytes = bwd_workspace_bytes(B, Hq, Hkv, Tq, D, q.dtype, Tk=Tk)
    ws = workspace if workspace is not None else torch.empty(max(ws_bytes, 16), dtype=torch.uint8,
                                                             device=q.device)
    if ws.numel() * ws.element_size() < ws_bytes:
        raise ValueError("workspace too small")
    lib = library()
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr())
    if Tq == Tk and (off == 0 or not causal):
        _check(lib.fa_bwd(*ptrs, B, Hq, Hkv, Tq, D, _scale(scale, D), int(bool(causal)), dt,
                          _stream(q)), "fa_bwd")
    else:
        _check(lib.fa_bwd_kv(*ptrs, B, Hq, Hkv, Tq, Tk, D, _scale(scale, D), int(bool(causal)), off,
                             dt, _stream(q)), "fa_bwd_kv")
    return dq, dk, dv


def bwd_atomic_workspace_bytes(B, Hq, T, D, dtype=torch.bfloat16) -> int:
    """Bytes of the workspace of bwd_atomic (0: unsupported shapes)."""
    return int(library().fa_bwd_atomic_workspace_bytes(B, Hq, T, D, _DTYPES[dtype]))


def bwd_atomic(q, k, v, o, dout, lse, scale=None, causal: bool = True, workspace=None, grads=None):
    """The single-kernel backward with dQ accumulated by atomic adds
    (fa_bwd_atomic; bf16, D = 64, equal query and key lengths); returns
    (dq, dk, dv).  dK, dV are bitwise those of bwd_dkdv; dQ is not bitwise
    reproducible."""
    B, Hq, Hkv, Tq, Tk, D = _dims(q, k, v)
    if Tq != Tk:
        raise ValueError("bwd_atomic takes equal query and key lengths")
    _expect(o, q.shape, "o")
    _expect(dout, q.shape, "dout")
    _expect(lse, (B, Hq, Tq), "lse", torch.float32)
    if grads is not None:
        for t, like, name in zip(grads, (q, k, v), ("dq", "dk", "dv")):
            _expect(t, like.shape, name, q.dtype)
    dt = _dtype_code(q, k, v, o, dout, *(grads or ()))
    _same_device(q, lse, workspace)
    dq, dk, dv = grads if grads is not None else (torch.empty_like(q), torch.empty_like(k),
                                                  torch.empty_like(v))
    ws_bytes = bwd_atomic_workspace_bytes(B, Hq, Tq, D, q.dtype)
    ws = workspace if workspace is not None else torch.empty(max(ws_bytes, 16), dtype=torch.uint8,
                                                             device=q.device)
    if ws.numel() * ws.element_size() < ws_bytes:
        raise ValueError("workspace too small")
    _check(library().fa_bwd_atomic(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                   dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                   dv.data_ptr(), ws.data_ptr(), B, Hq, Hkv, Tq, D,
                                   _scale(scale, D), int(bool(causal)), dt, _stream(q)),
           "fa_bwd_atomic")
    return dq, dk, dv


def bwd_noalloc(q, k, v, o, dout, lse, scale=None, causal: bool = True, grads=None,
                q_offset=None):
    """bwd through fa_bwd_noalloc: the library takes its workspace from a
    static per-GPU scratch instead of a buffer (raises FAError with status
    FA_ERR_SCRATCH = 6 for shapes whose workspace exceeds
    NOALLOC_SCRATCH_BYTES).  Allocates nothing when `grads` = (dq, dk, dv) is
    given.  Calls on one GPU share the scratch: overlapping calls race."""
    B, Hq, Hkv, Tq, Tk, D = _dims(q, k, v)
    _expect(o, q.shape, "o")
    _expect(dout, q.shape, "dout")
    _expect(lse, (B, Hq, Tq), "lse", torch.float32)
    if grads is not None:
        for t, like, name in zip(grads, (q, k, v), ("dq", "dk", "dv")):
            _expect(t, like.shape, name, o.dtype)
    dt = _out_code(q.dtype, o.dtype)  # float32 o with bf16 inputs: float32 gradients
    _dtype_code(q, k, v, dout)
    _same_device(q, o, *(grads or ()))
    _same_device(q, lse)
    off = _offset(Tq, Tk, q_offset)
    dq, dk, dv = grads if grads is not None else (torch.empty_like(q, dtype=o.dtype),
                                                  torch.empty_like(k, dtype=o.dtype),
                                                  torch.empty_like(v, dtype=o.dtype))
    with torch.cuda.device(q.device):  # the library uses the current device's scratch
        _check(library().fa_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                        dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                        dv.data_ptr(), B, Hq, Hkv, Tq, Tk, D, _scale(scale, D),
                                        int(bool(causal)), off, dt, _stream(q)), "fa_bwd_noalloc")
    return dq, dk, dv


def bwd_preprocess(o, dout, delta=None):
    """delta = rowsum(dout * o) as float32 [B, Hq, T]."""
    if o.dim() != 4:
        raise ValueError("o must be [B,Hq,T,D]")
    B, Hq, T, D = o.shape
    _expect(dout, o.shape, "dout")
    _expect(delta, (B, Hq, T), "delta", torch.float32)
    dt = _out_code(dout.dtype, o.dtype)  # float32 o with bf16 dout: FA_BF16_F32OUT
    _dtype_code(dout)
    _same_device(dout, o, delta)
    d = torch.empty((B, Hq, T), dtype=torch.float32, device=o.device) if delta is None else delta
    _check(library().fa_bwd_preprocess(o.data_ptr(), dout.data_ptr(), d.data_ptr(), B, Hq, T, D,
                                       dt, _stream(o)), "fa_bwd_preprocess")
    return d


def bwd_dkdv(q, k, v, dout, lse, delta, scale=None, causal: bool = True, dk=None, dv=None,
             q_offset=None, partial=None, out_dtype=None):
    """dK, dV (of out_dtype: as the inputs, or float32 for bfloat16 inputs); with `partial` (a device tensor of at least dkdv_split_bytes(...)
    bytes) the query side is split over more workgroups when the shapes call
    for it (fa_bwd_dkdv_split)."""
    B, Hq, Hkv, Tq, Tk, D = _dims(q, k, v)
    _expect(dout, q.shape, "dout")
    _expect(lse, (B, Hq, Tq), "lse", torch.float32)
    _expect(delta, (B, Hq, Tq), "delta", torch.float32)
    odt = _result_dtype(q, dk if dk is not None else dv, out_dtype)
    _expect(dk, k.shape, "dk", odt)
    _expect(dv, v.shape, "dv", odt)
    dt = _out_code(q.dtype, odt)
    _dtype_code(q, k, v, dout)
    _same_device(q, dk, dv, lse, delta, partial)
    off = _offset(Tq, Tk, q_offset)
    dk = torch.empty_like(k, dtype=odt) if dk is None else dk
    dv = torch.empty_like(v, dtype=odt) if dv is None else dv
    lib = library()
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(), lse.data_ptr(),
            delta.data_ptr(), dk.data_ptr(), dv.data_ptr())
    if partial is not None:
        need = dkdv_split_bytes(B, Hq, Hkv, Tq, Tk, D, q.dtype)
        if partial.numel() * partial.element_size() < need:
            raise ValueError("partial buffer too small")
        _check(lib.fa_bwd_dkdv_split(*ptrs, partial.data_ptr() if need else None, B, Hq, Hkv, Tq,
                                     Tk, D, _scale(scale, D), int(bool(causal)), off, dt,
                                     _stream(q)), "fa_bwd_dkdv_split")
    elif Tq == Tk and (off == 0 or not causal):
        _check(lib.fa_bwd_dkdv(*ptrs, B, Hq, Hkv, Tq, D, _scale(scale, D), int(bool(causal)), dt,
                               _stream(q)), "fa_bwd_dkdv")
    else:
        _check(lib.fa_bwd_dkdv_kv(*ptrs, B, Hq, Hkv, Tq, Tk, D, _scale(scale, D), int(bool(causal)),
                                  off, dt, _stream(q)), "fa_bwd_dkdv_kv")
    return dk, dv


def bwd_dq_delta(q, k, v, o, dout, lse, scale=None, causal: bool = True, dq=None, delta=None,
                 q_offset=None, partial=None):
    """dQ forming Delta itself (fa_bwd_dq_delta, bf16): returns (dq, delta),
    delta bitwise as bwd_preprocess would give it, for bwd_dkdv to read."""
    B, Hq, Hkv, Tq, Tk, D = _dims(q, k, v)
    _expect(o, q.shape, "o")
    _expect(dout, q.shape, "dout")
    _expect(lse, (B, Hq, Tq), "lse", torch.float32)
    _expect(delta, (B, Hq, Tq), "delta", torch.float32)
    _expect(dq, q.shape, "dq", o.dtype)
    dt = _out_code(q.dtype, o.dtype)  # float32 o with bf16 inputs: float32 dq
    _dtype_code(q, k, v, dout)
    _same_device(q, o, dq, lse, delta, partial)
    off = _offset(Tq, Tk, q_offset)
    dq = torch.empty_like(q, dtype=o.dtype) if dq is None else dq
    if delta is None:
        delta = torch.empty(B, Hq, Tq, dtype=torch.float32, device=q.device)
    need = dq_split_bytes(B, Hq, Hkv, Tq, Tk, D, q.dtype)
    if partial is not None and partial.numel() * partial.element_size() < need:
        raise ValueError("partial buffer too small")
    _check(library().fa_bwd_dq_delta(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                     dout.data_ptr(), lse.data_ptr(), delta.data_ptr(), dq.data_ptr(),
                                     partial.data_ptr() if partial is not None and need else None,
                                     B, Hq, Hkv, Tq, Tk, D, _scale(scale, D), int(bool(causal)), off,
                                     dt, _stream(q)), "fa_bwd_dq_delta")
    return dq, delta


def bwd_dq(q, k, v, dout, lse, delta, scale=None, causal: bool = True, dq=None, q_offset=None,
           partial=None, out_dtype=None):
    """dQ (of out_dtype: as the inputs, or float32 for bfloat16 inputs); with `partial` (at least dq_split_bytes(...) bytes) the key range is
    split over more workgroups when the shapes call for it (fa_bwd_dq_split)."""
    B, Hq, Hkv, Tq, Tk, D = _dims(q, k, v)
    _expect(dout, q.shape, "dout")
    _expect(lse, (B, Hq, Tq), "lse", torch.float32)
    _expect(delta, (B, Hq, Tq), "delta", torch.float32)
    odt = _result_dtype(q, dq, out_dtype)
    _expect(dq, q.shape, "dq", odt)
    dt = _out_code(q.dtype, odt)
    _dtype_code(q, k, v, dout)
    _same_device(q, dq, lse, delta, partial)
    off = _offset(Tq, Tk, q_offset)
    dq = torch.empty_like(q, dtype=odt) if dq is None else dq
    lib = library()
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(), lse.data_ptr(),
            delta.data_ptr(), dq.data_ptr())
    if partial is not None:
        need = dq_split_bytes(B, Hq, Hkv, Tq, Tk, D, q.dtype)
        if partial.numel() * partial.element_size() < need:
            raise ValueError("partial buffer too small")
        _check(lib.fa_bwd_dq_split(*ptrs, partial.data_ptr() if need else None, B, Hq, Hkv, Tq, Tk,
                                   D, _scale(scale, D), int(bool(causal)), off, dt, _stream(q)),
               "fa_bwd_dq_split")
    elif Tq == Tk and (off == 0 or not causal):
        _check(lib.fa_bwd_dq(*ptrs, B, Hq, Hkv, Tq, D, _scale(scale, D), int(bool(causal)), dt,
                             _stream(q)), "fa_bwd_dq")
    else:
        _check(lib.fa_bwd_dq_kv(*ptrs, B, Hq, Hkv, Tq, Tk, D, _scale(scale, D), int(bool(causal)),
                                off, dt, _stream(q)), "fa_bwd_dq_kv")
    return dq
