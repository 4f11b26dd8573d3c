"""fp64 CPU oracle for exact attention — TEST INFRASTRUCTURE ONLY.

Thin ctypes wrapper around ``oracle.c``: the plain unfused three-step
definition of attention (scores, safe softmax, weighted sum of values) and its
gradients written from the softmax Jacobian, in double precision.  It shares no
code with the HIP library; only the tests, the smoke check and the benchmark's
CPU-baseline leg use it.

Pages the oracle follows (cited by title and section):
  * "L'attention fusionnée" (Smallem) — «Ce que l'attention écrit en mémoire»
    gives the three unfused steps; «Une opération plutôt que trois» says the
    GPU is tested against that CPU definition; «La passe arrière» gives
    L = m + ln(l) and the gradient equations.
  * "Optimización de Flash Attention ... NVIDIA CUDA Tile" — «Atención causal»
    gives the mask (query i sees key j iff i >= j); the kernel interface of
    «Parte 1» adds a position offset for it (input_pos): with Tq query rows
    against Tk keys, query row i stands at position i + q_offset, and the
    default offset Tk - Tq puts the last query on the last key.
  * "FlashAttention: l'attenzione che non spreca memoria" — «La online softmax,
    con i numeri» gives the safe (max-subtracted) softmax.

All arrays are C-contiguous float64: q [B,Hq,Tq,D], k/v [B,Hkv,Tk,D].
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")


def build(src: str = SOURCE, out: str = LIB_PATH) -> str:
    """Compile the oracle's C source with gcc into a shared library (always
    rebuilds)."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int64)


def _p(a: np.ndarray):
    return a.ctypes.data_as(_dp)


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _idx(idx) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(idx, dtype=np.int64).reshape(-1, 3))


def _shapes(q, k, v, dout=None):
    if q.ndim != 4 or k.ndim != 4 or v.shape != k.shape:
        raise ValueError("q must be [B,Hq,Tq,D], k and v [B,Hkv,Tk,D]")
    B, Hq, Tq, D = q.shape
    if k.shape[0] != B or k.shape[3] != D or Hq % k.shape[1] != 0:
        raise ValueError(f"incompatible shapes q{q.shape} k{k.shape}")
    if dout is not None and dout.shape != q.shape:
        raise ValueError("dout must have the shape of q")
    return B, Hq, k.shape[1], Tq, k.shape[2], D


def _offset(Tq: int, Tk: int, q_offset) -> int:
    """Position of query row 0 among the keys: Tk - Tq unless given."""
    return int(Tk - Tq if q_offset is None else q_offset)


def _check(rc: int):
    if rc != 0:
        raise RuntimeError(f"oracle returned error {rc}")


class Oracle:
    """The oracle's entry points bound to one compiled library."""

    def __init__(self, lib_path: str = LIB_PATH):
        lib = ctypes.CDLL(lib_path)
        i, d, l = ctypes.c_int, ctypes.c_double, ctypes.c_long
        dp, ip = _dp, _ip
        shp = [i, i, i, i, i, i, d, i, i]  # B, Hq, Hkv, Tq, Tk, D, scale, causal, offset
        lib.oracle_fwd.argtypes = [dp, dp, dp, dp, dp, dp] + shp
        lib.oracle_bwd.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp] + shp
        lib.oracle_fwd_rows.argtypes = [dp, dp, dp, ip, l, dp, dp] + shp
        lib.oracle_dq_rows.argtypes = [dp, dp, dp, dp, ip, l, dp] + shp
        lib.oracle_dkdv_rows.argtypes = [dp, dp, dp, dp, ip, l, dp, dp] + shp
        for f in (lib.oracle_fwd, lib.oracle_bwd, lib.oracle_fwd_rows, lib.oracle_dq_rows,
                  lib.oracle_dkdv_rows):
            f.restype = ctypes.c_int
        lib.oracle_threads.argtypes = []
        lib.oracle_threads.restype = ctypes.c_int
        self.lib = lib

    def threads(self) -> int:
        """OpenMP threads the oracle's parallel loops use."""
        return int(self.lib.oracle_threads())

    def fwd(self, q, k, v, scale: float, causal: bool, return_mag: bool = False, q_offset=None):
        """Return (o [B,Hq,Tq,D], lse [B,Hq,Tq]) in float64; with return_mag also
        o_mag, the per-element sum of absolute terms sum_j |P_ij v_jd|.
        q_offset: position of query row 0 among the keys (default Tk - Tq)."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, Hq, Hkv, Tq, Tk, D = _shapes(q, k, v)
        o = np.zeros((B, Hq, Tq, D))
        lse = np.zeros((B, Hq, Tq))
        om = np.zeros((B, Hq, Tq, D)) if return_mag else None
        _check(self.lib.oracle_fwd(_p(q), _p(k), _p(v), _p(o), _p(lse),
                                   _p(om) if return_mag else None, B, Hq, Hkv, Tq, Tk, D,
                                   float(scale), int(bool(causal)), _offset(Tq, Tk, q_offset)))
        return (o, lse, om) if return_mag else (o, lse)

    def bwd(self, q, k, v, dout, scale: float, causal: bool, return_jac: bool = False,
            return_mag: bool = False, q_offset=None):
        """Return (dq, dk, dv) of the loss sum(O * dout); with return_jac also
        the per-row Jacobian term c_i = sum_j P_ij dP_ij ([B,Hq,Tq]); with
        return_mag also (dq_mag, dk_mag, dv_mag), the per-element sums of the
        absolute values of the terms.  q_offset as in fwd."""
        q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
        B, Hq, Hkv, Tq, Tk, D = _shapes(q, k, v, dout)
        dq = np.zeros_like(q)
        dk = np.zeros_like(k)
        dv = np.zeros_like(v)
        jac = np.zeros((B, Hq, Tq))
        mags = (np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)) if return_mag else None
        mp = [_p(m) for m in mags] if return_mag else [None, None, None]
        _check(self.lib.oracle_bwd(_p(q), _p(k), _p(v), _p(dout), _p(dq), _p(dk), _p(dv),
                                   _p(jac), *mp, B, Hq, Hkv, Tq, Tk, D, float(scale),
                                   int(bool(causal)), _offset(Tq, Tk, q_offset)))
        out = (dq, dk, dv)
        if return_jac:
            out = out + (jac,)
        if return_mag:
            out = out + (mags,)
        return out

    def fwd_rows(self, q, k, v, idx, scale: float, causal: bool, q_offset=None):
        """Output rows for query rows idx = [(b, h, i), ...]: (o [n,D], lse [n])."""
        q, k, v = _f64(q), _f64(k), _f64(v)
        B, Hq, Hkv, Tq, Tk, D = _shapes(q, k, v)
        ix = _idx(idx)
        o = np.zeros((len(ix), D))
        lse = np.zeros(len(ix))
        _check(self.lib.oracle_fwd_rows(_p(q), _p(k), _p(v), ix.ctypes.data_as(_ip), len(ix),
                                        _p(o), _p(lse), B, Hq, Hkv, Tq, Tk, D, float(scale),
                                        int(bool(causal)), _offset(Tq, Tk, q_offset)))
        return o, lse

    def dq_rows(self, q, k, v, dout, idx, scale: float, causal: bool, q_offset=None):
        """dq rows for query rows idx = [(b, h, i), ...]: [n, D]."""
        q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
        B, Hq, Hkv, Tq, Tk, D = _shapes(q, k, v, dout)
        ix = _idx(idx)
        dq = np.zeros((len(ix), D))
        _check(self.lib.oracle_dq_rows(_p(q), _p(k), _p(v), _p(dout), ix.ctypes.data_as(_ip),
                                       len(ix), _p(dq), B, Hq, Hkv, Tq, Tk, D, float(scale),
                                       int(bool(causal)), _offset(Tq, Tk, q_offset)))
        return dq

    def dkdv_rows(self, q, k, v, dout, idx, scale: float, causal: bool, q_offset=None):
        """dk and dv rows for key rows idx = [(b, hkv, j), ...]: ([n, D], [n, D])."""
        q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
        B, Hq, Hkv, Tq, Tk, D = _shapes(q, k, v, dout)
        ix = _idx(idx)
        dk = np.zeros((len(ix), D))
        dv = np.zeros((len(ix), D))
        _check(self.lib.oracle_dkdv_rows(_p(q), _p(k), _p(v), _p(dout), ix.ctypes.data_as(_ip),
                                         len(ix), _p(dk), _p(dv), B, Hq, Hkv, Tq, Tk, D,
                                         float(scale), int(bool(causal)),
                                         _offset(Tq, Tk, q_offset)))
        return dk, dv


_default = None


def default() -> Oracle:
    """The oracle built from this directory's source (built on first use if
    the library is missing or older than the source)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SOURCE):
            build()
        _default = Oracle(LIB_PATH)
    return _default


def fwd(q, k, v, scale: float, causal: bool, return_mag: bool = False, q_offset=None):
    return default().fwd(q, k, v, scale, causal, return_mag, q_offset)


def bwd(q, k, v, dout, scale: float, causal: bool, return_jac: bool = False,
        return_mag: bool = False, q_offset=None):
    return default().bwd(q, k, v, dout, scale, causal, return_jac, return_mag, q_offset)


def fwd_rows(q, k, v, idx, scale: float, causal: bool, q_offset=None):
    return default().fwd_rows(q, k, v, idx, scale, causal, q_offset)


def dq_rows(q, k, v, dout, idx, scale: float, causal: bool, q_offset=None):
    return default().dq_rows(q, k, v, dout, idx, scale, causal, q_offset)


def dkdv_rows(q, k, v, dout, idx, scale: float, causal: bool, q_offset=None):
    return default().dkdv_rows(q, k, v, dout, idx, scale, causal, q_offset)
