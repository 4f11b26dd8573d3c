"""CPU emulation of the bf16 roundings of the recomputing backward — test-side
arithmetic, used only to explain tolerances; neither the oracle nor the
library.

The backward of "L'attention fusionnée" («La passe arrière») recomputes
P_ij = exp(s_ij - L_i) from the saved log-sum-exp, forms
Delta_i = sum_d dO_id O_id from the stored output, and
    dS_ij = P_ij (dP_ij - Delta_i),  dP_ij = <dO_i, v_j>,
    dq_i = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i,
    dv_j = sum_i P_ij dO_i.
With bf16 inputs the stored O is a bf16 number, and P and dS enter the
products rounded to bf16 ("Sur les Tensor Cores" of the same page packs the
weights to bf16).  This module applies exactly those roundings to exact (fp64)
quantities: O is the oracle's output rounded to bf16, L the oracle's lse, and
every sum is taken in fp64.  What it returns is the result of the pages'
method with bf16 operands and otherwise exact arithmetic, so its distance
from the oracle is the part of a kernel's error that these roundings alone
cause.

Arrays are per head, float64: q, do, o [Tq, D]; k, v [Tk, D]; lse [Tq].
Query row i sees key j iff j <= i + q_offset when causal.
"""
from __future__ import annotations

import numpy as np
import torch


def bf16(x) -> np.ndarray:
    """Round to the nearest bf16 (ties to even), back in float64."""
    return torch.from_numpy(np.asarray(x, dtype=np.float64)).to(torch.bfloat16).double().numpy()


def bf16_torch(x: torch.Tensor) -> torch.Tensor:
    """bf16 rounding of a float64 torch tensor, back in float64."""
    return x.to(torch.bfloat16).double()


def _visible(Tk: int, i: int, causal: bool, q_offset: int) -> int:
    """Number of keys row i sees (keys 0 .. n-1)."""
    return min(Tk, i + q_offset + 1) if causal else Tk


def dq_rows(q, k, v, do, o, lse, scale, causal, q_offset, rows, round_delta=True,
            round_operands=True):
    """dq for the given query rows of one head, with Delta from bf16(o)
    (round_delta) and P, dS rounded to bf16 (round_operands)."""
    Tk = k.shape[0]
    out = np.zeros((len(rows), q.shape[1]))
    for n, i in enumerate(rows):
        m = _visible(Tk, i, causal, q_offset)
        if m <= 0:
            continue
        kv, vv = k[:m], v[:m]
        p = np.exp(scale * (kv @ q[i]) - lse[i])
        dp = vv @ do[i]
        oi = bf16(o[i]) if round_delta else o[i]
        delta = float(do[i] @ oi) if round_delta else float(p @ dp)
        ds = p * (dp - delta)
        if round_operands:
            ds = bf16(ds)
        out[n] = scale * (ds @ kv)
    return out


def dkdv_rows(q, k, v, do, o, lse, scale, causal, q_offset, keys, round_delta=True,
              round_operands=True):
    """dk, dv for the given keys of one kv head.  q, do, o: [G, Tq, D] (the
    query heads of its group), lse [G, Tq]; k, v: [Tk, D]."""
    G, Tq, D = q.shape
    dk = np.zeros((len(keys), D))
    dv = np.zeros((len(keys), D))
    for g in range(G):
        oi = bf16(o[g]) if round_delta else o[g]
        for n, j in enumerate(keys):
            # rows that see key j: j <= i + q_offset
            i0 = max(0, j - q_offset) if causal else 0
            if i0 >= Tq:
                continue
            qs, dos = q[g, i0:], do[g, i0:]
            p = np.exp(scale * (qs @ k[j]) - lse[g, i0:])
            dp = dos @ v[j]
            if round_delta:
                delta = np.sum(dos * oi[i0:], axis=1)
            else:
                # the Jacobian term needs whole rows of P: exact Delta = <dO, O>
                delta = np.sum(dos * o[g, i0:], axis=1)
            ds = p * (dp - delta)
            pr = bf16(p) if round_operands else p
            if round_operands:
                ds = bf16(ds)
            dk[n] += scale * (ds @ qs)
            dv[n] += pr @ dos
    return dk, dv


def rel_l2(got, ref) -> float:
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    den = float(np.linalg.norm(ref.ravel()))
    err = float(np.linalg.norm((got - ref).ravel()))
    return err / den if den > 0 else err
