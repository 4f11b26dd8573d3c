"""Helpers shared by the GPU tests: device inputs, metrics, tolerances."""
import sys

import numpy as np
import torch

# Tolerances.  bf16 inputs: max-abs <= 1e-2 and relative L2 <= 5e-3 on O and
# the gradients; fp32 inputs: max-abs <= 1e-5.  The outputs of the bf16 path
# are bf16 numbers, which are 2^-5 apart between 4 and 8: rounding a value of
# that size can alone move it by more than 1e-2.  The max-abs bound is
# therefore read as |got - ref| <= tol * max(1, |ref|): absolute for values up
# to 1, relative above.  The same reading is applied to the fp32 path.
# lse (not fixed by the target): 1e-3 for bf16 inputs, 1e-5 for fp32 (scores
# of exactly-representable products accumulate in fp32 on both paths).
#
# That bound is the target on the benchmark workloads.  Shapes beyond them
# (other scales, ragged lengths) can hold outputs that are sums of large terms
# of both signs; there the bf16 rounding of P and dS before the matrix cores
# (unit roundoff u = 2^-8) bounds the error by u * (M + |ref|), where M is the
# sum of the absolute values of the element's terms (returned by the oracle).
# For those cases an element passes if it meets either bound.
#
# The backward's Delta_i = sum_d dO_id O_id is formed from the kernel's own bf16
# O ("L'attention fusionnée", «La passe arrière»), whose rounding moves Delta by
# up to u * a_i, a_i = sum_d |dO_id O_id|; through dS_ij = P_ij (dP_ij - Delta_i)
# that reaches dQ_id as scale * sum_j P_ij |k_jd| * u a_i and dK_jd as
# scale * sum_i P_ij u a_i |q_id|.  Where P is peaked (large scores) those terms
# are not covered by the term magnitudes above, so the tests that reach such
# scales add them (delta_terms) to the rounding bound.
BF16_UNIT_ROUNDOFF = 2.0 ** -8
BF16_MAX_ABS = 1e-2
BF16_REL_L2 = 5e-3
FP32_MAX_ABS = 1e-5
LSE_TOL = {torch.bfloat16: 1e-3, torch.float32: 1e-5}


def say(msg: str):
    """Name the case before a GPU step, flushed, so a fault can be traced."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(inputs: dict) -> dict:
    return {k: v.cuda() for k, v in inputs.items()}


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def metrics(got: np.ndarray, ref: np.ndarray):
    """(max over elements of |err| / max(1, |ref|), relative L2 error)."""
    err = got - ref
    max_abs = float(np.max(np.abs(err) / np.maximum(1.0, np.abs(ref)))) if err.size else 0.0
    den = float(np.linalg.norm(ref.ravel()))
    rel_l2 = float(np.linalg.norm(err.ravel()) / den) if den > 0 else float(np.linalg.norm(err.ravel()))
    return max_abs, rel_l2


def delta_terms(q, k, do, o, lse, scale, causal, q_offset=None):
    """The dQ and dK terms through which the rounding of Delta (from the bf16 O)
    can move the gradients, per element, without the factor u (fp64; q, k, do,
    o, lse: the oracle's inputs and outputs)."""
    B, Hq, Tq, D = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    off = Tk - Tq if q_offset is None else q_offset
    a = np.abs(do * o).sum(-1)  # [B, Hq, Tq]
    tq = np.zeros(q.shape)
    tk = np.zeros(k.shape)
    for b in range(B):
        for h in range(Hq):
            s = scale * q[b, h] @ k[b, h // G].T
            if causal:
                s = np.where(np.arange(Tk)[None, :] <= np.arange(Tq)[:, None] + off, s, -np.inf)
            P = np.exp(s - lse[b, h][:, None])
            tq[b, h] = scale * a[b, h][:, None] * (P @ np.abs(k[b, h // G]))
            tk[b, h // G] += scale * (P * a[b, h][:, None]).T @ np.abs(q[b, h])
    return tq, tk


def assert_close(name: str, got, ref, dtype, mag=None, extra=None, target_l2=True):
    """Check got against the oracle's ref; `mag` (bf16 only) enables the
    rounding bound u * (mag + |ref|) as an alternative per-element bound, to
    which `extra` (per element, without the factor u) is added.  target_l2=False
    (shapes beyond the benchmark workloads, with `mag`) drops the whole-tensor
    rel-L2 target and keeps the per-element bounds."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    max_abs, rel_l2 = metrics(got, ref)
    if dtype == torch.float32:
        assert max_abs <= FP32_MAX_ABS, f"{name}: max-abs {max_abs:.3e} > {FP32_MAX_ABS}"
        return max_abs, rel_l2
    assert rel_l2 <= BF16_REL_L2 or (mag is not None and not target_l2), \
        f"{name}: rel-L2 {rel_l2:.3e} > {BF16_REL_L2}"
    if mag is None:
        assert max_abs <= BF16_MAX_ABS, f"{name}: max-abs {max_abs:.3e} > {BF16_MAX_ABS}"
    else:
        err = np.abs(got - ref)
        more = 0.0 if extra is None else np.asarray(extra)
        bound = np.maximum(BF16_MAX_ABS * np.maximum(1.0, np.abs(ref)),
                           BF16_UNIT_ROUNDOFF * (np.asarray(mag) + np.abs(ref) + more))
        worst = float(np.max(err / bound)) if err.size else 0.0
        assert worst <= 1.0, f"{name}: error {worst:.3f}x the per-element bound"
    return max_abs, rel_l2


def assert_lse_close(got, ref, dtype):
    err = float(np.max(np.abs(np.asarray(got, np.float64) - ref))) if np.size(ref) else 0.0
    assert err <= LSE_TOL[dtype], f"lse: max-abs {err:.3e} > {LSE_TOL[dtype]}"
    return err
