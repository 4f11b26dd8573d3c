"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (the library's default tiles, one fa_fwd and one fa_bwd call;
C5-prefill: 4096 query rows against 16384 keys with the default causal
offset, through fa_fwd_kv and fa_bwd_kv).

The oracle cannot redo these in full, so it checks sampled rows it can afford
one by one: query rows (O, lse, dQ) spread over heads and positions, and key
rows near the end of the sequence (dK, dV), where few query rows see the key.
Every row, early keys included, is also held to identities that exact
gradients satisfy at any size, per kv group:
    sum_j dK_j = 0                  (each row of dS sums to zero)
    sum_j dV_j = sum_i dO_i         (each row of P sums to one)
    K^T dK = dQ^T Q                 (both equal scale * sum_ij dS_ij k_j q_i^T)
"""
import numpy as np
import pytest
import torch

import exact_attention_30_amd as fa
import oracle
from tests.gpu_util import BF16_MAX_ABS, BF16_REL_L2, assert_close, assert_lse_close, f64, say
from workloads import WORKLOADS, make_inputs, workload_inputs

pytestmark = pytest.mark.gpu

_cache = {}


def run(name):
    """Inputs (CPU) and GPU outputs (CPU copies) of one workload."""
    if name in _cache:
        return _cache[name]
    w = WORKLOADS[name]
    x = workload_inputs(w)
    d = {k: v.cuda() for k, v in x.items()}
    say(f"full-size {name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} Tq={w.T} Tk={w.Tkv} D={w.D} "
        f"causal={w.causal}")
    o, lse = fa.fwd(d["q"], d["k"], d["v"], scale=w.scale, causal=w.causal)
    out = {"o": o, "lse": lse}
    if w.backward:
        out["dq"], out["dk"], out["dv"] = fa.bwd(d["q"], d["k"], d["v"], o, d["dout"], lse,
                                                 scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    out = {k: v.cpu() for k, v in out.items()}
    del d
    torch.cuda.empty_cache()
    _cache.clear()
    _cache[name] = (w, x, out)
    return _cache[name]


def query_rows(w):
    T = w.T
    pos = sorted({0, 1, 63, 64, 127, 128, 129, 255, 256, T // 2 - 1, T // 2, T - 129, T - 128,
                  T - 65, T - 64, T - 2, T - 1})
    heads = sorted({0, w.Hq // 2, w.Hq - 1})
    return [(b, h, i) for b in sorted({0, w.B - 1}) for h in heads for i in pos if 0 <= i < T]


def head_slice(x, b, h0, h1):
    return x[b:b + 1, h0:h1].double().numpy()


@pytest.mark.parametrize("name", ["C3", "C4", "C5", "C5-prefill", "C5-d96"])
def test_forward_sampled_rows(name):
    w, x, out = run(name)
    G = w.Hq // w.Hkv
    got_o, got_l, ref_o, ref_l = [], [], [], []
    for b, h, i in query_rows(w):
        hk = h // G
        ro, rl = oracle.fwd_rows(head_slice(x["q"], b, h, h + 1), head_slice(x["k"], b, hk, hk + 1),
                                 head_slice(x["v"], b, hk, hk + 1), [(0, 0, i)], w.scale, w.causal)
        ref_o.append(ro[0])
        ref_l.append(rl[0])
        got_o.append(out["o"][b, h, i].double().numpy())
        got_l.append(float(out["lse"][b, h, i]))
    assert_close("O rows", np.array(got_o), np.array(ref_o), w.dtype)
    assert_lse_close(np.array(got_l), np.array(ref_l), w.dtype)


@pytest.mark.parametrize("name", ["C3", "C5", "C5-prefill", "C5-d96"])
def test_dq_sampled_rows(name):
    w, x, out = run(name)
    G = w.Hq // w.Hkv
    got, ref = [], []
    for b, h, i in query_rows(w):
        hk = h // G
        r = oracle.dq_rows(head_slice(x["q"], b, h, h + 1), head_slice(x["k"], b, hk, hk + 1),
                           head_slice(x["v"], b, hk, hk + 1), head_slice(x["dout"], b, h, h + 1),
                           [(0, 0, i)], w.scale, w.causal)
        ref.append(r[0])
        got.append(out["dq"][b, h, i].double().numpy())
    assert_close("dQ rows", np.array(got), np.array(ref), w.dtype)


@pytest.mark.parametrize("name", ["C3", "C5", "C5-prefill", "C5-d96"])
def test_dkdv_sampled_rows(name):
    w, x, out = run(name)
    G = w.Hq // w.Hkv
    T = w.Tkv
    keys = [T - 1, T - 2, T - 33, T - 64, T - 65, T - 100, T - 128]
    if name == "C3":  # short enough for early keys too
        keys += [0, 1, 63, 64, 1000]
    got_k, got_v, ref_k, ref_v = [], [], [], []
    for b in sorted({0, w.B - 1}):
        for hk in sorted({0, w.Hkv - 1}):
            rk, rv = oracle.dkdv_rows(head_slice(x["q"], b, hk * G, (hk + 1) * G),
                                      head_slice(x["k"], b, hk, hk + 1),
                                      head_slice(x["v"], b, hk, hk + 1),
                                      head_slice(x["dout"], b, hk * G, (hk + 1) * G),
                                      [(0, 0, j) for j in keys], w.scale, w.causal)
            ref_k.extend(rk)
            ref_v.extend(rv)
            got_k.extend(out["dk"][b, hk, keys].double().numpy())
            got_v.extend(out["dv"][b, hk, keys].double().numpy())
    assert_close("dK rows", np.array(got_k), np.array(ref_k), w.dtype)
    assert_close("dV rows", np.array(got_v), np.array(ref_v), w.dtype)


@pytest.mark.parametrize("name", ["C3", "C5", "C5-prefill", "C5-d96"])
def test_gradient_identities_all_rows(name):
    w, x, out = run(name)
    G = w.Hq // w.Hkv
    dk = out["dk"].double()
    dv = out["dv"].double()
    dq = out["dq"].double()
    q = x["q"].double()
    k = x["k"].double()
    do = x["dout"].double()
    B, Hkv, _, D = dk.shape
    T = w.T  # query rows
    # sum_j dK_j = 0, relative to the size of dK's columns
    s = dk.sum(dim=2)
    col = dk.norm(dim=2)
    assert float((s.abs() / col).max()) < 2e-2
    # sum_j dV_j = sum over the group's heads and rows of dO
    want = do.reshape(B, Hkv, G, T, D).sum(dim=(2, 3))
    col = dv.norm(dim=2)
    assert float(((dv.sum(dim=2) - want).abs() / col).max()) < 2e-2
    # K^T dK = sum over the group's heads of dQ^T Q
    lhs = torch.einsum("bhtd,bhte->bhde", k, dk)
    rhs = torch.einsum("bhgtd,bhgte->bhde", dq.reshape(B, Hkv, G, T, D), q.reshape(B, Hkv, G, T, D))
    rel = float((lhs - rhs).norm() / rhs.norm())
    assert rel < 1e-2, rel
    assert torch.isfinite(dq).all() and torch.isfinite(dk).all() and torch.isfinite(dv).all()


def dq_row_terms(qi, k, v, doi, oi, lse_i, scale):
    """For one causal query row (keys 0 .. len(k) - 1 visible): the magnitude
    scale sum_j |dS_ij k_jd| of dQ's terms, and the term through which the
    rounding of Delta (from the bf16 O) moves it, without the factor u (fp64)."""
    s = scale * (k @ qi)
    p = np.exp(s - lse_i)
    dp = v @ doi
    ds = p * (dp - p @ dp)
    mag = scale * np.abs(ds) @ np.abs(k)
    delta = scale * float(np.abs(doi * oi).sum()) * (p @ np.abs(k))
    return mag, delta


def test_long_sequence_sampled_rows():
    """One head at T = 100003 (ragged against every tile size, and long enough
    that a 32-bit product of two positions would overflow): forward and
    backward in the library's default configuration, sampled query rows (O,
    lse, dQ) and the last key rows (dK, dV) against the oracle.  dQ rows sum up
    to 10^5 terms whose dS add to zero; beyond the benchmark workloads they are
    held to the per-element rounding bound (with the Delta term), not to the
    whole-tensor rel-L2 target."""
    B, Hq, Hkv, T, D = 1, 2, 1, 100003, 64
    scale = 1 / 8
    x = make_inputs(B, Hq, Hkv, T, D, torch.bfloat16, seed=100003)
    d = {k: v.cuda() for k, v in x.items()}
    say(f"long sequence T={T} D={D}")
    o, lse = fa.fwd(d["q"], d["k"], d["v"], scale=scale, causal=True)
    dq, dk, dv = fa.bwd(d["q"], d["k"], d["v"], o, d["dout"], lse, scale=scale, causal=True)
    torch.cuda.synchronize()
    o, lse, dq, dk, dv = (t.cpu() for t in (o, lse, dq, dk, dv))
    del d
    q, k, v, do = (x[n][0].double().numpy() for n in ("q", "k", "v", "dout"))
    rows = [0, 1, 255, 256, 65535, 65536, 99999, T - 2, T - 1]
    for h in range(Hq):
        qh, dh = q[h][None, None], do[h][None, None]
        kh, vh = k[0][None, None], v[0][None, None]
        ro, rl = oracle.fwd_rows(qh, kh, vh, [(0, 0, i) for i in rows], scale, True)
        rdq = oracle.dq_rows(qh, kh, vh, dh, [(0, 0, i) for i in rows], scale, True)
        assert_close(f"O rows h{h}", o[0, h, rows].double().numpy(), ro, torch.bfloat16)
        assert_lse_close(lse[0, h, rows].double().numpy(), rl, torch.bfloat16)
        terms = [dq_row_terms(q[h, i], k[0, : i + 1], v[0, : i + 1], do[h, i], ro[n], rl[n], scale)
                 for n, i in enumerate(rows)]
        mag = np.array([t[0] for t in terms])
        extra = np.array([t[1] for t in terms])
        assert_close(f"dQ rows h{h}", dq[0, h, rows].double().numpy(), rdq, torch.bfloat16, mag,
                     extra, target_l2=False)
    keys = [T - 1, T - 2, T - 33, T - 64, T - 65, T - 200]
    rk, rv = oracle.dkdv_rows(q[None], k[0][None, None], v[0][None, None], do[None],
                              [(0, 0, j) for j in keys], scale, True)
    assert_close("dK rows", dk[0, 0, keys].double().numpy(), rk, torch.bfloat16)
    assert_close("dV rows", dv[0, 0, keys].double().numpy(), rv, torch.bfloat16)
