"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times: fa_fwd with its split scratch (the forward splits key ranges
when the shapes call for it) and fa_bwd (the dQ kernel forming Delta, then
dK/dV; both split when the shapes call for it); C5-prefill, 4096 query rows
against 16384 keys with the default causal offset, through the _kv calls.

Whole tensors against the oracle ("L'attention fusionnée", «Une opération
plutôt que trois»: the GPU result is checked against the plain CPU
definition), at the target tolerance with no magnitude bound:
  * C3: every element of O, lse, dQ, dK, dV;
  * C5, C5-prefill, C5-d96: every element of kv group 0: O, lse and dQ of its
    query heads at all rows, dK and dV of its kv head at all keys (each early
    key sums up to 4 x 16384 query rows);
  * C4 (forward only): O and lse of four whole heads.
Beyond kv group 0, sampled rows of other heads are compared with the oracle
one by one, and every row is held to identities that exact gradients satisfy
at any size, per kv group:
    sum_j dK_j = 0                  (each row of dS sums to zero)
    sum_j dV_j = sum_i dO_i         (each row of P sums to one)
    K^T dK = dQ^T Q                 (both equal scale * sum_ij dS_ij k_j q_i^T)
"""
import numpy as np
import pytest
import torch

import exact_attention_30_amd as fa
import oracle
from tests.gpu_util import Emulation, assert_close, assert_grad_close, assert_lse_close, f64, say
from workloads import WORKLOADS, make_inputs, workload_inputs

pytestmark = pytest.mark.gpu

_cache = {}


def run(name):
    """Inputs (CPU) and GPU outputs (CPU copies) of one workload, launched as
    the benchmark launches it."""
    if name in _cache:
        return _cache[name]
    w = WORKLOADS[name]
    x = workload_inputs(w)
    d = {k: v.cuda() for k, v in x.items()}
    say(f"full-size {name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} Tq={w.T} Tk={w.Tkv} D={w.D} "
        f"causal={w.causal}")
    fpart = torch.empty(max(fa.fwd_split_bytes(w.B, w.Hq, w.Hkv, w.T, w.Tkv, w.D, w.dtype), 16),
                        dtype=torch.uint8, device="cuda")
    o, lse = fa.fwd(d["q"], d["k"], d["v"], scale=w.scale, causal=w.causal, partial=fpart)
    out = {"o": o, "lse": lse}
    if w.backward:
        out["dq"], out["dk"], out["dv"] = fa.bwd(d["q"], d["k"], d["v"], o, d["dout"], lse,
                                                 scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    out = {k: v.cpu() for k, v in out.items()}
    del d, fpart
    torch.cuda.empty_cache()
    _cache.clear()
    _cache[name] = (w, x, out)
    return _cache[name]


def group_arrays(w, x, b, hk):
    """fp64 inputs of kv group hk of batch b: q, dout [1,G,T,D], k, v [1,1,Tk,D]."""
    G = w.Hq // w.Hkv
    sl = lambda t, h0, h1: t[b:b + 1, h0:h1].double().numpy()  # noqa: E731
    out = {"q": sl(x["q"], hk * G, (hk + 1) * G), "k": sl(x["k"], hk, hk + 1),
           "v": sl(x["v"], hk, hk + 1)}
    if "dout" in x:
        out["dout"] = sl(x["dout"], hk * G, (hk + 1) * G)
    return out


def test_c3_every_element():
    """C3 in full: every element of O, lse, dQ, dK, dV against the oracle."""
    w, x, out = run("C3")
    q, k, v, do = (x[n].double().numpy() for n in ("q", "k", "v", "dout"))
    ro, rl = oracle.fwd(q, k, v, w.scale, w.causal)
    rdq, rdk, rdv = oracle.bwd(q, k, v, do, w.scale, w.causal)
    assert_close("O", f64(out["o"]), ro, w.dtype)
    assert_lse_close(f64(out["lse"]), rl, w.dtype)
    assert_close("dQ", f64(out["dq"]), rdq, w.dtype)
    assert_close("dK", f64(out["dk"]), rdk, w.dtype)
    assert_close("dV", f64(out["dv"]), rdv, w.dtype)


@pytest.mark.parametrize("name", ["C5", "C5-prefill", "C5-d96"])
def test_kv_group0_every_element(name):
    """Every element of kv group 0: O, lse, dQ of its query heads at all rows;
    dK, dV of its kv head at all keys."""
    w, x, out = run(name)
    G = w.Hq // w.Hkv
    g = group_arrays(w, x, 0, 0)
    say(f"oracle on kv group 0 of {name}")
    ro, rl = oracle.fwd(g["q"], g["k"], g["v"], w.scale, w.causal)
    rdq, rdk, rdv = oracle.bwd(g["q"], g["k"], g["v"], g["dout"], w.scale, w.causal)
    # elements past the target are also compared with the emulation of the
    # method's bf16 roundings, computed for their rows only
    em = Emulation(g, rl, w.scale, w.causal)
    assert_close("O", f64(out["o"][:1, :G]), ro, w.dtype, em.o_rows)
    assert_lse_close(f64(out["lse"][:1, :G]), rl, w.dtype)
    assert_close("dQ", f64(out["dq"][:1, :G]), rdq, w.dtype, em.dq_rows)
    assert_close("dK", f64(out["dk"][:1, :1]), rdk, w.dtype, em.dk_rows)
    assert_close("dV", f64(out["dv"][:1, :1]), rdv, w.dtype, em.dv_rows)


def test_c4_whole_heads():
    """C4 (non-causal, forward only): O and lse of four whole heads."""
    w, x, out = run("C4")
    for h in (0, 5, 10, 15):
        say(f"oracle on C4 head {h}")
        g = group_arrays(w, x, 0, h)
        ro, rl = oracle.fwd(g["q"], g["k"], g["v"], w.scale, w.causal)
        assert_close(f"O head {h}", f64(out["o"][:1, h:h + 1]), ro, w.dtype)
        assert_lse_close(f64(out["lse"][:1, h:h + 1]), rl, w.dtype)


def sampled_groups(w):
    """(batch, kv head) groups beyond kv group 0 whose rows are sampled."""
    return [(b, hk) for b in sorted({0, w.B - 1}) for hk in sorted({w.Hkv // 2, w.Hkv - 1})
            if (b, hk) != (0, 0)]


def query_positions(w):
    T = w.T
    return sorted({0, 1, 63, 64, 127, 128, 129, 255, 256, T // 2 - 1, T // 2, T - 129, T - 128,
                   T - 65, T - 64, T - 2, T - 1})


@pytest.mark.parametrize("name", ["C4", "C5", "C5-prefill", "C5-d96"])
def test_forward_sampled_rows(name):
    """Sampled query rows of other kv groups: O and lse against the oracle
    (elements past the target also against the emulation of the method's
    bf16 roundings, gpu_util)."""
    w, x, out = run(name)
    G = w.Hq // w.Hkv
    pos = query_positions(w)
    for b, hk in sampled_groups(w):
        g = group_arrays(w, x, b, hk)
        idx = [(0, h, i) for h in range(G) for i in pos]
        ro, rl = oracle.fwd_rows(g["q"], g["k"], g["v"], idx, w.scale, w.causal)
        got_o = np.stack([out["o"][b, hk * G + h, i].double().numpy() for _, h, i in idx])
        got_l = np.array([float(out["lse"][b, hk * G + h, i]) for _, h, i in idx])
        em = Emulation(g, None, w.scale, w.causal)
        assert_close(f"O rows b{b} kv{hk}", got_o, ro, w.dtype,
                     lambda r: em.o_rows([idx[n] for n in r[:, 0]]))
        assert_lse_close(got_l, rl, w.dtype)


@pytest.mark.parametrize("name", ["C5", "C5-prefill", "C5-d96"])
def test_dq_sampled_rows(name):
    w, x, out = run(name)
    G = w.Hq // w.Hkv
    pos = query_positions(w)
    for b, hk in sampled_groups(w):
        g = group_arrays(w, x, b, hk)
        idx = [(0, h, i) for h in range(G) for i in pos]
        ref = oracle.dq_rows(g["q"], g["k"], g["v"], g["dout"], idx, w.scale, w.causal)
        got = np.stack([out["dq"][b, hk * G + h, i].double().numpy() for _, h, i in idx])
        em = Emulation(g, None, w.scale, w.causal)
        assert_close(f"dQ rows b{b} kv{hk}", got, ref, w.dtype,
                     lambda r: em.dq_rows([idx[n] for n in r[:, 0]]))


@pytest.mark.parametrize("name", ["C5", "C5-prefill", "C5-d96"])
def test_dkdv_sampled_rows(name):
    """Sampled keys of other kv groups, early ones (summed over every query
    row of the group) and late ones."""
    w, x, out = run(name)
    T = w.Tkv
    keys = [0, 1, 63, 64, 1000, T // 2, T - 1, T - 2, T - 33, T - 64, T - 65, T - 100, T - 128]
    for b, hk in sampled_groups(w):
        g = group_arrays(w, x, b, hk)
        idx = [(0, 0, j) for j in keys]
        rk, rv = oracle.dkdv_rows(g["q"], g["k"], g["v"], g["dout"], idx, w.scale, w.causal)
        em = Emulation(g, None, w.scale, w.causal)
        assert_close(f"dK rows b{b} kv{hk}", out["dk"][b, hk, keys].double().numpy(), rk, w.dtype,
                     lambda r: em.dk_rows([idx[n] for n in r[:, 0]]))
        assert_close(f"dV rows b{b} kv{hk}", out["dv"][b, hk, keys].double().numpy(), rv, w.dtype,
                     lambda r: em.dv_rows([idx[n] for n in r[:, 0]]))


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


def test_long_sequence_sampled_rows():
    """One head pair at T = 100003 (ragged against every tile size, and long
    enough that a 32-bit product of two positions would overflow): forward
    and backward in the library's default configuration; 49 sampled query rows
    (O, lse, dQ) and the last 200 keys (dK, dV) against the oracle.  Its dQ
    rows sum up to 10^5 terms; where the bf16 roundings of the method alone
    (Delta from the stored bf16 O) move them past the rel-L2 target, the
    target is applied against their emulation (gpu_util)."""
    from tests import bf16_emulation as em
    from tests import lazy_model

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
    rng = np.random.default_rng(100003)
    rows = sorted({0, 1, 255, 256, 65535, 65536, 99999, T - 2, T - 1}
                  | set(rng.integers(0, T, 40).tolist()))
    tail = list(range(T - 200, T))
    o_ref = np.zeros((Hq, T, D))
    l_ref = np.zeros((Hq, T))
    o_em = np.zeros((Hq, T, D))  # the emulated bf16 O of the rows that need it
    blocks = {i // lazy_model.BLOCK for i in rows + tail}
    for h in range(Hq):
        qh, dh = q[h][None, None], do[h][None, None]
        kh, vh = k[0][None, None], v[0][None, None]
        ro, rl = oracle.fwd_rows(qh, kh, vh, [(0, 0, i) for i in rows + tail], scale, True)
        o_ref[h, rows + tail], l_ref[h, rows + tail] = ro, rl
        o_em[h] = em.bf16(lazy_model.forward_head(q[h], k[0], v[0], scale, True, 0,
                                                  round_p=em.bf16, blocks=blocks)[0])
        rdq = oracle.dq_rows(qh, kh, vh, dh, [(0, 0, i) for i in rows], scale, True)
        assert_close(f"O rows h{h}", o[0, h, rows].double().numpy(), o_ref[h, rows], torch.bfloat16)
        assert_lse_close(lse[0, h, rows].double().numpy(), l_ref[h, rows], torch.bfloat16)
        edq = em.dq_rows(q[h], k[0], v[0], do[h], o_em[h], l_ref[h], scale, True, 0, rows)
        assert_grad_close(f"dQ rows h{h}", dq[0, h, rows].double().numpy(), rdq, edq)
    rk, rv = oracle.dkdv_rows(q[None], k[0][None, None], v[0][None, None], do[None],
                              [(0, 0, j) for j in tail], scale, True)
    ek, ev = em.dkdv_rows(q, k[0], v[0], do, o_em, l_ref, scale, True, 0, tail)
    assert_grad_close("dK rows", dk[0, 0, tail].double().numpy(), rk, ek)
    assert_grad_close("dV rows", dv[0, 0, tail].double().numpy(), rv, ev)
