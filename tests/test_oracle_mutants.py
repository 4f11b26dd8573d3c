"""Planted mistakes in the oracle must be caught by its pins.

Each mutant is the oracle's C source with one plausible slip (a dropped term,
a wrong sign, index or operand), compiled on the CPU into a temporary library.
A compact battery of the pins of test_oracle.py runs against it; the real
oracle passes every pin, and each mutant must fail at least one.  CPU only.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from tests.conftest import read_golden

MUTANTS = {
    "mask_off_by_one": [("return s->causal ? ((long)j <= (long)i + s->off) : 1;",
                         "return s->causal ? ((long)j < (long)i + s->off) : 1;")],
    "mask_reversed": [("return s->causal ? ((long)j <= (long)i + s->off) : 1;",
                       "return s->causal ? ((long)j >= (long)i + s->off) : 1;")],
    "offset_ignored": [("return s->causal ? ((long)j <= (long)i + s->off) : 1;",
                        "return s->causal ? ((long)j <= (long)i) : 1;")],
    "offset_sign": [("return s->causal ? ((long)j <= (long)i + s->off) : 1;",
                     "return s->causal ? ((long)j <= (long)i - s->off) : 1;")],
    "lse_sign": [("m + log(l)", "m - log(l)")],
    "no_normalisation": [("for (int j = 0; j < T; ++j) p[j] /= l;", "")],
    "scores_unscaled": [("s->scale * dot(q_i", "dot(q_i")],
    "gqa_modulo_map": [("const int G = s->Hq / s->Hkv, hk = h / G, D = s->D, T = s->Tk;\n"
                        "    const double* k_head = kvrow(k, s, b, hk, 0);\n"
                        "    const double* v_head = kvrow(v, s, b, hk, 0);\n"
                        "    double m, l;",
                        "const int hk = h % s->Hkv, D = s->D, T = s->Tk;\n"
                        "    const double* k_head = kvrow(k, s, b, hk, 0);\n"
                        "    const double* v_head = kvrow(v, s, b, hk, 0);\n"
                        "    double m, l;")],
    "jacobian_sign": [("c += p[j] * dp[j];", "c -= p[j] * dp[j];")],
    "dS_without_c": [("p[j] * (dp[j] - c)", "p[j] * dp[j]"),
                     ("pij * (dpij - cst[qr])", "pij * dpij")],
    "dq_unscaled": [("for (int d = 0; d < D; ++d) dq_i[d] *= scale;", "")],
    "dk_unscaled": [("for (int d = 0; d < D; ++d) dk_j[d] *= scale;", "")],
    "dv_uses_dS": [("dv_j[d] += pij * do_i[d];", "dv_j[d] += ds * do_i[d];")],
    "dk_uses_dO": [("dk_j[d] += ds * q_i[d];", "dk_j[d] += ds * do_i[d];")],
    "dq_uses_v": [("const double ds = p[j] * (dp[j] - c);\n"
                   "            const double* kj = kvrow(k, &s, b, hk, j);",
                   "const double ds = p[j] * (dp[j] - c);\n"
                   "            const double* kj = kvrow(v, &s, b, hk, j);")],
}


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def scalar_problem(scores, values):
    n = len(scores)
    return (np.ones((1, 1, n, 1)), np.asarray(scores, float).reshape(1, 1, n, 1),
            np.asarray(values, float).reshape(1, 1, n, 1))


def battery(orc) -> dict:
    """pin name -> passed?"""
    res = {}
    g = read_golden("fig79_eight_scores.txt")
    o, _ = orc.fwd(*scalar_problem(g["scores"], g["values"]), 1.0, False)
    res["fig79"] = abs(o[0, 0, 0, 0] - g["result"]) < 5e-4

    g = read_golden("block_mean_counterexample.txt")
    o, _ = orc.fwd(*scalar_problem(g["scores"], g["values"]), 1.0, False)
    res["block_mean"] = abs(o[0, 0, 0, 0] - g["result"]) < 1e-15

    g = read_golden("online_softmax_four_scores.txt")
    _, lse = orc.fwd(*scalar_problem(g["scores"], [0.0] * 4), 1.0, False)
    res["worked_l2"] = abs(math.exp(lse[0, 0, 0] - g["block2_m"]) - g["block2_l"]) < 5e-4

    q, k, v = rnd((1, 2, 9, 4), 1), rnd((1, 1, 9, 4), 2), rnd((1, 1, 9, 4), 3)
    o, _ = orc.fwd(q, k, v, 0.5, True)
    res["causal_row0"] = np.array_equal(o[:, :, 0], np.repeat(v[:, :, 0], 2, axis=1))

    T, D, scale = 11, 3, 0.4
    qz, k, v, do = np.zeros((1, 1, T, D)), rnd((1, 1, T, D), 4), rnd((1, 1, T, D), 5), rnd((1, 1, T, D), 6)
    o, lse = orc.fwd(qz, k, v, scale, True)
    dq, dk, dv = orc.bwd(qz, k, v, do, scale, True)
    n = np.arange(1, T + 1)
    exp_o = np.cumsum(v[0, 0], axis=0) / n[:, None]
    exp_dv = np.array([sum(do[0, 0, i] / n[i] for i in range(j, T)) for j in range(T)])
    exp_dq = np.array([scale / n[i] * sum(np.dot(do[0, 0, i], v[0, 0, j] - exp_o[i]) * k[0, 0, j]
                                          for j in range(i + 1)) for i in range(T)])
    res["closed_form"] = (np.allclose(o[0, 0], exp_o, atol=1e-13) and
                          np.allclose(lse[0, 0], np.log(n), atol=1e-13) and
                          np.max(np.abs(dk)) == 0 and np.allclose(dv[0, 0], exp_dv, atol=1e-13) and
                          np.allclose(dq[0, 0], exp_dq, atol=1e-12))

    ok = True
    for causal in (True, False):
        B, Hq, Hkv, T, D = 1, 4, 2, 6, 3
        q, k, v, do = rnd((B, Hq, T, D), 7), rnd((B, Hkv, T, D), 8), rnd((B, Hkv, T, D), 9), rnd((B, Hq, T, D), 10)
        grads = orc.bwd(q, k, v, do, 0.6, causal)
        h = 1e-6
        for which, x in enumerate((q, k, v)):
            fd = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                args_p = [q, k, v]
                args_m = [q, k, v]
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p[which], args_m[which] = xp, xm
                fd[idx] = (np.sum(orc.fwd(*args_p, 0.6, causal)[0] * do) -
                           np.sum(orc.fwd(*args_m, 0.6, causal)[0] * do)) / (2 * h)
            ok &= bool(np.max(np.abs(fd - grads[which])) < 1e-6)
    res["finite_differences"] = ok

    ok = True
    for causal in (True, False):
        B, Hq, Hkv, T, D = 1, 4, 2, 13, 5
        q, k, v = (torch.from_numpy(rnd((B, h, T, D), s)) for h, s in ((Hq, 11), (Hkv, 12), (Hkv, 13)))
        ot = torch.nn.functional.scaled_dot_product_attention(
            q, k.repeat_interleave(2, dim=1), v.repeat_interleave(2, dim=1), is_causal=causal,
            scale=0.5)
        o, _ = orc.fwd(q.numpy(), k.numpy(), v.numpy(), 0.5, causal)
        ok &= bool(np.allclose(o, ot.numpy(), atol=1e-10))
    res["sdpa"] = ok

    # bottom-right alignment: Tq queries against Tk keys with the default
    # offset Tk - Tq are the last Tq rows of the square causal problem
    # ("Optimización de Flash Attention ...", input_pos of «Parte 1»)
    Tq, Tk, D = 3, 8, 4
    kk, vv = rnd((1, 1, Tk, D), 14), rnd((1, 1, Tk, D), 15)
    qs = rnd((1, 1, Tk, D), 16)
    o_sq, lse_sq = orc.fwd(qs, kk, vv, 0.7, True)
    o_kv, lse_kv = orc.fwd(qs[:, :, Tk - Tq:], kk, vv, 0.7, True)
    res["kv_offset"] = (np.allclose(o_kv, o_sq[:, :, Tk - Tq:], atol=1e-14) and
                        np.allclose(lse_kv, lse_sq[:, :, Tk - Tq:], atol=1e-14))
    return res


def test_battery_passes_on_the_oracle():
    res = battery(oracle.default())
    assert all(res.values()), res


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    src = open(oracle.SOURCE).read()
    for old, new in MUTANTS[name]:
        assert old in src, f"mutation site of {name} not found"
        src = src.replace(old, new)
    path = os.path.join(tmp_path, f"{name}.c")
    with open(path, "w") as f:
        f.write(src)
    lib = oracle.build(path, os.path.join(tmp_path, f"lib{name}.so"))
    res = battery(oracle.Oracle(lib))
    assert not all(res.values()), f"mutant {name} passed every pin"
