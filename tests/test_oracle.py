"""Pins of the fp64 oracle against what the pages and the mathematics fix.

None of these compares the oracle with itself: each value comes from a page
(golden fixtures, cited in their headers), a closed form, an invariant, brute
force (finite differences) or an independent library routine (PyTorch's CPU
scaled_dot_product_attention in float64).  CPU only.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import make_inputs


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def scalar_problem(scores, values):
    """One query with D = 1, q = 1 and scale = 1, so that s_j = k_j exactly."""
    n = len(scores)
    q = np.ones((1, 1, n, 1))
    k = np.asarray(scores, dtype=np.float64).reshape(1, 1, n, 1)
    v = np.asarray(values, dtype=np.float64).reshape(1, 1, n, 1)
    return q, k, v


# ---------------------------------------------------------------------------
# Worked examples printed on the pages
# ---------------------------------------------------------------------------

def test_worked_example_weights_and_running_sums(golden):
    """«La online softmax, con i numeri»: weights of s = (1,3,2,4), and the
    running sums l1 = 1.135 (block [1,3]) and l2 = 1.553 (whole row)."""
    g = golden("online_softmax_four_scores.txt")
    tol = 0.5 * 10 ** (-g["decimals"])
    s = g["scores"]
    # values e_j (D = 4) turn the output row into the weight row
    q = np.ones((1, 1, 4, 1))
    k = np.asarray(s).reshape(1, 1, 4, 1)
    eye = np.eye(4)
    # D of q/k is 1 but v needs D = 4: run one column at a time
    w = []
    for d in range(4):
        o, lse = oracle.fwd(q, k, eye[:, d].reshape(1, 1, 4, 1), 1.0, False)
        w.append(o[0, 0, 0, 0])
    np.testing.assert_allclose(w, g["weights"], atol=tol)
    assert abs(sum(w) - 1.0) < 1e-15
    # lse = m + ln l  =>  l = exp(lse - m)
    _, lse = oracle.fwd(*scalar_problem(s, [0.0] * 4), 1.0, False)
    assert abs(math.exp(lse[0, 0, 0] - g["block2_m"]) - g["block2_l"]) < tol
    _, lse1 = oracle.fwd(*scalar_problem(s[:2], [0.0] * 2), 1.0, False)
    assert abs(math.exp(lse1[0, 0, 0] - g["block1_m"]) - g["block1_l"]) < tol


def test_fig79_result(golden):
    """Fig. 7.9: o / l = 5.257 for the eight scores and values."""
    g = golden("fig79_eight_scores.txt")
    o, _ = oracle.fwd(*scalar_problem(g["scores"], g["values"]), 1.0, False)
    assert abs(o[0, 0, 0, 0] - g["result"]) < 0.5 * 10 ** (-g["decimals"])


def test_block_mean_counterexample(golden):
    """«Blockergebnisse einfach zu mitteln reicht nicht»: 0.75, not the 0.5
    that the mean of the per-block results would give."""
    g = golden("block_mean_counterexample.txt")
    o, _ = oracle.fwd(*scalar_problem(g["scores"], g["values"]), 1.0, False)
    assert abs(o[0, 0, 0, 0] - g["result"]) < 1e-15
    bs = int(g["block_size"])
    blocks = []
    for b0 in range(0, 4, bs):
        ob, _ = oracle.fwd(*scalar_problem(g["scores"][b0:b0 + bs], g["values"][b0:b0 + bs]),
                           1.0, False)
        blocks.append(ob[0, 0, 0, 0])
    np.testing.assert_allclose(blocks, g["block_results"], atol=1e-15)
    assert abs(np.mean(blocks) - g["naive_mean"]) < 1e-15
    assert abs(np.mean(blocks) - o[0, 0, 0, 0]) > 0.2


def online_model(scores, values, block):
    """Test-side scalar model of the online-softmax update of "L'attention
    fusionnée", «Le softmax en ligne» (and the note's u / l form): running max
    m, sum l and numerator u, rescaled by exp(m - m') when the max rises.
    Returns the per-block (m, l, alpha) trace and u / l."""
    m, l, u, trace = -math.inf, 0.0, 0.0, []
    for b0 in range(0, len(scores), block):
        s = scores[b0:b0 + block]
        v = values[b0:b0 + block]
        m_new = max(m, max(s))
        alpha = math.exp(m - m_new) if m != -math.inf else 0.0
        p = [math.exp(x - m_new) for x in s]
        l = l * alpha + sum(p)
        u = u * alpha + sum(pi * vi for pi, vi in zip(p, v))
        m = m_new
        trace.append((m, l, alpha))
    return trace, u / l


def test_online_rule_reproduces_pages_tables(golden):
    """The update rule the kernels use reproduces the pages' per-block numbers
    and agrees with the oracle's one-shot result."""
    g = golden("online_softmax_four_scores.txt")
    tol = 0.5 * 10 ** (-g["decimals"])
    trace, _ = online_model(g["scores"], [0.0] * 4, int(g["block_size"]))
    assert trace[0][0] == g["block1_m"] and abs(trace[0][1] - g["block1_l"]) < tol
    assert trace[1][0] == g["block2_m"] and abs(trace[1][1] - g["block2_l"]) < tol
    assert abs(trace[1][2] - g["alpha_block2"]) < tol

    g = golden("fig79_eight_scores.txt")
    trace, res = online_model(g["scores"], g["values"], int(g["block_size"]))
    rescaled = [i + 1 for i, (_, _, a) in enumerate(trace) if i > 0 and a < 1.0]
    assert rescaled == [int(x) for x in g["rescaled_blocks"]]
    for b in rescaled:
        assert abs(trace[b - 1][2] - g["alpha"]) < 0.5 * 10 ** (-g["decimals"])
    o, _ = oracle.fwd(*scalar_problem(g["scores"], g["values"]), 1.0, False)
    assert abs(res - o[0, 0, 0, 0]) < 1e-12


# ---------------------------------------------------------------------------
# Invariants and closed forms
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [True, False])
def test_rows_of_P_sum_to_one(causal):
    """A value column of ones comes out as ones: every row of P sums to 1."""
    q, k, v = rnd((2, 4, 37, 16), 1), rnd((2, 2, 37, 16), 2), rnd((2, 2, 37, 16), 3)
    v[..., 5] = 1.0
    o, _ = oracle.fwd(q, k, v, 0.3, causal)
    assert np.max(np.abs(o[..., 5] - 1.0)) < 1e-14


def test_causal_row_zero_is_v0():
    """With the causal mask, query 0 sees only key 0: o_0 = v_0 exactly and
    lse_0 = scale * <q_0, k_0>."""
    q, k, v = rnd((2, 6, 19, 8), 4), rnd((2, 3, 19, 8), 5), rnd((2, 3, 19, 8), 6)
    o, lse = oracle.fwd(q, k, v, 0.7, True)
    for h in range(6):
        hk = h // 2
        assert np.array_equal(o[:, h, 0, :], v[:, hk, 0, :])
        s00 = 0.7 * np.einsum("bd,bd->b", q[:, h, 0, :], k[:, hk, 0, :])
        np.testing.assert_allclose(lse[:, h, 0], s00, rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [True, False])
def test_uniform_scores_closed_form(causal):
    """Q = 0 makes every visible score 0: causal o_i = mean(v_0..v_i),
    lse_i = ln(i+1); non-causal o_i = mean(v), lse = ln T.  Backward:
    dK = 0, dV_j = sum_{i sees j} dO_i / n_i,
    dq_i = scale / n_i * sum_{j seen} <dO_i, v_j - o_i> k_j."""
    B, H, T, D, scale = 1, 2, 23, 5, 0.4
    q = np.zeros((B, H, T, D))
    k, v, do = rnd((B, H, T, D), 7), rnd((B, H, T, D), 8), rnd((B, H, T, D), 9)
    o, lse = oracle.fwd(q, k, v, scale, causal)
    dq, dk, dv = oracle.bwd(q, k, v, do, scale, causal)
    n = np.arange(1, T + 1) if causal else np.full(T, T)
    exp_o = np.zeros_like(o)
    exp_dv = np.zeros_like(v)
    exp_dq = np.zeros_like(q)
    for b in range(B):
        for h in range(H):
            for i in range(T):
                js = range(i + 1) if causal else range(T)
                exp_o[b, h, i] = np.mean(v[b, h, list(js)], axis=0)
            for i in range(T):
                js = list(range(i + 1)) if causal else list(range(T))
                for j in js:
                    exp_dv[b, h, j] += do[b, h, i] / n[i]
                    exp_dq[b, h, i] += scale / n[i] * np.dot(do[b, h, i], v[b, h, j] - exp_o[b, h, i]) * k[b, h, j]
    np.testing.assert_allclose(o, exp_o, atol=1e-13)
    np.testing.assert_allclose(lse, np.broadcast_to(np.log(n), lse.shape), atol=1e-13)
    assert np.max(np.abs(dk)) == 0.0
    np.testing.assert_allclose(dv, exp_dv, atol=1e-13)
    np.testing.assert_allclose(dq, exp_dq, atol=1e-12)


@pytest.mark.parametrize("shape", [(1, 1, 1, 5, 3), (1, 2, 1, 7, 5), (2, 4, 2, 9, 4)])
@pytest.mark.parametrize("causal", [True, False])
def test_gradients_match_finite_differences(shape, causal):
    """Brute force: central differences of the loss sum(O * dO) in every input
    element ("L'attention fusionnée", «La passe arrière» gives the equations;
    odd shapes as in «Un premier kernel plus lent»)."""
    B, Hq, Hkv, T, D = shape
    scale = 0.6
    q, k, v = rnd((B, Hq, T, D), 10), rnd((B, Hkv, T, D), 11), rnd((B, Hkv, T, D), 12)
    do = rnd((B, Hq, T, D), 13)
    dq, dk, dv = oracle.bwd(q, k, v, do, scale, causal)

    def loss(q_, k_, v_):
        o, _ = oracle.fwd(q_, k_, v_, scale, causal)
        return float(np.sum(o * do))

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = {"q": q, "k": k, "v": v}
            args_m = dict(args_p)
            args_p[name], args_m[name] = xp, xm
            fd[idx] = (loss(args_p["q"], args_p["k"], args_p["v"]) -
                       loss(args_m["q"], args_m["k"], args_m["v"])) / (2 * h)
        err = np.max(np.abs(fd - g) / np.maximum(1.0, np.abs(g)))
        assert err < 1e-7, (name, err)


def test_jacobian_term_equals_rowsum_dO_O():
    """The shortcut of «La passe arrière»: sum_j P_ij dP_ij = sum_d dO_id O_id.
    The oracle computes the left side from its definition; the right side
    uses the oracle's forward output."""
    q, k, v, do = rnd((2, 4, 45, 12), 14), rnd((2, 2, 45, 12), 15), rnd((2, 2, 45, 12), 16), rnd((2, 4, 45, 12), 17)
    for causal in (True, False):
        o, _ = oracle.fwd(q, k, v, 0.5, causal)
        *_, jac = oracle.bwd(q, k, v, do, 0.5, causal, return_jac=True)
        np.testing.assert_allclose(jac, np.sum(do * o, axis=-1), atol=1e-12)


@pytest.mark.parametrize("causal", [True, False])
def test_gqa_equals_mha_with_repeated_kv(causal):
    """Grouped-query attention: query head h reads kv head h // (Hq/Hkv).  The
    result equals multi-head attention on K/V repeated along heads, and dK/dV
    are the sums over each group of the repeated heads' gradients."""
    B, Hq, Hkv, T, D = 2, 6, 2, 21, 8
    q, k, v, do = rnd((B, Hq, T, D), 18), rnd((B, Hkv, T, D), 19), rnd((B, Hkv, T, D), 20), rnd((B, Hq, T, D), 21)
    G = Hq // Hkv
    kr, vr = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    o1, l1 = oracle.fwd(q, k, v, 0.35, causal)
    o2, l2 = oracle.fwd(q, kr, vr, 0.35, causal)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    dq1, dk1, dv1 = oracle.bwd(q, k, v, do, 0.35, causal)
    dq2, dk2, dv2 = oracle.bwd(q, kr, vr, do, 0.35, causal)
    np.testing.assert_array_equal(dq1, dq2)
    np.testing.assert_allclose(dk1, dk2.reshape(B, Hkv, G, T, D).sum(axis=2), atol=1e-13)
    np.testing.assert_allclose(dv1, dv2.reshape(B, Hkv, G, T, D).sum(axis=2), atol=1e-13)


def test_future_keys_do_not_leak():
    """«Atención causal»: changing k_j, v_j for j > i leaves o_i, lse_i and
    dq_i unchanged (bit for bit: masked keys never enter the sums)."""
    B, H, T, D = 1, 2, 30, 6
    q, k, v, do = rnd((B, H, T, D), 22), rnd((B, H, T, D), 23), rnd((B, H, T, D), 24), rnd((B, H, T, D), 25)
    i = 13
    k2, v2 = k.copy(), v.copy()
    k2[:, :, i + 1:] = rnd(k2[:, :, i + 1:].shape, 26)
    v2[:, :, i + 1:] = rnd(v2[:, :, i + 1:].shape, 27)
    o1, l1 = oracle.fwd(q, k, v, 0.5, True)
    o2, l2 = oracle.fwd(q, k2, v2, 0.5, True)
    assert np.array_equal(o1[:, :, :i + 1], o2[:, :, :i + 1])
    assert np.array_equal(l1[:, :, :i + 1], l2[:, :, :i + 1])
    dq1, _, _ = oracle.bwd(q, k, v, do, 0.5, True)
    dq2, _, _ = oracle.bwd(q, k2, v2, do, 0.5, True)
    assert np.array_equal(dq1[:, :, :i + 1], dq2[:, :, :i + 1])
    assert not np.array_equal(o1[:, :, i + 1:], o2[:, :, i + 1:])


def test_scale_moves_into_q():
    """f(q, k, scale) = f(scale * q, k, 1), and dq scales back by `scale`."""
    q, k, v, do = rnd((1, 3, 17, 7), 28), rnd((1, 3, 17, 7), 29), rnd((1, 3, 17, 7), 30), rnd((1, 3, 17, 7), 31)
    o1, l1 = oracle.fwd(q, k, v, 0.25, True)
    o2, l2 = oracle.fwd(0.25 * q, k, v, 1.0, True)
    np.testing.assert_allclose(o1, o2, atol=1e-14)
    np.testing.assert_allclose(l1, l2, atol=1e-14)
    dq1, dk1, dv1 = oracle.bwd(q, k, v, do, 0.25, True)
    dq2, dk2, dv2 = oracle.bwd(0.25 * q, k, v, do, 1.0, True)
    np.testing.assert_allclose(dq1, 0.25 * dq2, atol=1e-13)
    np.testing.assert_allclose(dk1, dk2, atol=1e-13)
    np.testing.assert_allclose(dv1, dv2, atol=1e-13)


def test_gradient_sums_over_keys():
    """Two identities of the softmax gradient, for every kv head:
    sum_j dk_j = 0 (each row of dS sums to zero) and
    sum_j dv_j = sum over the group's query heads of sum_i dO_i."""
    B, Hq, Hkv, T, D = 2, 4, 2, 33, 6
    q, k, v, do = rnd((B, Hq, T, D), 32), rnd((B, Hkv, T, D), 33), rnd((B, Hkv, T, D), 34), rnd((B, Hq, T, D), 35)
    for causal in (True, False):
        _, dk, dv = oracle.bwd(q, k, v, do, 0.45, causal)
        assert np.max(np.abs(dk.sum(axis=2))) < 1e-12
        np.testing.assert_allclose(dv.sum(axis=2), do.reshape(B, Hkv, 2, T, D).sum(axis=(2, 3)), atol=1e-12)


# ---------------------------------------------------------------------------
# Independent library routine
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("case", [
    dict(B=1, Hq=1, Hkv=1, T=128, D=64, causal=True, scale=1 / 8),      # C1 shape
    dict(B=2, Hq=8, Hkv=8, T=512, D=64, causal=True, scale=1 / 8),      # C2 shape
    dict(B=1, Hq=4, Hkv=2, T=70, D=5, causal=False, scale=0.3),
    dict(B=1, Hq=3, Hkv=1, T=70, D=3, causal=True, scale=0.7),
])
def test_matches_torch_sdpa_float64(case):
    """PyTorch's CPU scaled_dot_product_attention in float64 (with autograd for
    the gradients) as an independent implementation ("FlashAttention:
    l'attenzione che non spreca memoria", «Cosa si guadagna (e cosa costa)»
    shows the call).  K/V are repeated along heads for GQA."""
    B, Hq, Hkv, T, D = (case[x] for x in ("B", "Hq", "Hkv", "T", "D"))
    inp = make_inputs(B, Hq, Hkv, T, D, torch.float64, seed=77)
    q, k, v, do = (inp[n] for n in ("q", "k", "v", "dout"))
    G = Hq // Hkv
    qt = q.clone().requires_grad_(True)
    kt = k.clone().requires_grad_(True)
    vt = v.clone().requires_grad_(True)
    ot = torch.nn.functional.scaled_dot_product_attention(
        qt, kt.repeat_interleave(G, dim=1), vt.repeat_interleave(G, dim=1),
        is_causal=case["causal"], scale=case["scale"])
    (ot * do).sum().backward()
    o, lse = oracle.fwd(q.numpy(), k.numpy(), v.numpy(), case["scale"], case["causal"])
    dq, dk, dv = oracle.bwd(q.numpy(), k.numpy(), v.numpy(), do.numpy(), case["scale"], case["causal"])
    np.testing.assert_allclose(o, ot.detach().numpy(), atol=1e-10)
    np.testing.assert_allclose(dq, qt.grad.numpy(), atol=1e-10)
    np.testing.assert_allclose(dk, kt.grad.numpy(), atol=1e-10)
    np.testing.assert_allclose(dv, vt.grad.numpy(), atol=1e-10)
    # lse against a direct logsumexp of the masked score matrix
    s = torch.einsum("bhid,bhjd->bhij", q, k.repeat_interleave(G, dim=1)) * case["scale"]
    if case["causal"]:
        s = s.masked_fill(torch.ones(T, T, dtype=torch.bool).triu(1), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, dim=-1).numpy(), atol=1e-12)


# ---------------------------------------------------------------------------
# Sampled-row entry points and edge cases
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [True, False])
def test_row_entry_points_match_full(causal):
    """The per-row entry points (used at sizes where the full oracle is too
    slow) give the same rows as the full computation."""
    B, Hq, Hkv, T, D = 2, 4, 2, 41, 9
    q, k, v, do = rnd((B, Hq, T, D), 36), rnd((B, Hkv, T, D), 37), rnd((B, Hkv, T, D), 38), rnd((B, Hq, T, D), 39)
    o, lse = oracle.fwd(q, k, v, 0.5, causal)
    dq, dk, dv = oracle.bwd(q, k, v, do, 0.5, causal)
    qi = [(0, 0, 0), (1, 3, 40), (0, 2, 17), (1, 1, 5)]
    oo, ll = oracle.fwd_rows(q, k, v, qi, 0.5, causal)
    dqr = oracle.dq_rows(q, k, v, do, qi, 0.5, causal)
    for n, (b, h, i) in enumerate(qi):
        np.testing.assert_allclose(oo[n], o[b, h, i], atol=1e-14)
        assert abs(ll[n] - lse[b, h, i]) < 1e-14
        np.testing.assert_allclose(dqr[n], dq[b, h, i], atol=1e-14)
    ki = [(0, 0, 0), (1, 1, 40), (0, 1, 22)]
    dkr, dvr = oracle.dkdv_rows(q, k, v, do, ki, 0.5, causal)
    for n, (b, hk, j) in enumerate(ki):
        np.testing.assert_allclose(dkr[n], dk[b, hk, j], atol=1e-13)
        np.testing.assert_allclose(dvr[n], dv[b, hk, j], atol=1e-13)


def test_empty_sequence_is_a_no_op():
    z = np.zeros((1, 2, 0, 4))
    o, lse = oracle.fwd(z, z, z, 0.5, True)
    assert o.shape == (1, 2, 0, 4) and lse.shape == (1, 2, 0)
    dq, dk, dv = oracle.bwd(z, z, z, z, 0.5, True)
    assert dq.shape == z.shape


def test_bad_shapes_are_rejected():
    q = np.zeros((1, 3, 4, 2))
    k = np.zeros((1, 2, 4, 2))
    with pytest.raises(ValueError):
        oracle.fwd(q, k, k, 1.0, True)
    with pytest.raises(RuntimeError):
        oracle.fwd_rows(np.zeros((1, 2, 4, 2)), k, k, [(0, 0, 4)], 1.0, True)


def test_term_magnitudes():
    """The oracle's per-element sums of absolute terms: at least |value|,
    equal to it when every term has one sign, and equal to a brute-force
    numpy evaluation of sum |terms| on a tiny case."""
    B, Hq, Hkv, T, D, scale = 1, 2, 1, 9, 3, 0.7
    q, k, v, do = rnd((B, Hq, T, D), 40), rnd((B, Hkv, T, D), 41), rnd((B, Hkv, T, D), 42), rnd((B, Hq, T, D), 43)
    for causal in (True, False):
        o, _, om = oracle.fwd(q, k, v, scale, causal, return_mag=True)
        dq, dk, dv, (mq, mk, mv) = oracle.bwd(q, k, v, do, scale, causal, return_mag=True)
        for val, mag in ((o, om), (dq, mq), (dk, mk), (dv, mv)):
            assert np.all(mag >= np.abs(val) - 1e-14)
        o2, _, om2 = oracle.fwd(q, k, np.abs(v), scale, causal, return_mag=True)
        np.testing.assert_allclose(om2, o2, rtol=1e-14)
        _, _, dv2, (_, _, mv2) = oracle.bwd(q, k, v, np.abs(do), scale, causal, return_mag=True)
        np.testing.assert_allclose(mv2, dv2, rtol=1e-14)
        # brute force with full matrices, one query head at a time
        mask = np.tril(np.ones((T, T), bool)) if causal else np.ones((T, T), bool)
        mk_bf = np.zeros_like(mk)
        for h in range(Hq):
            s = np.where(mask, scale * q[0, h] @ k[0, 0].T, -np.inf)
            p = np.exp(s - s.max(1, keepdims=True))
            p /= p.sum(1, keepdims=True)
            dp = do[0, h] @ v[0, 0].T
            ds = p * (dp - (p * dp).sum(1, keepdims=True))
            np.testing.assert_allclose(mq[0, h], scale * np.abs(ds) @ np.abs(k[0, 0]), rtol=1e-12)
            np.testing.assert_allclose(om[0, h], p @ np.abs(v[0, 0]), rtol=1e-12)
            mk_bf[0, 0] += scale * np.abs(ds).T @ np.abs(q[0, h])
        np.testing.assert_allclose(mk, mk_bf, rtol=1e-12)


def test_kdk_equals_dqq():
    """K^T dK = dQ^T Q per kv group (both are scale * sum_ij dS_ij k_j q_i^T);
    the full-size GPU checks rely on this identity."""
    B, Hq, Hkv, T, D = 1, 4, 2, 50, 8
    q, k, v, do = rnd((B, Hq, T, D), 44), rnd((B, Hkv, T, D), 45), rnd((B, Hkv, T, D), 46), rnd((B, Hq, T, D), 47)
    for causal in (True, False):
        dq, dk, _ = oracle.bwd(q, k, v, do, 0.3, causal)
        lhs = np.einsum("bhtd,bhte->bhde", k, dk)
        rhs = np.einsum("bhgtd,bhgte->bhde", dq.reshape(B, Hkv, 2, T, D), q.reshape(B, Hkv, 2, T, D))
        np.testing.assert_allclose(lhs, rhs, atol=1e-12)


# ---------------------------------------------------------------------------
# Query rows against a longer (or shorter) key sequence, causal offset
# ("Optimización de Flash Attention ...", «Parte 1»: the kernel takes a
# position offset for the causal mask, input_pos; "L'attention fusionnée",
# «Un premier kernel plus lent»: one query against 70 positions, as in
# generation).  Query row i stands at position i + q_offset among the keys and
# sees key j iff j <= i + q_offset; the default offset is Tk - Tq.
# ---------------------------------------------------------------------------

def sdpa_masked(q, k, v, do, scale, causal, off):
    """PyTorch float64 SDPA with an explicit boolean mask, and autograd."""
    G = q.shape[1] // k.shape[1]
    Tq, Tk = q.shape[2], k.shape[2]
    qt, kt, vt = (torch.from_numpy(x).clone().requires_grad_(True) for x in (q, k, v))
    mask = None
    if causal:
        i = torch.arange(Tq)[:, None]
        j = torch.arange(Tk)[None, :]
        mask = j <= i + off
    ot = torch.nn.functional.scaled_dot_product_attention(
        qt, kt.repeat_interleave(G, dim=1), vt.repeat_interleave(G, dim=1), attn_mask=mask,
        scale=scale)
    (ot * torch.from_numpy(do)).sum().backward()
    return ot.detach().numpy(), qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy()


@pytest.mark.parametrize("D", [5, 3])
def test_single_query_against_70_keys(D):
    """One query against 70 positions (the page's generation-shaped test, with
    its head sizes 5 and 3): with the default offset the query stands after
    every key, so causal and non-causal attention agree, and both match
    PyTorch's float64 SDPA over all keys."""
    q, k, v, do = rnd((1, 1, 1, D), 40), rnd((1, 1, 70, D), 41), rnd((1, 1, 70, D), 42), rnd((1, 1, 1, D), 43)
    oc, lc = oracle.fwd(q, k, v, 0.5, True)
    on, ln = oracle.fwd(q, k, v, 0.5, False)
    np.testing.assert_array_equal(oc, on)
    np.testing.assert_array_equal(lc, ln)
    ot, dqt, dkt, dvt = sdpa_masked(q, k, v, do, 0.5, False, 0)
    np.testing.assert_allclose(oc, ot, atol=1e-12)
    dq, dk, dv = oracle.bwd(q, k, v, do, 0.5, True)
    np.testing.assert_allclose(dq, dqt, atol=1e-12)
    np.testing.assert_allclose(dk, dkt, atol=1e-12)
    np.testing.assert_allclose(dv, dvt, atol=1e-12)
    # with offset 0 the single query sees key 0 only: o = v_0 exactly
    o0, l0 = oracle.fwd(q, k, v, 0.5, True, q_offset=0)
    np.testing.assert_array_equal(o0[0, 0, 0], v[0, 0, 0])
    assert abs(l0[0, 0, 0] - 0.5 * float(np.dot(q[0, 0, 0], k[0, 0, 0]))) < 1e-15


@pytest.mark.parametrize("Tq,Tk", [(3, 8), (5, 5), (1, 9), (7, 20)])
def test_bottom_right_rows_are_the_last_rows_of_the_square_problem(Tq, Tk):
    """With the default offset the Tq query rows are the last Tq rows of the
    square causal problem over the same keys: o, lse and dq equal those rows,
    and dk, dv equal the square problem's with dO = 0 on its first Tk - Tq rows
    (rows that then add nothing to any gradient)."""
    B, Hq, Hkv, D = 1, 4, 2, 6
    qs, k, v, dos = rnd((B, Hq, Tk, D), 44), rnd((B, Hkv, Tk, D), 45), rnd((B, Hkv, Tk, D), 46), rnd((B, Hq, Tk, D), 47)
    dos[:, :, :Tk - Tq] = 0.0
    o_sq, lse_sq = oracle.fwd(qs, k, v, 0.45, True)
    dq_sq, dk_sq, dv_sq = oracle.bwd(qs, k, v, dos, 0.45, True)
    q, do = qs[:, :, Tk - Tq:].copy(), dos[:, :, Tk - Tq:].copy()
    o, lse = oracle.fwd(q, k, v, 0.45, True)
    dq, dk, dv = oracle.bwd(q, k, v, do, 0.45, True)
    np.testing.assert_allclose(o, o_sq[:, :, Tk - Tq:], atol=1e-14)
    np.testing.assert_allclose(lse, lse_sq[:, :, Tk - Tq:], atol=1e-14)
    np.testing.assert_allclose(dq, dq_sq[:, :, Tk - Tq:], atol=1e-13)
    np.testing.assert_allclose(dk, dk_sq, atol=1e-13)
    np.testing.assert_allclose(dv, dv_sq, atol=1e-13)


@pytest.mark.parametrize("case", [
    dict(B=1, Hq=2, Hkv=1, Tq=4, Tk=9, off=None, causal=True),
    dict(B=1, Hq=1, Hkv=1, Tq=4, Tk=9, off=1, causal=True),
    dict(B=2, Hq=2, Hkv=2, Tq=6, Tk=3, off=0, causal=True),
    dict(B=1, Hq=2, Hkv=1, Tq=5, Tk=7, off=None, causal=False),
])
def test_kv_gradients_match_finite_differences(case):
    """Brute force with Tq != Tk and several offsets: central differences of
    sum(O * dO) in every input element."""
    B, Hq, Hkv, Tq, Tk = (case[x] for x in ("B", "Hq", "Hkv", "Tq", "Tk"))
    D, scale, causal, off = 3, 0.8, case["causal"], case["off"]
    q, k, v, do = rnd((B, Hq, Tq, D), 48), rnd((B, Hkv, Tk, D), 49), rnd((B, Hkv, Tk, D), 50), rnd((B, Hq, Tq, D), 51)
    grads = oracle.bwd(q, k, v, do, scale, causal, q_offset=off)

    def loss(*a):
        return float(np.sum(oracle.fwd(*a, scale, causal, q_offset=off)[0] * do))

    h = 1e-6
    for which, x in enumerate((q, k, v)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            args_p, args_m = [q, k, v], [q, k, v]
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p[which], args_m[which] = xp, xm
            fd[idx] = (loss(*args_p) - loss(*args_m)) / (2 * h)
        err = np.max(np.abs(fd - grads[which]) / np.maximum(1.0, np.abs(grads[which])))
        assert err < 1e-7, (which, err)


@pytest.mark.parametrize("case", [
    dict(Hq=4, Hkv=2, Tq=33, Tk=70, D=5, off=None),
    dict(Hq=3, Hkv=1, Tq=70, Tk=70, D=3, off=0),
    dict(Hq=2, Hkv=2, Tq=20, Tk=50, D=8, off=7),
    dict(Hq=2, Hkv=1, Tq=40, Tk=25, D=4, off=3),
])
def test_kv_matches_torch_sdpa_with_explicit_mask(case):
    """PyTorch's float64 SDPA with the mask j <= i + offset written out as a
    boolean matrix, with autograd for the gradients."""
    Hq, Hkv, Tq, Tk, D, off = (case[x] for x in ("Hq", "Hkv", "Tq", "Tk", "D", "off"))
    q, k, v, do = rnd((1, Hq, Tq, D), 52), rnd((1, Hkv, Tk, D), 53), rnd((1, Hkv, Tk, D), 54), rnd((1, Hq, Tq, D), 55)
    o, lse = oracle.fwd(q, k, v, 0.6, True, q_offset=off)
    dq, dk, dv = oracle.bwd(q, k, v, do, 0.6, True, q_offset=off)
    ot, dqt, dkt, dvt = sdpa_masked(q, k, v, do, 0.6, True, Tk - Tq if off is None else off)
    np.testing.assert_allclose(o, ot, atol=1e-12)
    np.testing.assert_allclose(dq, dqt, atol=1e-12)
    np.testing.assert_allclose(dk, dkt, atol=1e-12)
    np.testing.assert_allclose(dv, dvt, atol=1e-12)


def test_rows_without_a_visible_key():
    """A negative offset leaves the first rows without any visible key: the
    oracle defines their output as 0 and their lse as -inf, and they add
    nothing to any gradient; the other rows are unaffected."""
    q, k, v, do = rnd((1, 1, 6, 4), 56), rnd((1, 1, 6, 4), 57), rnd((1, 1, 6, 4), 58), rnd((1, 1, 6, 4), 59)
    o, lse = oracle.fwd(q, k, v, 0.5, True, q_offset=-2)
    assert np.all(o[0, 0, :2] == 0.0) and np.all(np.isneginf(lse[0, 0, :2]))
    dq, dk, dv = oracle.bwd(q, k, v, do, 0.5, True, q_offset=-2)
    assert np.all(dq[0, 0, :2] == 0.0)
    ot, dqt, dkt, dvt = sdpa_masked(q[:, :, 2:].copy(), k, v, do[:, :, 2:].copy(), 0.5, True, 0)
    np.testing.assert_allclose(o[:, :, 2:], ot, atol=1e-12)
    np.testing.assert_allclose(dq[:, :, 2:], dqt, atol=1e-12)
    np.testing.assert_allclose(dk, dkt, atol=1e-12)
    np.testing.assert_allclose(dv, dvt, atol=1e-12)


def test_kv_row_entry_points_match_full():
    """The per-row entry points with Tq != Tk and an explicit offset."""
    B, Hq, Hkv, Tq, Tk, D, off = 1, 4, 2, 23, 57, 7, 20
    q, k, v, do = rnd((B, Hq, Tq, D), 60), rnd((B, Hkv, Tk, D), 61), rnd((B, Hkv, Tk, D), 62), rnd((B, Hq, Tq, D), 63)
    o, lse = oracle.fwd(q, k, v, 0.5, True, q_offset=off)
    dq, dk, dv = oracle.bwd(q, k, v, do, 0.5, True, q_offset=off)
    qi = [(0, 0, 0), (0, 3, 22), (0, 2, 9)]
    oo, ll = oracle.fwd_rows(q, k, v, qi, 0.5, True, q_offset=off)
    dqr = oracle.dq_rows(q, k, v, do, qi, 0.5, True, q_offset=off)
    for n, (b, h, i) in enumerate(qi):
        np.testing.assert_allclose(oo[n], o[b, h, i], atol=1e-14)
        assert abs(ll[n] - lse[b, h, i]) < 1e-14
        np.testing.assert_allclose(dqr[n], dq[b, h, i], atol=1e-14)
    ki = [(0, 0, 0), (0, 1, 56), (0, 1, 30)]
    dkr, dvr = oracle.dkdv_rows(q, k, v, do, ki, 0.5, True, q_offset=off)
    for n, (b, hk, j) in enumerate(ki):
        np.testing.assert_allclose(dkr[n], dk[b, hk, j], atol=1e-13)
        np.testing.assert_allclose(dvr[n], dv[b, hk, j], atol=1e-13)
