"""GPU parity of the fp8 (e4m3) forward (fa_fwd_fp8, fa_fp8_transpose_v,
fa_fwd_fp8_vt) against the fp64 oracle run on the exactly decoded inputs
(code times descale).

Tolerance, derived from the kernel's arithmetic.
  * Scores.  The e4m3 matrix instruction (v_mfma_f32_32x32x64_f8f6f4) forms
    the e4m3 products exactly and adds them in groups of eight: within a
    group the products are aligned to the largest one and bits below
    2^(e - 13) are dropped, e the exponent of that largest product; the group
    sums and the fp32 accumulator then add with fp32 rounding.  (Measured with
    an in-bounds probe of single instructions on chosen operands: with one
    product of 256-448 and seven of 2^-6 in its group, the seven vanish, with
    products 2^-5 apart from the same exponent they stay; a product shares
    its group with the seven others of the same 8-byte span of a lane's
    operand; patterns of N(0,1) codes come out exact.)  In this kernel's
    operand layout a group is 8 consecutive head dimensions, so a score moves
    by at most scale * (7 * 2^-13 * sum over those 8-dimension blocks of the
    block's largest |q_id k_jd| + 2^-22 * sum_d |q_id k_jd|), and lse, a
    weighted mean of its row's scores' moves, by at most the largest such
    move in its row (plus 1e-5 for its own fp32 arithmetic).
  * O uses the weights rounded to e4m3: relative to the row's reference a
    weight p lies in [0, 2^8]; rounded to nearest it moves by at most 2^-4 p
    (normal range, 3 mantissa bits) or 2^-10 (half the subnormal spacing
    2^-9).  With L >= l >= 1 the reference-relative and max-relative row sums,
        |O_id - O_ref| <= 2^-4 sum_j P_ij |v_jd| + 2^-10 sum_j |v_jd| / l_i
    plus the bf16 rounding of O (2^-9 |O|, taken as 2^-8 with the fp32 sums)
    and 1e-5.  The first term is the oracle's term magnitude; it also covers
    the P V products' group alignment (at most 7 * 2^-13 of each group's
    largest term) and the scores' moves above.
A layout mistake could hide under that bound, so a second test uses inputs
whose weights are exact powers of two (e4m3 then rounds nothing) and holds O
to bf16 rounding.
"""
import functools
import math
import zlib

import numpy as np
import pytest
import torch

import exact_attention_30_amd as fa
import oracle
from tests.gpu_util import f64, say
from workloads import WORKLOADS, make_fp8_inputs, workload_inputs

pytestmark = pytest.mark.gpu

E4M3_U = 2.0 ** -4      # unit roundoff of e4m3 (round to nearest even)
MFMA8_DROP = 7 * 2.0 ** -13  # group alignment: the 7 other products of a group, each < 2^-13 of its largest
MFMA8_GROUP = 8              # products per group = consecutive head dimensions in the kernel's layout
FP32_SUM = 2.0 ** -22        # fp32 rounding of the group sums and the accumulator
E4M3_SUB = 2.0 ** -10   # half the spacing of e4m3's subnormals
OUT_U = 2.0 ** -8       # bf16 rounding of O, with room for the fp32 sums

# name: (B, Hq, Hkv, Tq, Tk, D, causal, q_offset (None: Tk - Tq), scale)
CASES = {
    "t70_d64_causal": (1, 2, 2, 70, 70, 64, True, None, 1 / 8),
    "t129_d64_b2_gqa": (2, 2, 1, 129, 129, 64, True, None, 1 / 8),
    "t333_d128_full_gqa": (1, 4, 2, 333, 333, 128, False, None, 1 / math.sqrt(128)),
    "t1000_d128_causal_gqa4": (1, 4, 1, 1000, 1000, 128, True, None, 1 / math.sqrt(128)),
    "q1_k300_d128": (1, 2, 1, 1, 300, 128, True, None, 1 / math.sqrt(128)),
    "q300_k900_d64_off250_gqa": (1, 4, 2, 300, 900, 64, True, 250, 1 / 8),
    "q257_k513_d128_cross": (2, 2, 2, 257, 513, 128, False, None, 1 / math.sqrt(128)),
    "t64_d128_single_tile": (1, 1, 1, 64, 64, 128, True, None, 1 / math.sqrt(128)),
}


def real(x: torch.Tensor, descale: float) -> np.ndarray:
    """The real values of e4m3 codes (exact in fp64)."""
    return x.to(torch.float64).numpy() * descale


def case_inputs(name):
    B, Hq, Hkv, Tq, Tk, D, causal, off, scale = CASES[name]
    return make_fp8_inputs(B, Hq, Hkv, Tq, D, seed=zlib.crc32(name.encode()) % 100000, Tk=Tk)


def offset(name):
    B, Hq, Hkv, Tq, Tk, D, causal, off, scale = CASES[name]
    return Tk - Tq if off is None else off


def subnormal_term(q, k, v, scale, causal, off):
    """2^-10 sum_j |v_jd| / l_i per element, l_i the row sum of exp(s - max)
    over the visible keys (fp64)."""
    B, Hq, Tq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    out = np.zeros(q.shape)
    for b in range(B):
        for h in range(Hq):
            s = scale * q[b, h] @ k[b, h // G].T
            if causal:
                i = np.arange(Tq)[:, None]
                j = np.arange(k.shape[2])[None, :]
                s = np.where(j <= i + off, s, -np.inf)
            vis = np.isfinite(s)
            m = np.where(vis.any(1), np.max(np.where(vis, s, -np.inf), 1), 0.0)[:, None]
            l = np.where(vis, np.exp(np.where(vis, s, 0.0) - m), 0.0).sum(1)
            a = vis.astype(np.float64) @ np.abs(v[b, h // G])
            out[b, h] = E4M3_SUB * a / np.maximum(l, 1.0)[:, None]
    return out


def _block_max(x):
    """Largest |x| of each 8-dimension block of the last axis."""
    a = np.abs(x)
    return a.reshape(*a.shape[:-1], a.shape[-1] // MFMA8_GROUP, MFMA8_GROUP).max(axis=-1)


def score_bound(qi, kk, scale):
    """Largest move of the scores of one query row qi [D] against keys kk
    [n, D] (fp64), per key: scale * (7 * 2^-13 * sum over 8-dimension blocks
    of the block's largest |q k| + 2^-22 * sum |q k|), with the block's
    largest |q k| taken no larger than (largest |q|) (largest |k|) of the
    block."""
    return scale * (MFMA8_DROP * (_block_max(kk) @ _block_max(qi)) + FP32_SUM * (np.abs(kk) @ np.abs(qi)))


def lse_bound(q, k, scale, causal, off):
    """Per query row: the largest score move (score_bound) over its visible
    keys, plus 1e-5 (fp64)."""
    B, Hq, Tq, D = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    out = np.zeros((B, Hq, Tq))
    for b in range(B):
        for h in range(Hq):
            kk = k[b, h // G]
            sb = scale * (MFMA8_DROP * (_block_max(q[b, h]) @ _block_max(kk).T)
                          + FP32_SUM * (np.abs(q[b, h]) @ np.abs(kk).T))    # [Tq, Tk]
            if causal:
                vis = np.arange(Tk)[None, :] <= np.arange(Tq)[:, None] + off
                sb = np.where(vis, sb, 0.0)
            out[b, h] = sb.max(axis=1) + 1e-5
    return out


def assert_fp8_close(name, got, ref, mag, sub):
    bound = E4M3_U * mag + sub + OUT_U * np.abs(ref) + 1e-5
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    worst = float(np.max(err / bound)) if err.size else 0.0
    assert worst <= 1.0, f"{name}: error {worst:.3f}x the e4m3 bound"
    return worst


@functools.lru_cache(maxsize=None)
def reference(name):
    B, Hq, Hkv, Tq, Tk, D, causal, off, scale = CASES[name]
    x, ds = case_inputs(name)
    q, k, v = (real(x[n], ds) for n in ("q", "k", "v"))
    o, lse, om = oracle.fwd(q, k, v, scale, causal, return_mag=True, q_offset=offset(name))
    return o, lse, om, subnormal_term(q, k, v, scale, causal, offset(name))


@pytest.mark.parametrize("name", list(CASES))
def test_fp8_forward_matches_oracle(name):
    B, Hq, Hkv, Tq, Tk, D, causal, off, scale = CASES[name]
    x, ds = case_inputs(name)
    d = {n: t.cuda() for n, t in x.items()}
    say(f"fp8 fwd {name} B={B} Hq={Hq} Hkv={Hkv} Tq={Tq} Tk={Tk} D={D} causal={causal}")
    o, lse = fa.fwd_fp8(d["q"], d["k"], d["v"], ds, ds, ds, scale=scale, causal=causal,
                        q_offset=offset(name))
    torch.cuda.synchronize()
    ro, rl, om, sub = reference(name)
    assert o.dtype == torch.bfloat16
    assert_fp8_close(f"O {name}", f64(o), ro, om, sub)
    q, k = real(x["q"], ds), real(x["k"], ds)
    assert np.all(np.abs(f64(lse) - rl) <= lse_bound(q, k, scale, causal, offset(name)))


@pytest.mark.parametrize("D,causal", [(128, True), (64, False), (128, False)])
def test_fp8_exact_weights(D, causal):
    """Scores with c = scale * log2(e) = 1 that are small integers make every
    weight an exact power of two in e4m3's normal range (2^-4 .. 2^4 around
    the reference), so the kernel rounds no weight: O must match the oracle to
    bf16 rounding.  Query i is the one-hot e_(i mod D), key j holds integers
    0 .. -4, so the score of (i, j) is k_j[i mod D]; a wrong key or column
    order in any operand shows up at once."""
    B, Hq, Hkv, T = 1, 2, 1, 333
    g = torch.Generator().manual_seed(404 + D)
    q = torch.zeros(B, Hq, T, D)
    q[0, :, torch.arange(T), torch.arange(T) % D] = 1.0
    k = -torch.randint(0, 5, (B, Hkv, T, D), generator=g).to(torch.float32)
    v = torch.randn(B, Hkv, T, D, generator=g) * 16
    q8, k8, v8 = (t.to(torch.float8_e4m3fn) for t in (q, k, v))
    scale = math.log(2.0)  # with descales 1 (q, k) the base-2 score is the integer itself
    vd = 1 / 16
    say(f"fp8 exact weights D={D} causal={causal}")
    o, lse = fa.fwd_fp8(q8.cuda(), k8.cuda(), v8.cuda(), 1.0, 1.0, vd, scale=scale, causal=causal)
    torch.cuda.synchronize()
    ro, rl = oracle.fwd(real(q8, 1.0), real(k8, 1.0), real(v8, vd), scale, causal)
    err = np.abs(f64(o) - ro)
    assert float(np.max(err / (OUT_U * np.abs(ro) + 1e-5))) <= 1.0
    assert float(np.max(np.abs(f64(lse) - rl))) <= 1e-5


def vt_key(q: int) -> int:
    """Key held by byte q of a transposed tile row (the documented layout)."""
    return 32 * (q // 32) + 8 * ((q % 16) // 4) + 4 * ((q // 16) % 2) + q % 4


@pytest.mark.parametrize("Tk,D", [(70, 64), (129, 128), (64, 128)])
def test_fp8_transpose_layout(Tk, D):
    """fa_fp8_transpose_v writes, per kv head and 64-key tile t, D rows of 64
    bytes with byte q of row d = V[64t + vt_key(q)][d] and zeros past Tk:
    checked byte for byte."""
    B, Hkv = 2, 3
    x, _ = make_fp8_inputs(B, Hkv, Hkv, 1, D, seed=77 + Tk, Tk=Tk)
    v = x["v"]
    say(f"fp8 transpose Tk={Tk} D={D}")
    vt = fa.fp8_transpose_v(v.cuda())
    torch.cuda.synchronize()
    ntk = (Tk + 63) // 64
    got = vt[: B * Hkv * ntk * D * 64].cpu().view(B, Hkv, ntk, D, 64)
    codes = v.view(torch.uint8)
    pad = torch.zeros(B, Hkv, ntk * 64, D, dtype=torch.uint8)
    pad[:, :, :Tk] = codes
    perm = torch.tensor([vt_key(q) for q in range(64)])
    want = pad.view(B, Hkv, ntk, 64, D)[:, :, :, perm, :].transpose(3, 4)
    assert torch.equal(got, want)


def test_fp8_two_step_equals_one_call():
    """fa_fwd_fp8 is fa_fp8_transpose_v followed by fa_fwd_fp8_vt (bitwise)."""
    x, ds = make_fp8_inputs(1, 4, 2, 300, 128, seed=31)
    d = {n: t.cuda() for n, t in x.items()}
    say("fp8 two-step")
    o1, l1 = fa.fwd_fp8(d["q"], d["k"], d["v"], ds, ds, ds)
    vt = fa.fp8_transpose_v(d["v"])
    o2, l2 = fa.fwd_fp8_vt(d["q"], d["k"], vt, d["v"].shape, ds, ds, ds)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_fp8_gqa_equals_repeated_kv_and_causality():
    """GQA gives the MHA result with K, V repeated per group (bitwise), and
    keys a causal row cannot see do not change it (bitwise)."""
    B, Hq, Hkv, T, D = 1, 4, 2, 400, 128
    x, ds = make_fp8_inputs(B, Hq, Hkv, T, D, seed=57)
    d = {n: t.cuda() for n, t in x.items()}
    say("fp8 gqa / causality")
    o, l = fa.fwd_fp8(d["q"], d["k"], d["v"], ds, ds, ds)
    rep = {n: d[n].view(torch.uint8).repeat_interleave(Hq // Hkv, dim=1).view(torch.float8_e4m3fn)
           for n in ("k", "v")}
    o2, l2 = fa.fwd_fp8(d["q"], rep["k"], rep["v"], ds, ds, ds)
    k3 = d["k"].view(torch.uint8).clone()
    v3 = d["v"].view(torch.uint8).clone()
    k3[:, :, 200:] = 0x38  # 1.0
    v3[:, :, 200:] = 0xB8  # -1.0
    o3, l3 = fa.fwd_fp8(d["q"], k3.view(torch.float8_e4m3fn), v3.view(torch.float8_e4m3fn), ds, ds, ds)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(l, l2)
    assert torch.equal(o[:, :, :200], o3[:, :, :200]) and torch.equal(l[:, :, :200], l3[:, :, :200])


def test_fp8_fullsize_sampled_rows():
    """C5-fp8 in the benchmark's configuration: sampled query rows against
    the oracle's rows, each held to the e4m3 bound computed for that row."""
    w = WORKLOADS["C5-fp8"]
    x = workload_inputs(w)
    ds = 1.0 / w.input_scale
    d = {n: t.cuda() for n, t in x.items()}
    say(f"fp8 full size {w.name}")
    o, lse = fa.fwd_fp8(d["q"], d["k"], d["v"], ds, ds, ds, scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    o, lse = o.cpu(), lse.cpu()
    del d
    G = w.Hq // w.Hkv
    T = w.T
    rows = [0, 1, 63, 64, 255, 256, T // 2, T - 65, T - 64, T - 2, T - 1]
    for h in (0, w.Hq // 2, w.Hq - 1):
        hk = h // G
        qh = real(x["q"][0, h], ds)
        kh = real(x["k"][0, hk], ds)
        vh = real(x["v"][0, hk], ds)
        ro, rl = oracle.fwd_rows(qh[None, None], kh[None, None], vh[None, None],
                                 [(0, 0, i) for i in rows], w.scale, w.causal)
        for n, i in enumerate(rows):
            s = w.scale * kh[: i + 1] @ qh[i]
            p = np.exp(s - s.max())
            l = p.sum()
            mag = (p / l) @ np.abs(vh[: i + 1])
            sub = E4M3_SUB * np.abs(vh[: i + 1]).sum(0) / l
            assert_fp8_close(f"row {i} head {h}", o[0, h, i].double().numpy(), ro[n], mag, sub)
            tol = float(score_bound(qh[i], kh[: i + 1], w.scale).max()) + 1e-5
            assert abs(float(lse[0, h, i]) - rl[n]) <= tol


def test_fp8_lse_with_dominant_products():
    """Scores whose dot products hold one product of 120-352 among small ones
    (the case where the instruction's group alignment drops bits): lse stays
    within the derived bound, and O within its e4m3 bound."""
    B, Hq, Hkv, T, D = 1, 2, 1, 300, 128
    rng = np.random.default_rng(352)
    def codes(a):
        return torch.from_numpy(a).to(torch.float8_e4m3fn)
    q = 0.25 * rng.standard_normal((B, Hq, T, D))
    k = 0.25 * rng.standard_normal((B, Hkv, T, D))
    v = rng.standard_normal((B, Hkv, T, D))
    q[..., 0] = 16.0
    k[..., 0] = rng.choice([-22.0, -14.0, -7.5, 7.5, 14.0, 22.0], (B, Hkv, T))
    x = {n: codes(a) for n, a in (("q", q), ("k", k), ("v", v))}
    d = {n: t.cuda() for n, t in x.items()}
    say("fp8 dominant products")
    scale = 1 / 8
    o, lse = fa.fwd_fp8(d["q"], d["k"], d["v"], 1.0, 1.0, 1.0, scale=scale, causal=True)
    torch.cuda.synchronize()
    qr, kr, vr = (real(x[n], 1.0) for n in ("q", "k", "v"))
    ro, rl, om = oracle.fwd(qr, kr, vr, scale, True, return_mag=True)
    assert_fp8_close("O", f64(o), ro, om, subnormal_term(qr, kr, vr, scale, True, 0))
    lb = lse_bound(qr, kr, scale, True, 0)
    err = np.abs(f64(lse) - rl)
    say(f"fp8 dominant products: worst lse error {float((err / lb).max()):.3f}x the bound, "
        f"largest error {float(err.max()):.3e}")
    assert np.all(err <= lb)
