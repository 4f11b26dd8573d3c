"""GPU parity where the forward kernels must move their reference max.

The kernels rescale o and l only when a row's scores rise more than 8 log2
units above its reference (the online softmax of "L'attention fusionnée",
«Le softmax en ligne», done lazily).  The inputs of tests/rescale_inputs.py
put such rises at key-tile boundaries; tests/test_lazy_model.py shows on the
CPU that they reach that branch at the second tile, inside waves' ranges of
both parities, at rows' last tiles and in later chunks of the split forward,
and that a planted mistake in the branch fails the tolerance used here.  The
forward (bf16 unsplit and split, fp32, e4m3) and the backward that reads its
lse are compared with the oracle element by element.  The row of Fig. 7.9
("FlashAttention: l'attenzione che non spreca memoria", «La online softmax,
con i numeri») goes through the bf16 kernel with its blocks in different
tiles, once as printed (5.257) and once scaled so that each rise of its
running max moves the kernels' reference.
"""
import numpy as np
import pytest
import torch

import exact_attention_30_amd as fa
import oracle
from tests.gpu_util import (assert_close, assert_grad_close, assert_lse_close, emulated_fwd,
                            emulated_grads, f64, say)
from tests.rescale_inputs import (CASES, FP8_CASES, FP32_CASES, SCALE, as_torch, fig79_inputs,
                                  make_case)

pytestmark = pytest.mark.gpu

bf16, fp32 = torch.bfloat16, torch.float32


def run_fwd(x, dt, causal, off, partial=False):
    d = {n: t.cuda() for n, t in as_torch(x, dt).items()}
    B, Hq, Tq, D = x["q"].shape
    Hkv, Tk = x["k"].shape[1], x["k"].shape[2]
    part = None
    if partial:
        nbytes = fa.fwd_split_bytes(B, Hq, Hkv, Tq, Tk, D, dt)
        assert nbytes > 0, "shape expected to split"
        part = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    o, lse = fa.fwd(d["q"], d["k"], d["v"], scale=SCALE, causal=causal, q_offset=off, partial=part)
    return d, o, lse


@pytest.mark.parametrize("name", list(CASES) + list(FP32_CASES))
def test_forward_and_backward(name):
    B, Hq, Hkv, Tq, Tk, D, causal, off, seed, big = {**CASES, **FP32_CASES}[name]
    dt = fp32 if name in FP32_CASES else bf16
    x, _ = make_case(name)
    say(f"rescale {name}: B={B} Hq={Hq} Hkv={Hkv} Tq={Tq} Tk={Tk} D={D} causal={causal} "
        f"off={off} {dt}")
    d, o, lse = run_fwd(x, dt, causal, off)
    dq, dk, dv = fa.bwd(d["q"], d["k"], d["v"], o, d["dout"], lse, scale=SCALE, causal=causal,
                        q_offset=off)
    torch.cuda.synchronize()
    ro, rl = oracle.fwd(x["q"], x["k"], x["v"], SCALE, causal, q_offset=off)
    rdq, rdk, rdv = oracle.bwd(x["q"], x["k"], x["v"], x["dout"], SCALE, causal, q_offset=off)
    if dt == fp32:
        assert_close(f"O {name}", f64(o), ro, dt)
        assert_lse_close(f64(lse), rl, dt)
        for n, g, r in (("dQ", dq, rdq), ("dK", dk, rdk), ("dV", dv, rdv)):
            assert_close(f"{n} {name}", f64(g), r, dt)
        return
    eo = emulated_fwd(x, SCALE, causal, off)
    assert_close(f"O {name}", f64(o), ro, dt, eo)
    assert_lse_close(f64(lse), rl, dt)
    em = emulated_grads(x, eo, rl, SCALE, causal, off)
    for n, g, r, e in (("dQ", dq, rdq, em[0]), ("dK", dk, rdk, em[1]), ("dV", dv, rdv, em[2])):
        assert_grad_close(f"{n} {name}", f64(g), r, e)


def test_split_forward():
    """The split forward: each chunk keeps its own reference; jumps fall on
    chunks' second and last tiles; the chunks merge to the oracle's result."""
    name = "causal_split_t2048_d128"
    B, Hq, Hkv, Tq, Tk, D, causal, off, seed, big = CASES[name]
    x, _ = make_case(name)
    say(f"rescale split {name}")
    _, o1, l1 = run_fwd(x, bf16, causal, off, partial=True)
    _, o2, l2 = run_fwd(x, bf16, causal, off, partial=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    ro, rl = oracle.fwd(x["q"], x["k"], x["v"], SCALE, causal, q_offset=off)
    assert_close(f"O split {name}", f64(o1), ro, bf16)
    assert_lse_close(f64(l1), rl, bf16)


@pytest.mark.parametrize("name", list(FP8_CASES))
def test_fp8_forward(name):
    """The e4m3 forward: its weights must stay below 448 (e4m3's largest), so
    every rise past the threshold has to move the reference."""
    from tests.test_gpu_fp8 import E4M3_U, OUT_U, lse_bound, subnormal_term

    B, Hq, Hkv, Tq, Tk, D, causal, off, seed, big = FP8_CASES[name]
    x, _ = make_case(name)
    codes = {n: torch.from_numpy(x[n]).to(torch.float8_e4m3fn).cuda() for n in ("q", "k", "v")}
    say(f"rescale fp8 {name}")
    o, lse = fa.fwd_fp8(codes["q"], codes["k"], codes["v"], 1.0, 1.0, 1.0, scale=SCALE,
                        causal=causal, q_offset=off)
    torch.cuda.synchronize()
    ro, rl, om = oracle.fwd(x["q"], x["k"], x["v"], SCALE, causal, return_mag=True, q_offset=off)
    sub = subnormal_term(x["q"], x["k"], x["v"], SCALE, causal, off)
    got = f64(o)
    assert np.all(np.isfinite(got))
    bound = E4M3_U * om + sub + OUT_U * np.abs(ro) + 1e-5
    assert float(np.max(np.abs(got - ro) / bound)) <= 1.0
    lerr = np.abs(f64(lse) - rl)
    lb = lse_bound(x["q"], x["k"], SCALE, causal, off)
    worst = np.unravel_index(np.argmax(lerr / lb), lerr.shape)
    say(f"fp8 lse: worst {float((lerr / lb)[worst]):.3f}x the bound at {worst}: error "
        f"{float(lerr[worst]):.3e}, bound {float(lb[worst]):.3e}, lse {float(rl[worst]):.4f}")
    assert np.all(lerr <= lb)


@pytest.mark.parametrize("lam", [1.0, 8.0])
def test_fig79_row_across_tiles(lam, golden):
    """Fig. 7.9's row with its four blocks in four 64-key tiles.  As printed
    (lam = 1) every row gives 5.257 (to one bf16 step); scaled by 8 each rise of
    the running max (at the 2nd and 4th block) moves the reference, and the
    result matches the oracle's."""
    g = golden("fig79_eight_scores.txt")
    x, scale = fig79_inputs(lam)
    say(f"fig79 across tiles lam={lam}")
    d = {n: t.cuda() for n, t in as_torch(x, bf16).items()}
    o, lse = fa.fwd(d["q"], d["k"], d["v"], scale=scale, causal=False)
    torch.cuda.synchronize()
    ro, rl = oracle.fwd(x["q"], x["k"], x["v"], scale, False)
    assert_close("O fig79", f64(o), ro, bf16)
    assert_lse_close(f64(lse), rl, bf16)
    if lam == 1.0:
        # bf16 numbers near 5.26 are 2^-5 apart
        assert np.max(np.abs(f64(o)[..., 0] - g["result"])) <= 2.0 ** -5
