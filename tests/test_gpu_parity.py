"""GPU parity: the HIP kernels (through the C ABI) against the fp64 oracle,
element by element, at sizes the oracle finishes in seconds that span several
tiles, ragged tails, GQA and both mask modes; plus the pages' worked examples
pushed through the kernels at tile boundaries.
"""
import functools
import math
import zlib

import numpy as np
import pytest
import torch

import exact_attention_30_amd as fa
import oracle
from tests import lazy_model
from tests.gpu_util import (assert_close, assert_lse_close, emulated_fwd, emulated_grads, f64, say,
                            to_dev)
from workloads import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

bf16, fp32 = torch.bfloat16, torch.float32

# name: (B, Hq, Hkv, T, D, dtype, causal, scale)
CASES = {
    "C1": (1, 1, 1, 128, 64, fp32, True, 1 / 8),
    "C2": (2, 8, 8, 512, 64, bf16, True, 1 / 8),
    "t70_d64_causal": (1, 2, 2, 70, 64, bf16, True, 1 / 8),
    "t70_d64_full_gqa": (1, 2, 1, 70, 64, bf16, False, 1 / 8),
    "t1_d128": (2, 2, 1, 1, 128, bf16, True, 1 / math.sqrt(128)),
    "t129_d128_gqa": (2, 4, 2, 129, 128, bf16, True, 1 / math.sqrt(128)),
    "t333_d128_full_gqa": (1, 8, 2, 333, 128, bf16, False, 1 / math.sqrt(128)),
    "t777_d64_causal_gqa": (1, 6, 3, 777, 64, bf16, True, 0.15),
    "t1000_d128_causal_gqa4": (1, 4, 1, 1000, 128, bf16, True, 1 / math.sqrt(128)),
    "t70_d96_causal": (1, 2, 2, 70, 96, bf16, True, 1 / math.sqrt(96)),
    "t333_d96_full_gqa": (1, 4, 2, 333, 96, bf16, False, 1 / math.sqrt(96)),
    "t1000_d96_causal_gqa4": (1, 4, 1, 1000, 96, bf16, True, 1 / math.sqrt(96)),
    "t333_d128_causal_gqa3_bhkv8": (2, 12, 4, 333, 128, bf16, True, 1 / math.sqrt(128)),
    "t700_d64_full_gqa3": (1, 6, 2, 700, 64, bf16, False, 1 / 8),
    "t300_d128_causal_gqa8": (1, 16, 2, 300, 128, bf16, True, 1 / math.sqrt(128)),
    "t200_d64_causal_gqa8_bhkv8": (4, 16, 2, 200, 64, bf16, True, 1 / 8),
    "t1100_d96_causal_gqa8": (1, 8, 1, 1100, 96, bf16, True, 1 / math.sqrt(96)),
    "fp32_t200_d128": (1, 2, 1, 200, 128, fp32, True, 1 / math.sqrt(128)),
    "fp32_t150_d64_gqa3": (1, 3, 1, 150, 64, fp32, True, 1 / 8),
    "fp32_t70_d64_full": (1, 2, 2, 70, 64, fp32, False, 1 / 8),
}


def case_inputs(name):
    B, Hq, Hkv, T, D, dt, causal, scale = CASES[name]
    if name in WORKLOADS:
        w = WORKLOADS[name]
        return make_inputs(w.B, w.Hq, w.Hkv, w.T, w.D, w.dtype, w.seed)
    return make_inputs(B, Hq, Hkv, T, D, dt, seed=zlib.crc32(name.encode()) % 100000)


@functools.lru_cache(maxsize=None)
def reference(name):
    """Oracle outputs and, for the bf16 cases beyond the benchmark workloads,
    the emulation of the method's bf16 roundings (gpu_util)."""
    B, Hq, Hkv, T, D, dt, causal, scale = CASES[name]
    x = case_inputs(name)
    q, k, v, do = (x[n].double().numpy() for n in ("q", "k", "v", "dout"))
    o, lse = oracle.fwd(q, k, v, scale, causal)
    dq, dk, dv = oracle.bwd(q, k, v, do, scale, causal)
    if name in WORKLOADS or dt == fp32:  # the target tolerance alone
        return (o, lse, dq, dk, dv), (None, None, None, None)
    xs = {"q": q, "k": k, "v": v, "dout": do}
    eo = emulated_fwd(xs, scale, causal)
    return (o, lse, dq, dk, dv), (eo, *emulated_grads(xs, eo, lse, scale, causal))


@pytest.mark.parametrize("name", list(CASES))
def test_forward_matches_oracle(name):
    B, Hq, Hkv, T, D, dt, causal, scale = CASES[name]
    x = to_dev(case_inputs(name))
    say(f"fwd {name} B={B} Hq={Hq} Hkv={Hkv} T={T} D={D} {dt} causal={causal}")
    o, lse = fa.fwd(x["q"], x["k"], x["v"], scale=scale, causal=causal)
    torch.cuda.synchronize()
    (ro, rlse, *_), (eo, *_) = reference(name)
    assert_close("O", f64(o), ro, dt, eo)
    assert_lse_close(f64(lse), rlse, dt)


@pytest.mark.parametrize("name", list(CASES))
def test_backward_matches_oracle(name):
    B, Hq, Hkv, T, D, dt, causal, scale = CASES[name]
    x = to_dev(case_inputs(name))
    say(f"bwd {name} B={B} Hq={Hq} Hkv={Hkv} T={T} D={D} {dt} causal={causal}")
    o, lse = fa.fwd(x["q"], x["k"], x["v"], scale=scale, causal=causal)
    dq, dk, dv = fa.bwd(x["q"], x["k"], x["v"], o, x["dout"], lse, scale=scale, causal=causal)
    torch.cuda.synchronize()
    (_, _, rdq, rdk, rdv), (_, eq, ek, ev) = reference(name)
    assert_close("dQ", f64(dq), rdq, dt, eq)
    assert_close("dK", f64(dk), rdk, dt, ek)
    assert_close("dV", f64(dv), rdv, dt, ev)


@pytest.mark.parametrize("dt,D", [(bf16, 64), (bf16, 96), (bf16, 128), (fp32, 64), (fp32, 128)])
def test_preprocess_matches_jacobian_term(dt, D):
    """Delta = rowsum(dO * O) ("L'attention fusionnée", «La passe arrière»):
    exact (fp32 rounding) on the kernel's own inputs, and equal to the
    oracle's Jacobian form sum_j P_ij dP_ij up to the rounding of O."""
    B, Hq, Hkv, T = 1, 4, 2, 300
    x = make_inputs(B, Hq, Hkv, T, D, dt, seed=91)
    xd = to_dev(x)
    say(f"preprocess {dt} T={T} D={D}")
    o, lse = fa.fwd(xd["q"], xd["k"], xd["v"], scale=0.1, causal=True)
    delta = fa.bwd_preprocess(o, xd["dout"])
    torch.cuda.synchronize()
    direct = (o.double() * xd["dout"].double()).sum(-1).cpu().numpy()
    assert np.max(np.abs(f64(delta) - direct) / np.maximum(1.0, np.abs(direct))) < 1e-5
    q, k, v, do = (x[n].double().numpy() for n in ("q", "k", "v", "dout"))
    o_ref, _ = oracle.fwd(q, k, v, 0.1, True)
    *_, jac = oracle.bwd(q, k, v, do, 0.1, True, return_jac=True)
    # O enters Delta rounded to the output dtype: the difference is bounded by
    # u * sum_d |dO_id O_id| (u = 2^-8 for bf16); fp32 keeps max-abs 1e-5
    if dt == bf16:
        mag = np.sum(np.abs(do * o_ref), axis=-1)
        assert np.max(np.abs(f64(delta) - jac) / (2.0 ** -8 * (mag + np.abs(jac)) + 1e-6)) <= 1.0
    else:
        assert np.max(np.abs(f64(delta) - jac) / np.maximum(1.0, np.abs(jac))) < 1e-5


# ---------------------------------------------------------------------------
# The pages' worked examples, pushed through the kernels
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dt", [bf16, fp32])
def test_block_mean_counterexample_across_tiles(dt, golden):
    """"FlashAttention" note, «Blockergebnisse einfach zu mitteln reicht
    nicht»: scores 0 and ln 3 in ratio [1,1,3,3] give 0.75.  Here the two
    blocks are whole key tiles (keys 0-127 score 0, keys 128-255 score ln 3,
    values 0 and 1), so merging tiles by their plain mean would give 0.5."""
    g = golden("block_mean_counterexample.txt")
    T, D = 256, 64
    q = torch.zeros(1, 1, T, D)
    q[..., 0] = 1.0
    k = torch.zeros(1, 1, T, D)
    v = torch.zeros(1, 1, T, D)
    k[:, :, 128:, 0] = 1.0
    v[:, :, 128:, 0] = 1.0
    say(f"block-mean pin {dt}")
    o, _ = fa.fwd(q.to(dt).cuda(), k.to(dt).cuda(), v.to(dt).cuda(), scale=g["scores"][2],
                  causal=False)
    o = f64(o)
    assert np.max(np.abs(o[..., 0] - g["result"])) < 1e-6
    assert np.max(np.abs(o[..., 1:])) == 0.0


def test_fig79_row_through_kernel(golden):
    """Fig. 7.9 of "FlashAttention: l'attenzione che non spreca memoria": the
    eight scores and values give 5.257, padded to D = 64 on the fp32 path."""
    g = golden("fig79_eight_scores.txt")
    T, D = 8, 64
    q = torch.zeros(1, 1, T, D)
    q[..., 0] = 1.0
    k = torch.zeros(1, 1, T, D)
    v = torch.zeros(1, 1, T, D)
    k[0, 0, :, 0] = torch.tensor(g["scores"])
    v[0, 0, :, 0] = torch.tensor(g["values"])
    say("fig79 pin")
    o, lse = fa.fwd(q.cuda(), k.cuda(), v.cuda(), scale=1.0, causal=False)
    o = f64(o)
    assert np.max(np.abs(o[0, 0, :, 0] - g["result"])) < 0.5 * 10 ** (-g["decimals"])
    ro, rl = oracle.fwd(q.double().numpy(), k.double().numpy(), v.double().numpy(), 1.0, False)
    assert np.max(np.abs(o - ro)) < 1e-5
    assert np.max(np.abs(f64(lse) - rl)) < 1e-5


def test_causal_row_zero_is_v0():
    """Causal query 0 sees only key 0, so O row 0 is v_0 (bit for bit on the
    bf16 path) and lse_0 = scale q_0.k_0."""
    x = make_inputs(2, 8, 2, 300, 128, bf16, seed=5)
    xd = to_dev(x)
    say("causal row 0")
    o, lse = fa.fwd(xd["q"], xd["k"], xd["v"], scale=0.09, causal=True)
    o = o.cpu()
    for h in range(8):
        assert torch.equal(o[:, h, 0], x["v"][:, h // 4, 0])
    s00 = 0.09 * (x["q"][:, :, 0].double() * x["k"][:, :, 0].double().repeat_interleave(4, 1)).sum(-1)
    assert np.max(np.abs(f64(lse)[:, :, 0] - s00.numpy())) < 1e-4


def test_rows_of_P_sum_to_one():
    """A value column of ones comes out as ones (to bf16 rounding of the
    weights that enter the P V product)."""
    x = make_inputs(1, 4, 2, 517, 128, bf16, seed=6)
    x["v"][..., 7] = 1.0
    xd = to_dev(x)
    say("ones column")
    for causal in (True, False):
        o, _ = fa.fwd(xd["q"], xd["k"], xd["v"], scale=0.1, causal=causal)
        assert np.max(np.abs(f64(o)[..., 7] - 1.0)) <= 4e-3


# ---------------------------------------------------------------------------
# Invariants of the GPU path
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal,G,B,Hkv,T,D", [(True, 4, 1, 2, 400, 128), (False, 4, 1, 2, 400, 128),
                                                (True, 3, 2, 4, 333, 128), (False, 3, 1, 2, 700, 64),
                                                (True, 8, 1, 2, 1100, 64), (False, 8, 4, 2, 200, 128)])
def test_gqa_equals_repeated_kv(causal, G, B, Hkv, T, D):
    """Grouped heads read the same K/V as multi-head attention on K/V repeated
    along heads: identical O, lse, dQ; dK/dV equal the group sums.  Group
    sizes 3, 4 and 8, with B*Hkv a multiple of 8 and not; the forward both
    unsplit and split (where the shapes split)."""
    Hq = G * Hkv
    x = to_dev(make_inputs(B, Hq, Hkv, T, D, bf16, seed=7 + G))
    kr = x["k"].repeat_interleave(G, 1).contiguous()
    vr = x["v"].repeat_interleave(G, 1).contiguous()
    nbytes = fa.fwd_split_bytes(B, Hq, Hkv, T, T, D)
    if nbytes:
        part = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        say(f"gqa split forward G={G} causal={causal}")
        o1, l1 = fa.fwd(x["q"], x["k"], x["v"], causal=causal, partial=part)
        o2, l2 = fa.fwd(x["q"], kr, vr, causal=causal,
                        partial=torch.empty(fa.fwd_split_bytes(B, Hq, Hq, T, T, D), dtype=torch.uint8,
                                            device="cuda"))
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
    say(f"gqa vs mha causal={causal}")
    o1, l1 = fa.fwd(x["q"], x["k"], x["v"], causal=causal)
    o2, l2 = fa.fwd(x["q"], kr, vr, causal=causal)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    g1 = fa.bwd(x["q"], x["k"], x["v"], o1, x["dout"], l1, causal=causal)
    g2 = fa.bwd(x["q"], kr, vr, o2, x["dout"], l2, causal=causal)
    assert torch.equal(g1[0], g2[0])
    for a, b in ((g1[1], g2[1]), (g1[2], g2[2])):
        # GQA sums the group in fp32 and rounds once; the reference rounds
        # each head to bf16 before summing
        ref = b.double().reshape(B, Hkv, G, T, D).sum(2)
        err = (a.double() - ref).abs().max().item()
        assert err <= 1e-2 * max(1.0, ref.abs().max().item())


def test_future_keys_do_not_leak():
    """Changing keys/values after position i leaves rows <= i of O, lse and dQ
    bit for bit unchanged."""
    x = make_inputs(1, 4, 2, 600, 128, bf16, seed=8)
    y = {k: v.clone() for k, v in x.items()}
    i = 250
    y["k"][:, :, i + 1:] = torch.randn(y["k"][:, :, i + 1:].shape).to(bf16)
    y["v"][:, :, i + 1:] = torch.randn(y["v"][:, :, i + 1:].shape).to(bf16)
    outs = []
    for inp in (x, y):
        d = to_dev(inp)
        say("causality")
        o, l = fa.fwd(d["q"], d["k"], d["v"], causal=True)
        dq, _, _ = fa.bwd(d["q"], d["k"], d["v"], o, d["dout"], l, causal=True)
        outs.append((o.cpu(), l.cpu(), dq.cpu()))
    for a, b in zip(outs[0], outs[1]):
        assert torch.equal(a[:, :, :i + 1], b[:, :, :i + 1])


def test_bitwise_deterministic():
    """Two runs give bit-identical outputs (no atomics anywhere)."""
    x = to_dev(make_inputs(1, 8, 2, 1100, 128, bf16, seed=9))
    runs = []
    for _ in range(2):
        say("determinism")
        o, l = fa.fwd(x["q"], x["k"], x["v"], causal=True)
        g = fa.bwd(x["q"], x["k"], x["v"], o, x["dout"], l, causal=True)
        runs.append([o, l, *g])
    for a, b in zip(*runs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("shape", [(2, 4, 4, 333, 333, 64, True, None),
                                   (1, 4, 2, 700, 700, 128, True, None),
                                   (2, 2, 1, 300, 300, 96, True, None),
                                   (1, 8, 2, 2048, 2048, 128, True, None),
                                   (1, 4, 2, 700, 700, 128, False, None),
                                   (1, 2, 1, 1500, 1500, 64, False, None),
                                   (1, 4, 2, 300, 900, 128, True, 250),
                                   (1, 2, 1, 1000, 2500, 64, True, None),
                                   (1, 4, 1, 257, 513, 128, False, None)])
def test_stage_entry_points_equal_fa_bwd(shape):
    """fa_bwd (fa_bwd_kv for Tq != Tk or an offset) gives bitwise the results
    of preprocess + dK/dV + dQ: in bf16 its dQ kernel forms Delta itself, in
    the preprocess kernel's order, and the Delta it leaves in the workspace
    equals the preprocess output.  Causal and not, Tq != Tk with and without
    an offset off the tile grid, and shapes whose stages split."""
    B, Hq, Hkv, Tq, Tk, D, causal, off = shape
    x = to_dev(make_inputs(B, Hq, Hkv, Tq, D, bf16, seed=10 + D + Tk, Tk=Tk))
    say(f"stages B={B} Hq={Hq} Hkv={Hkv} Tq={Tq} Tk={Tk} D={D} causal={causal} off={off}")
    kw = dict(causal=causal, q_offset=off)
    o, l = fa.fwd(x["q"], x["k"], x["v"], **kw)
    ws = torch.empty(fa.bwd_workspace_bytes(B, Hq, Hkv, Tq, D, Tk=Tk), dtype=torch.uint8,
                     device="cuda")
    dq, dk, dv = fa.bwd(x["q"], x["k"], x["v"], o, x["dout"], l, workspace=ws, **kw)
    delta = fa.bwd_preprocess(o, x["dout"])
    assert torch.equal(ws[:B * Hq * Tq * 4].view(torch.float32).view(B, Hq, Tq), delta)
    part = torch.empty(max(fa.dkdv_split_bytes(B, Hq, Hkv, Tq, Tk, D),
                           fa.dq_split_bytes(B, Hq, Hkv, Tq, Tk, D), 16), dtype=torch.uint8,
                       device="cuda")
    dk2, dv2 = fa.bwd_dkdv(x["q"], x["k"], x["v"], x["dout"], l, delta, partial=part, **kw)
    dq2 = fa.bwd_dq(x["q"], x["k"], x["v"], x["dout"], l, delta, partial=part, **kw)
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)


@pytest.mark.parametrize("shape", [(1, 4, 1, 1000, 128), (1, 8, 2, 700, 64), (2, 2, 1, 513, 128),
                                   (1, 4, 1, 900, 96)])
def test_split_dkdv(shape):
    """Few kv heads leave the dK/dV kernel few workgroups, so its query side
    is split into chunks whose fp32 partial sums are added in chunk order: the
    result is bitwise reproducible, within one bf16 rounding of the unsplit
    kernel's, and within the tolerance of the oracle."""
    B, Hq, Hkv, T, D = shape
    nbytes = fa.dkdv_split_bytes(B, Hq, Hkv, T, T, D)
    assert nbytes > 0, "shape expected to split"
    x = to_dev(make_inputs(B, Hq, Hkv, T, D, bf16, seed=12 + T))
    say(f"split dK/dV B={B} Hq={Hq} Hkv={Hkv} T={T} D={D}")
    o, l = fa.fwd(x["q"], x["k"], x["v"], causal=True)
    delta = fa.bwd_preprocess(o, x["dout"])
    part = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    args = (x["q"], x["k"], x["v"], x["dout"], l, delta)
    dk1, dv1 = fa.bwd_dkdv(*args, causal=True, partial=part)
    dk2, dv2 = fa.bwd_dkdv(*args, causal=True, partial=part)
    dk0, dv0 = fa.bwd_dkdv(*args, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(dk1, dk2) and torch.equal(dv1, dv2)
    for split, whole in ((dk1, dk0), (dv1, dv0)):
        a, b = f64(split), f64(whole)
        # the two fp32 sums differ in order only: at most one bf16 step apart
        assert np.all(np.abs(a - b) <= 2.0 ** -7 * np.maximum(np.abs(b), 1e-30) + 1e-6)
    q, k, v, do = (x[n].double().cpu().numpy() for n in ("q", "k", "v", "dout"))
    sc = 1 / math.sqrt(D)
    ro, rl = oracle.fwd(q, k, v, sc, True)
    _, rdk, rdv = oracle.bwd(q, k, v, do, sc, True)
    xs = {"q": q, "k": k, "v": v, "dout": do}
    _, ek, ev = emulated_grads(xs, emulated_fwd(xs, sc, True), rl, sc, True)
    assert_close("dK split", f64(dk1), rdk, bf16, ek)
    assert_close("dV split", f64(dv1), rdv, bf16, ev)


def test_no_device_allocation_by_the_library():
    """The library allocates nothing: with outputs and workspace allocated by
    the caller, free device memory is unchanged across fwd + bwd at a length
    where one fp32 score matrix per head would be 1 GiB (T = 16384)."""
    B, Hq, Hkv, T, D = 1, 4, 1, 16384, 128
    x = to_dev(make_inputs(B, Hq, Hkv, T, D, bf16, seed=11))
    o = torch.empty_like(x["q"])
    l = torch.empty(B, Hq, T, device="cuda")
    grads = (torch.empty_like(x["q"]), torch.empty_like(x["k"]), torch.empty_like(x["v"]))
    ws = torch.empty(fa.bwd_workspace_bytes(B, Hq, Hkv, T, D), dtype=torch.uint8, device="cuda")
    say("memory")
    fa.fwd(x["q"], x["k"], x["v"], out=o, lse=l)
    fa.bwd(x["q"], x["k"], x["v"], o, x["dout"], l, workspace=ws, grads=grads)
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    alloc0 = torch.cuda.memory_allocated()
    fa.fwd(x["q"], x["k"], x["v"], out=o, lse=l)
    fa.bwd(x["q"], x["k"], x["v"], o, x["dout"], l, workspace=ws, grads=grads)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert torch.cuda.memory_allocated() == alloc0
    assert abs(free1 - free0) < (1 << 20)


@pytest.mark.parametrize("shape", [(1, 4, 1, 2048, 128), (1, 2, 2, 1500, 64), (2, 1, 1, 700, 128),
                                   (1, 2, 1, 1500, 96)])
def test_split_dq(shape):
    """Few query blocks: dQ's key range is split into chunks whose fp32
    partial sums are added in chunk order; bitwise reproducible, within one
    bf16 rounding of the unsplit kernel, within the tolerance of the oracle."""
    B, Hq, Hkv, T, D = shape
    nbytes = fa.dq_split_bytes(B, Hq, Hkv, T, T, D)
    assert nbytes > 0, "shape expected to split"
    x = to_dev(make_inputs(B, Hq, Hkv, T, D, bf16, seed=13 + T))
    say(f"split dQ B={B} Hq={Hq} Hkv={Hkv} T={T} D={D}")
    o, l = fa.fwd(x["q"], x["k"], x["v"], causal=True)
    delta = fa.bwd_preprocess(o, x["dout"])
    part = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    args = (x["q"], x["k"], x["v"], x["dout"], l, delta)
    dq1 = fa.bwd_dq(*args, causal=True, partial=part)
    dq2 = fa.bwd_dq(*args, causal=True, partial=part)
    dq0 = fa.bwd_dq(*args, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(dq1, dq2)
    a, b = f64(dq1), f64(dq0)
    assert np.all(np.abs(a - b) <= 2.0 ** -7 * np.abs(b) + 1e-6)
    q, k, v, do = (x[n].double().cpu().numpy() for n in ("q", "k", "v", "dout"))
    sc = 1 / math.sqrt(D)
    ro, rl = oracle.fwd(q, k, v, sc, True)
    rdq, _, _ = oracle.bwd(q, k, v, do, sc, True)
    xs = {"q": q, "k": k, "v": v, "dout": do}
    eq, _, _ = emulated_grads(xs, emulated_fwd(xs, sc, True), rl, sc, True)
    assert_close("dQ split", a, rdq, bf16, eq)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("Hq,Hkv,T", [(16, 8, 4096), (24, 8, 3000)])
def test_forward_tile_invariance(causal, Hq, Hkv, T):
    """The forward's static tile table (the tile sizes of "Optimización de
    Flash Attention ...", «La pila de optimización»): at D = 64 a grid of
    fewer than 512 blocks of 256 rows runs 128-row workgroups of four waves,
    a larger one 256-row workgroups of eight.  Unsplit, a row's result does
    not depend on that choice: the heads of a batch of one (128-row blocks)
    equal, bit for bit, the same heads inside a batch of two (256-row
    blocks)."""
    D = 64
    assert fa.block_rows("fwd", 1, Hq, T, D) == 128 and fa.block_rows("fwd", 2, Hq, T, D) == 256
    x = to_dev(make_inputs(2, Hq, Hkv, T, D, bf16, seed=31 + T))
    say(f"tile invariance Hq={Hq} Hkv={Hkv} T={T} causal={causal}")
    o2, l2 = fa.fwd(x["q"], x["k"], x["v"], causal=causal)
    o1, l1 = fa.fwd(x["q"][:1].contiguous(), x["k"][:1].contiguous(), x["v"][:1].contiguous(),
                    causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2[:1]) and torch.equal(l1, l2[:1])


@pytest.mark.parametrize("causal", [True, False])
def test_dq_tile_invariance(causal):
    """The dQ stage's tile table: at D = 64, fewer than 256 blocks of 256
    rows run 128-row workgroups of four waves, more run 256-row workgroups.
    Unsplit, a row's dQ (and the Delta the stage forms) does not depend on
    that choice: a batch of one (128-row blocks) equals, bit for bit, the same
    heads inside a batch of two (256-row blocks)."""
    Hq, Hkv, T, D = 16, 8, 2048, 64
    assert fa.block_rows("dq", 1, Hq, T, D) == 128 and fa.block_rows("dq", 2, Hq, T, D) == 256
    x = to_dev(make_inputs(2, Hq, Hkv, T, D, bf16, seed=57))
    say(f"dQ tile invariance Hq={Hq} Hkv={Hkv} T={T} causal={causal}")
    o, lse = fa.fwd(x["q"], x["k"], x["v"], causal=causal)
    one = {n: t[:1].contiguous() for n, t in x.items()}
    dq2, d2 = fa.bwd_dq_delta(x["q"], x["k"], x["v"], o, x["dout"], lse, causal=causal)
    dq1, d1 = fa.bwd_dq_delta(one["q"], one["k"], one["v"], o[:1].contiguous(), one["dout"],
                              lse[:1].contiguous(), causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(dq1, dq2[:1]) and torch.equal(d1, d2[:1])


@pytest.mark.parametrize("causal", [True, False])
def test_dkdv_tile_invariance(causal):
    """The dK/dV stage's tile table: at D = 64, fewer than 256 blocks of 256
    keys run 128-key workgroups of four waves, more run 256-key workgroups.
    A wave visits the same query tiles in the same order either way, so
    unsplit, dK and dV of a batch of one (128-key blocks) equal, bit for bit,
    the same kv heads inside a batch of two (256-key blocks)."""
    Hq, Hkv, T, D = 16, 8, 4096, 64
    assert fa.block_rows("dkdv", 1, Hkv, T, D) == 128 and fa.block_rows("dkdv", 2, Hkv, T, D) == 256
    x = to_dev(make_inputs(2, Hq, Hkv, T, D, bf16, seed=58))
    say(f"dK/dV tile invariance Hq={Hq} Hkv={Hkv} T={T} causal={causal}")
    o, lse = fa.fwd(x["q"], x["k"], x["v"], causal=causal)
    delta = fa.bwd_preprocess(o, x["dout"])
    one = {n: t[:1].contiguous() for n, t in x.items()}
    dk2, dv2 = fa.bwd_dkdv(x["q"], x["k"], x["v"], x["dout"], lse, delta, causal=causal)
    dk1, dv1 = fa.bwd_dkdv(one["q"], one["k"], one["v"], one["dout"], lse[:1].contiguous(),
                           delta[:1].contiguous(), causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(dk1, dk2[:1]) and torch.equal(dv1, dv2[:1])


@pytest.mark.parametrize("shape", [(1, 1, 1, 2048, 2048, 128), (1, 4, 2, 1500, 1500, 64),
                                   (2, 2, 1, 300, 2000, 128), (1, 2, 1, 600, 1800, 96)])
def test_split_forward(shape):
    """Few query blocks: the forward splits each block's key range into
    chunks and merges their (numerator, reference max, sum) with the block
    merge rule.  O and lse match the oracle, agree with the unsplit forward to
    rounding, and are bitwise reproducible; chunks without keys (a query block
    with fewer key tiles than chunks) contribute nothing."""
    B, Hq, Hkv, Tq, Tk, D = shape
    nbytes = fa.fwd_split_bytes(B, Hq, Hkv, Tq, Tk, D)
    assert nbytes > 0, "shape expected to split"
    x = to_dev(make_inputs(B, Hq, Hkv, Tq, D, bf16, seed=14 + Tq, Tk=Tk))
    say(f"split forward B={B} Hq={Hq} Hkv={Hkv} Tq={Tq} Tk={Tk} D={D}")
    part = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    o1, l1 = fa.fwd(x["q"], x["k"], x["v"], causal=True, partial=part)
    o2, l2 = fa.fwd(x["q"], x["k"], x["v"], causal=True, partial=part)
    o0, l0 = fa.fwd(x["q"], x["k"], x["v"], causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert float((l1 - l0).abs().max()) < 1e-4
    a, b = f64(o1), f64(o0)
    assert np.all(np.abs(a - b) <= 2.0 ** -7 * np.abs(b) + 1e-3)
    q, k, v = (x[n].double().cpu().numpy() for n in ("q", "k", "v"))
    ro, rl = oracle.fwd(q, k, v, 1 / math.sqrt(D), True)
    eo = emulated_fwd({"q": q, "k": k, "v": v}, 1 / math.sqrt(D), True, Tk - Tq,
                      S=lazy_model.nsplit(B, Hq, Tq, Tk, D))
    assert_close("O split", a, ro, bf16, eo)
    assert_lse_close(f64(l1), rl, bf16)
