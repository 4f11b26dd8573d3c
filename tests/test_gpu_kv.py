"""GPU parity for query rows against a key sequence of another length, with
the causal position offset (query row i sees key j iff j <= i + q_offset):
the HIP kernels through fa_fwd_kv / fa_bwd_kv against the fp64 oracle,
element by element ("Optimización de Flash Attention ...", the input_pos
argument of «Parte 1»; "L'attention fusionnée", «Un premier kernel plus lent»:
one query against 70 positions, as in generation).
"""
import functools
import math
import zlib

import numpy as np
import pytest
import torch

import exact_attention_30_amd as fa
import oracle
from tests.gpu_util import (assert_close, assert_lse_close, emulated_fwd, emulated_grads, f64, say,
                            to_dev)
from workloads import make_inputs

pytestmark = pytest.mark.gpu

bf16, fp32 = torch.bfloat16, torch.float32
S128 = 1 / math.sqrt(128)

# name: (B, Hq, Hkv, Tq, Tk, D, dtype, causal, q_offset (None: Tk - Tq), scale)
CASES = {
    "q1_k70_d64_gqa": (1, 4, 1, 1, 70, 64, bf16, True, None, 1 / 8),
    "q1_k70_d128_fp32": (1, 2, 1, 1, 70, 128, fp32, True, None, S128),
    "q1_k3000_d128": (2, 2, 2, 1, 3000, 128, bf16, True, None, S128),
    "q100_k1000_d128_gqa": (1, 4, 2, 100, 1000, 128, bf16, True, None, S128),
    "q333_k777_d64_off17": (1, 4, 2, 333, 777, 64, bf16, True, 17, 0.15),
    "q600_k1000_d128_off400": (1, 2, 1, 600, 1000, 128, bf16, True, 400, S128),
    "q300_k200_d128_off0": (2, 2, 1, 300, 200, 128, bf16, True, 0, S128),
    "q257_k513_d128_cross": (1, 4, 4, 257, 513, 128, bf16, False, None, S128),
    "q64_k2048_d128_gqa4": (1, 8, 2, 64, 2048, 128, bf16, True, None, S128),
    "q1_k300_d96": (1, 2, 1, 1, 300, 96, bf16, True, None, 1 / math.sqrt(96)),
    "q300_k900_d96_off250_gqa": (1, 4, 2, 300, 900, 96, bf16, True, 250, 1 / math.sqrt(96)),
    "q257_k513_d96_cross": (1, 2, 2, 257, 513, 96, bf16, False, None, 1 / math.sqrt(96)),
    "fp32_q70_k200_d64_off40": (1, 2, 2, 70, 200, 64, fp32, True, 40, 1 / 8),
    "fp32_q129_k70_d128_cross": (1, 2, 1, 129, 70, 128, fp32, False, None, S128),
}


def offset(name):
    B, Hq, Hkv, Tq, Tk, D, dt, causal, off, scale = CASES[name]
    return Tk - Tq if off is None else off


def case_inputs(name):
    B, Hq, Hkv, Tq, Tk, D, dt, causal, off, scale = CASES[name]
    return make_inputs(B, Hq, Hkv, Tq, D, dt, seed=zlib.crc32(name.encode()) % 100000, Tk=Tk)


@functools.lru_cache(maxsize=None)
def reference(name):
    B, Hq, Hkv, Tq, Tk, D, dt, causal, off, scale = CASES[name]
    x = case_inputs(name)
    q, k, v, do = (x[n].double().numpy() for n in ("q", "k", "v", "dout"))
    o, lse = oracle.fwd(q, k, v, scale, causal, q_offset=offset(name))
    dq, dk, dv = oracle.bwd(q, k, v, do, scale, causal, q_offset=offset(name))
    if dt == fp32:
        return (o, lse, dq, dk, dv), (None, None, None, None)
    xs = {"q": q, "k": k, "v": v, "dout": do}
    eo = emulated_fwd(xs, scale, causal, offset(name))
    return (o, lse, dq, dk, dv), (eo, *emulated_grads(xs, eo, lse, scale, causal, offset(name)))


@pytest.mark.parametrize("name", list(CASES))
def test_forward_kv_matches_oracle(name):
    B, Hq, Hkv, Tq, Tk, D, dt, causal, off, scale = CASES[name]
    x = to_dev(case_inputs(name))
    say(f"fwd_kv {name} B={B} Hq={Hq} Hkv={Hkv} Tq={Tq} Tk={Tk} D={D} {dt} causal={causal} "
        f"off={offset(name)}")
    o, lse = fa.fwd(x["q"], x["k"], x["v"], scale=scale, causal=causal, q_offset=off)
    torch.cuda.synchronize()
    (ro, rlse, *_), (eo, *_) = reference(name)
    assert_close("O", f64(o), ro, dt, eo)
    assert_lse_close(f64(lse), rlse, dt)


@pytest.mark.parametrize("name", list(CASES))
def test_backward_kv_matches_oracle(name):
    B, Hq, Hkv, Tq, Tk, D, dt, causal, off, scale = CASES[name]
    x = to_dev(case_inputs(name))
    say(f"bwd_kv {name} B={B} Hq={Hq} Hkv={Hkv} Tq={Tq} Tk={Tk} D={D} {dt} causal={causal} "
        f"off={offset(name)}")
    o, lse = fa.fwd(x["q"], x["k"], x["v"], scale=scale, causal=causal, q_offset=off)
    dq, dk, dv = fa.bwd(x["q"], x["k"], x["v"], o, x["dout"], lse, scale=scale, causal=causal,
                        q_offset=off)
    torch.cuda.synchronize()
    (_, _, rdq, rdk, rdv), (_, edq, edk, edv) = reference(name)
    assert_close("dQ", f64(dq), rdq, dt, edq)
    assert_close("dK", f64(dk), rdk, dt, edk)
    assert_close("dV", f64(dv), rdv, dt, edv)


@pytest.mark.parametrize("Tq,Tk,D", [(100, 700, 128), (1, 300, 64), (257, 1000, 64)])
def test_bottom_right_rows_equal_the_square_problems_rows(Tq, Tk, D):
    """With the default offset, o, lse and dq of the Tq query rows are, bit for
    bit, the last Tq rows of the square causal problem over the same keys: each
    row walks the same key tiles in the same order (tiles past its last key
    add exact zeros).  dq comes from the unsplit dQ stage here (a split cuts a
    row's key range at boundaries that depend on its query block)."""
    x = to_dev(make_inputs(1, 4, 2, Tk, D, bf16, seed=9100 + Tq))
    q, k, v, do = x["q"], x["k"], x["v"], x["dout"]
    qt, dot = q[:, :, Tk - Tq:].contiguous(), do[:, :, Tk - Tq:].contiguous()
    say(f"bottom-right rows Tq={Tq} Tk={Tk} D={D}")
    o_sq, lse_sq = fa.fwd(q, k, v, causal=True)
    o_kv, lse_kv = fa.fwd(qt, k, v, causal=True)
    dq_sq = fa.bwd_dq(q, k, v, do, lse_sq, fa.bwd_preprocess(o_sq, do), causal=True)
    dq_kv = fa.bwd_dq(qt, k, v, dot, lse_kv, fa.bwd_preprocess(o_kv, dot), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o_kv, o_sq[:, :, Tk - Tq:])
    assert torch.equal(lse_kv, lse_sq[:, :, Tk - Tq:])
    assert torch.equal(dq_kv, dq_sq[:, :, Tk - Tq:])


@pytest.mark.parametrize("dt", [bf16, fp32])
def test_no_query_rows_gives_zero_key_gradients(dt):
    """Tq = 0: nothing to compute for the queries; every key gets dk = dv = 0
    (the outputs are overwritten, never left stale)."""
    x = to_dev(make_inputs(1, 2, 1, 0, 128, dt, seed=9200, Tk=300))
    say(f"no query rows {dt}")
    o, lse = fa.fwd(x["q"], x["k"], x["v"], causal=True)
    dk = torch.full_like(x["k"], 7.0)
    dv = torch.full_like(x["v"], 7.0)
    dq = torch.empty_like(x["q"])
    fa.bwd(x["q"], x["k"], x["v"], o, x["dout"], lse, causal=True, grads=(dq, dk, dv))
    torch.cuda.synchronize()
    assert o.numel() == 0 and lse.numel() == 0
    assert torch.count_nonzero(dk).item() == 0 and torch.count_nonzero(dv).item() == 0


def test_kv_call_with_equal_lengths_equals_the_square_call():
    """fa_fwd_kv / fa_bwd_kv with Tq = Tk and offset 0 are the square calls."""
    x = to_dev(make_inputs(1, 4, 2, 333, 128, bf16, seed=9300))
    lib = fa.library()
    q, k, v, do = x["q"], x["k"], x["v"], x["dout"]
    say("kv call with equal lengths")
    o, lse = fa.fwd(q, k, v, causal=True)
    o2, lse2 = torch.empty_like(o), torch.empty_like(lse)
    st = torch.cuda.current_stream().cuda_stream
    assert lib.fa_fwd_kv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o2.data_ptr(), lse2.data_ptr(),
                         1, 4, 2, 333, 333, 128, S128, 1, 0, 0, st) == 0
    dq, dk, dv = fa.bwd(q, k, v, o, do, lse, causal=True)
    g2 = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    ws = torch.empty(fa.bwd_workspace_bytes(1, 4, 2, 333, 128), dtype=torch.uint8, device="cuda")
    assert lib.fa_bwd_kv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                         lse.data_ptr(), g2[0].data_ptr(), g2[1].data_ptr(), g2[2].data_ptr(),
                         ws.data_ptr(), 1, 4, 2, 333, 333, 128, S128, 1, 0, 0, st) == 0
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
    assert torch.equal(dq, g2[0]) and torch.equal(dk, g2[1]) and torch.equal(dv, g2[2])
