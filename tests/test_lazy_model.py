"""CPU checks that the rescale tests' inputs reach the forward kernels'
reference-update branch and would expose a mistake in it.

The kernels move a row's reference max only when a tile's scores exceed it by
more than 8 log2 units (tests/lazy_model.py states the loop).  On the inputs
of tests/rescale_inputs.py:
  * the model without mistakes equals the oracle (exact arithmetic), and with
    its weights rounded to bf16 (e4m3 for the e4m3 cases) stays within the
    tolerance the GPU tests hold the kernels to;
  * the reference moves after a row's first tile at the places the GPU tests
    are meant to cover: the second tile of a chunk, tiles inside a wave's
    range with an odd and an even number of tiles, a row's last tile, and
    chunks after the first in the split forward; lanes' shares of a tile sum
    also exceed 2^8 without a move;
  * each planted mistake in the update (numerator or sum not rescaled, weights
    left against the old reference, the factor inverted, the previous tile's
    P V product left out of the rescale, a reference that never moves) gives
    O or lse outside that tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
from tests import lazy_model as lm
from tests.rescale_inputs import CASES, FP8_CASES, FP32_CASES, SCALE, e4m3, make_case
from tests.bf16_emulation import bf16
from tests.test_gpu_fp8 import E4M3_U, OUT_U, lse_bound, subnormal_term

ALL = {**CASES, **FP32_CASES, **FP8_CASES}
# (case, chunks): every case as the unsplit forward runs it, and the split
# case also as the split forward runs it (8 chunks per query block)
SPLIT_CASE = "causal_split_t2048_d128"
VARIANTS = [(n, 1) for n in ALL] + [(SPLIT_CASE, 8)]
IDS = [f"{n}-S{s}" for n, s in VARIANTS]


def within_target(name, o, lse):
    """The tolerance the GPU tests hold the kernels to: for bf16 max-abs <=
    1e-2 (relative above |ref| = 1) and rel-L2 <= 5e-3 on O, lse within
    1e-3; for e4m3 the derived per-element bound of the e4m3 forward; for
    fp32 max-abs 1e-5."""
    x, (ro, rl, om, sub, lsb) = reference(name)
    if not (np.all(np.isfinite(o)) and np.all(np.isfinite(lse))):
        return False
    if name in FP8_CASES:
        bound = E4M3_U * om + sub + OUT_U * np.abs(ro) + 1e-5
        return bool(np.all(np.abs(o - ro) <= bound) and np.all(np.abs(lse - rl) <= lsb))
    if name in FP32_CASES:
        return np.abs(o - ro).max() <= 1e-5 and np.abs(lse - rl).max() <= 1e-5
    err = np.abs(o - ro) / np.maximum(1.0, np.abs(ro))
    rel = np.linalg.norm(o - ro) / np.linalg.norm(ro)
    return err.max() <= 1e-2 and rel <= 5e-3 and np.abs(lse - rl).max() <= 1e-3


_ref = {}


def reference(name):
    if name not in _ref:
        B, Hq, Hkv, Tq, Tk, D, causal, off, seed, big = ALL[name]
        x, _ = make_case(name)
        ro, rl, om = oracle.fwd(x["q"], x["k"], x["v"], SCALE, causal, return_mag=True,
                                q_offset=off)
        sub = subnormal_term(x["q"], x["k"], x["v"], SCALE, causal, off)
        lsb = lse_bound(x["q"], x["k"], SCALE, causal, off)
        _ref[name] = (x, (ro, rl, om, sub, lsb))
    return _ref[name]


def rounding(name):
    return e4m3 if name in FP8_CASES else (None if name in FP32_CASES else bf16)


@pytest.mark.parametrize("name,S", VARIANTS, ids=IDS)
def test_model_matches_oracle(name, S):
    B, Hq, Hkv, Tq, Tk, D, causal, off, seed, big = ALL[name]
    x, (ro, rl, *_) = reference(name)
    o, lse = lm.forward(x["q"], x["k"], x["v"], SCALE, causal, off, S=S)
    assert np.max(np.abs(o - ro)) < 1e-9 and np.max(np.abs(lse - rl)) < 1e-9
    o, lse = lm.forward(x["q"], x["k"], x["v"], SCALE, causal, off, S=S,
                        round_p=rounding(name))
    assert within_target(name, o, lse)


@pytest.mark.parametrize("name,S", VARIANTS, ids=IDS)
@pytest.mark.parametrize("mutant", lm.MUTANTS)
def test_planted_mistakes_fail(name, S, mutant):
    B, Hq, Hkv, Tq, Tk, D, causal, off, seed, big = ALL[name]
    if mutant == "never_move" and not big and name not in FP8_CASES:
        pytest.skip("a reference that never moves is exact until the weights overflow: "
                    "only the big-rise inputs (past fp32) and e4m3 weights (past 448) show it")
    x, _ = reference(name)
    with np.errstate(all="ignore"):
        o, lse = lm.forward(x["q"], x["k"], x["v"], SCALE, causal, off, S=S,
                            round_p=rounding(name), mutant=mutant)
    assert not within_target(name, o, lse), f"{mutant} not caught on {name}"


def events(name, S):
    B, Hq, Hkv, Tq, Tk, D, causal, off, seed, big = ALL[name]
    x, _ = reference(name)
    rec = []
    lm.forward(x["q"], x["k"], x["v"], SCALE, causal, off, S=S, record=rec)
    return rec


@pytest.mark.parametrize("name,S", VARIANTS, ids=IDS)
def test_inputs_reach_the_branch(name, S):
    B, Hq, Hkv, Tq, Tk, D, causal, off, seed, big = ALL[name]
    rec = events(name, S)
    moves = [e for e in rec if e["kind"] == "move"]
    assert any(e["local"] == 1 for e in moves), "no move at a chunk's second tile"
    middle = [e for e in moves if 1 <= e["local"] < e["nkw"] - 1]
    assert any(e["nkw"] % 2 == 0 for e in middle) and any(e["nkw"] % 2 == 1 for e in middle) \
        or not causal, "no move inside a wave's range for both parities of its tile count"
    assert any(e["tile"] == e["row_last"] for e in moves), "no move at a row's last tile"
    if not big:
        assert any(e["kind"] == "checked" for e in rec), "no share above 2^8 without a move"


def test_split_case_moves_inside_later_chunks():
    B, Hq, Hkv, Tq, Tk, D, causal, off, seed, big = ALL[SPLIT_CASE]
    assert lm.nsplit(B, Hq, Tq, Tk, D) == 8
    moves = [e for e in events(SPLIT_CASE, 8) if e["kind"] == "move"]
    assert any(e["chunk"] >= 1 and e["local"] == 1 for e in moves)
    assert any(e["chunk"] >= 1 and e["tile"] == e["row_last"] for e in moves)
    # a chunk's last tile: tile j1 - 1 of a chunk that ends before the row's
    # diagonal (so the row continues in the next chunk)
    ends = [e for e in moves if e["chunk"] < 7 and e["tile"] == e["row_last"]
            and (e["row"] // 64) > e["tile"]]
    assert ends, "no move at the last tile of a chunk that a row continues past"


def test_fig79_scaled_moves_at_the_pages_blocks():
    """Fig. 7.9 of "FlashAttention: l'attenzione che non spreca memoria"
    (scores 1 3 2 4 1 0 5 2 in blocks of two): the running max rises at the
    2nd and 4th block.  Scaled by 8 and with each block in its own 64-key
    tile, the kernels' reference moves exactly there (each rise, 8 natural
    units, exceeds the threshold), and the scaled row still matches the
    oracle in the model."""
    from tests.rescale_inputs import fig79_inputs

    x, scale = fig79_inputs(8.0)
    rec = []
    o, lse = lm.forward(x["q"], x["k"], x["v"], scale, False, record=rec)
    ro, rl = oracle.fwd(x["q"], x["k"], x["v"], scale, False)
    assert np.max(np.abs(o - ro)) < 1e-9
    tiles = sorted({e["tile"] for e in rec if e["kind"] == "move" and e["row"] == 0})
    assert tiles == [1, 3]


@pytest.mark.parametrize("causal,off", [(True, 0), (False, 0), (True, 37)])
def test_all_rows_form_is_the_same_loop(causal, off):
    """The row-vectorised form of the unsplit loop (used for large emulations)
    gives the per-block loop's O and lse, with and without bf16 weights."""
    x, _ = make_case("big_rise_causal_t1000_d64")
    q, k, v = x["q"][0, 0, :700], x["k"][0, 0], x["v"][0, 0]
    for rp, rpt in ((None, None), (bf16, lambda t: t.to(torch.bfloat16).double())):
        o1, l1 = lm.forward_head(q, k, v, SCALE, causal, off, round_p=rp)
        o2, l2 = lm.forward_head_all_rows(q, k, v, SCALE, causal, off, round_p=rpt)
        assert np.max(np.abs(o1 - o2)) < 1e-12 and np.max(np.abs(l1 - l2)) < 1e-12
