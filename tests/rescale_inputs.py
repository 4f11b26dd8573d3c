"""Seeded inputs whose scores jump at key-tile boundaries — an input
generator only (no attention arithmetic).

The online softmax rescales its running numerator and sum whenever the running
max of a row rises ("L'attention fusionnée", «Le softmax en ligne»; the
rescale factor exp(m - m') of "FlashAttention: l'attenzione che non spreca
memoria", «La online softmax, con i numeri»).  The kernels move their
reference max only when a row's scores rise by more than 8 log2 units (5.55 in
natural units of the scaled score) above it, which N(0,1) inputs at the usual
scales never do after the first tile.  These inputs make them do it.

Construction, with scale = 1/8 and keys in tiles of 64 (key j is in tile
j // 64, the tile grid of every kernel):
  q[..., :8] = a,             q[..., 8:] = N(0,1)/2
  k[..., j, :8] = L_t / a,    k[..., 8:] = N(0,1)/2     (t = j // 64)
so the scaled score of key j is L_t plus a noise of standard deviation
sqrt(D-8)/32 (0.23 at D = 64, 0.34 at D = 128).  The level is spread over 8
dimensions because a key component common to the visible keys scales the
bf16 rounding of dS into dQ (the dS of a row sum to zero, their roundings do
not) by scale times that component, and the query component scales dK the same
way: with a = 8 both factors stay at most 1 (and no e4m3 product exceeds
|L_t|); the big-rise case, whose early rows see levels down to -146, takes
a = 32; the fp32 cases take a = 2, which keeps dK of order one for its
absolute 1e-5 target.  The level sequence L_t of
each (batch, kv head) starts at 0 and moves per tile by a step drawn from
  +12 (a jump of 17.3 log2 units: the reference must move),
  +8  (11.5 log2 units: must move),
  +4  (5.8 log2 units: no move, but a lane's share of the tile sum exceeds 2^8),
   0, -8,
with the second tile always a +12 jump, the last but one at the running max
and the last 12 above it (the others stay at most 36, then drop by 40).  Levels stay within [-40, 48], so
8 L_t is exact in bf16 and in e4m3 (multiples of 32 up to 384).  v and dout
are N(0,1).  With big_rise the steps are +12 or +8 only, without the cap, so
the levels climb past 89 natural units (128 log2 units): weights taken against
the first tile's max would overflow fp32.
"""
from __future__ import annotations

import numpy as np
import torch

TILE = 64
SCALE = 0.125
STEPS = (12, 8, 4, 0, -8)
STEP_P = (0.3, 0.15, 0.2, 0.2, 0.15)
LEVEL_MAX, LEVEL_MIN = 48, -40
TOP = 6.0      # top level of every sequence after the shift
E4M3_TOP, E4M3_MIN_LEVEL = 4.0, -60.0


def levels(ntiles: int, rng: np.random.Generator, big_rise: bool = False,
           top: float = TOP) -> np.ndarray:
    L = np.zeros(ntiles)
    for t in range(1, ntiles):
        if t == 1 or t == ntiles - 1:
            step = 12
        elif big_rise:
            step = 12 if rng.random() < 0.8 else 8
        else:
            step = STEPS[rng.choice(len(STEPS), p=STEP_P)]
        nxt = L[t - 1] + step
        if not big_rise and t == ntiles - 2 and t > 1:
            nxt = L[:t].max()  # back at the running max ...
        elif not big_rise and t == ntiles - 1 and t > 1:
            nxt = L[:t].max() + 12  # ... then above it: the reference moves
        elif not big_rise and nxt > LEVEL_MAX - 12:
            nxt = L[t - 1] - 40 if L[t - 1] - 40 >= LEVEL_MIN else LEVEL_MIN
        if nxt < LEVEL_MIN:
            nxt = LEVEL_MIN
        L[t] = nxt
    return L - L.max() + top


def make(B: int, Hq: int, Hkv: int, Tq: int, Tk: int, D: int, seed: int, big_rise: bool = False,
         top: float = TOP, a: float = 8.0):
    """float64 CPU arrays q [B,Hq,Tq,D], k, v [B,Hkv,Tk,D], dout [B,Hq,Tq,D]
    and the levels [B,Hkv,ntiles]; every value of q and k (and the scaled
    N(0,1) noise) is rounded to bf16 first, so the same numbers can be fed to
    every dtype (e4m3 callers round the noise again themselves)."""
    rng = np.random.default_rng(seed)
    nt = (Tk + TILE - 1) // TILE
    lv = np.stack([np.stack([levels(nt, rng, big_rise, top) for _ in range(Hkv)]) for _ in range(B)])
    q = 0.5 * rng.standard_normal((B, Hq, Tq, D))
    q[..., :8] = a
    k = 0.5 * rng.standard_normal((B, Hkv, Tk, D))
    k[..., :8] = (np.repeat(lv, TILE, axis=2)[:, :, :Tk] / a)[..., None]
    v = rng.standard_normal((B, Hkv, Tk, D))
    do = rng.standard_normal((B, Hq, Tq, D))
    r = lambda a: torch.from_numpy(a).to(torch.bfloat16).double().numpy()  # noqa: E731
    return {"q": r(q), "k": r(k), "v": r(v), "dout": r(do)}, lv


def as_torch(x: dict, dtype: torch.dtype) -> dict:
    """CPU tensors of the given dtype (exact for bf16 and fp32)."""
    return {n: torch.from_numpy(np.ascontiguousarray(a)).to(dtype).contiguous() for n, a in x.items()}


# The shapes the rescale tests run: name -> (B, Hq, Hkv, Tq, Tk, D, causal,
# q_offset, seed, big_rise).  The split case has few query blocks, so the
# forward cuts its key range into chunks (8 chunks of 4 tiles each for the
# last query block).
CASES = {
    "causal_gqa_t1000_d128": (2, 4, 2, 1000, 1000, 128, True, 0, 31, False),
    "full_t700_d64": (1, 2, 1, 700, 700, 64, False, 0, 32, False),
    "causal_split_t2048_d128": (1, 2, 1, 2048, 2048, 128, True, 0, 33, False),
    "causal_offset_q300_k900_d64": (1, 4, 2, 300, 900, 64, True, 250, 34, False),
    "big_rise_causal_t1000_d64": (1, 2, 1, 1000, 1000, 64, True, 0, 35, True),
}
FP32_CASES = {
    "fp32_full_t700_d64": (1, 2, 1, 700, 700, 64, False, 0, 36, False),
    "fp32_big_rise_full_t700_d128": (1, 2, 2, 700, 700, 128, False, 0, 37, True),
}
FP8_CASES = {
    "fp8_causal_gqa_t1000_d128": (1, 4, 2, 1000, 1000, 128, True, 0, 38, False),
    "fp8_full_t700_d64": (1, 2, 1, 700, 700, 64, False, 0, 39, False),
}


def e4m3(a: np.ndarray) -> np.ndarray:
    """Round to the nearest e4m3 value (torch.float8_e4m3fn), back in float64."""
    return torch.from_numpy(np.asarray(a, np.float64)).to(torch.float8_e4m3fn).double().numpy()


def make_case(name: str):
    """(inputs, levels) of a named case; the e4m3 cases have q, k, v rounded
    to e4m3 (the level column is exact in e4m3)."""
    allc = {**CASES, **FP32_CASES, **FP8_CASES}
    B, Hq, Hkv, Tq, Tk, D, causal, off, seed, big = allc[name]
    a = 2.0 if name in FP32_CASES else (32.0 if big else 8.0)
    x, lv = make(B, Hq, Hkv, Tq, Tk, D, seed, big, E4M3_TOP if name in FP8_CASES else TOP, a)
    if name in FP8_CASES:
        lv = np.maximum(lv, E4M3_MIN_LEVEL)
        x["k"][..., :8] = (np.repeat(lv, TILE, axis=2)[:, :, :Tk] / a)[..., None]
        x = {n: (e4m3(t) if n != "dout" else t) for n, t in x.items()}
    want = (np.repeat(lv, TILE, axis=2)[:, :, :Tk] / a)[..., None]
    assert np.array_equal(x["k"][..., :8], np.broadcast_to(want, x["k"][..., :8].shape))
    return x, lv


def fig79_inputs(lam: float, Tq: int = 64, D: int = 64):
    """The row of Fig. 7.9 of "FlashAttention: l'attenzione che non spreca
    memoria" («La online softmax, con i numeri»: eight scores read two at a
    time, with their values), spread over four 64-key tiles: block b's two
    keys sit at positions 64b + 2 and 64b + 45 (one in each lane half), with
    scores lam * s; the other keys score -1000 (weights underflow to zero)
    and carry random values.  Every query row is e_0 (scale 1), so each row
    is that row of the figure.  Returns (float64 inputs, scale)."""
    from tests.conftest import read_golden

    g = read_golden("fig79_eight_scores.txt")
    sc, vals, bs = g["scores"], g["values"], int(g["block_size"])
    Tk = TILE * (len(sc) // bs)
    rng = np.random.default_rng(79)
    q = np.zeros((1, 1, Tq, D))
    q[..., 0] = 1.0
    k = np.zeros((1, 1, Tk, D))
    k[..., 0] = -1000.0
    v = rng.standard_normal((1, 1, Tk, D))
    for n, (s, val) in enumerate(zip(sc, vals)):
        j = TILE * (n // bs) + (2 if n % bs == 0 else 45)
        k[0, 0, j, 0] = lam * s
        v[0, 0, j, 0] = val
    r = lambda a: torch.from_numpy(a).to(torch.bfloat16).double().numpy()  # noqa: E731
    return {"q": r(q), "k": r(k), "v": r(v)}, 1.0
