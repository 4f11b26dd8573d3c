"""A CPU model of the forward kernels' tile loop with a lazy reference max —
test-side arithmetic, neither the oracle nor the library.

It follows the online softmax of "L'attention fusionnée" («Le softmax en
ligne») tile by tile, with the kernels' one departure from it: the reference
max m of a row moves only when a tile's row max exceeds it by more than
THRESHOLD log2 units; then the numerator o and the sum l are multiplied by
2^(m - m') and the tile's weights are formed against m'.  Otherwise the
weights 2^(s c - m) are formed against the old reference (they stay below
2^THRESHOLD).  With the key range of a query block cut into chunks, each chunk
runs the loop on its own and the chunks merge by the block merge rule
("FlashAttention" note, «Blockergebnisse…»).

Its uses in the tests:
  * `mutant` plants one mistake in the reference update, to show that the
    inputs of the rescale tests (tests/rescale_inputs.py) make such a
    mistake visible at the bf16 tolerance;
  * `record` lists the tiles where a row's reference moved after its first
    visible tile, and those where a lane's share of the tile sum exceeded
    2^THRESHOLD without a move, to show those inputs reach the branch.

Per head, float64: q [Tq, D], k, v [Tk, D].  Query row i sees key j iff
j <= i + q_offset when causal.  Tiles hold 64 keys, a query block 256 rows
(the kernels' shapes); a lane holds the keys j of a tile with (j mod 8) // 4
equal to its half g (the 32x32 accumulator layout).
"""
from __future__ import annotations

import math

import numpy as np

THRESHOLD = 8.0
TILE = 64
BLOCK = 256
LOG2E = 1.0 / math.log(2.0)
FP32_MAX = 3.4028234663852886e38
MUTANTS = ("no_o_rescale", "no_l_rescale", "stale_weights", "alpha_inverted",
           "prev_tile_unscaled", "never_move")


def block_rows(B, Hq, Tq, D):
    """Query rows per workgroup of the bf16 forward (the library's tile
    table): 128 at D = 64 when the 256-row blocks number fewer than 512,
    else 256."""
    n256 = ((Tq + BLOCK - 1) // BLOCK) * B * Hq
    return 128 if D == 64 and n256 < 512 else BLOCK


def nsplit(B, Hq, Tq, Tk, D):
    """Chunks per query block of the split forward: about 512 workgroups,
    at most 8 chunks, at least 4 key tiles per chunk, 8 with 128-row blocks
    (the library's rule)."""
    br = block_rows(B, Hq, Tq, D)
    wgs = ((Tq + br - 1) // br) * B * Hq
    if wgs <= 0 or wgs >= 512:
        return 1
    s = min(8, (512 + wgs - 1) // wgs)
    cap = max(1, ((Tk + TILE - 1) // TILE) // (8 if br == 128 else 4))
    return min(s, cap)


def _fp32(x):
    """Values past the fp32 range become inf (the kernels' weights are fp32)."""
    with np.errstate(invalid="ignore"):
        return np.where(np.abs(x) > FP32_MAX, np.copysign(np.inf, x), x)


def forward_head(q, k, v, scale, causal, q_offset=0, S=1, round_p=None, mutant=None, record=None,
                 blocks=None, block=BLOCK):
    """O [Tq, D] and lse [Tq] of one head, in query blocks of `block` rows
    (which only matters with S > 1: they set where the chunks start).
    round_p rounds the weights that enter P V (not the sum l), e.g. to bf16;
    mutant is one of MUTANTS.  With `blocks` (query block indices), only
    those blocks' rows are computed (the others are left zero)."""
    Tq, D = q.shape
    Tk = k.shape[0]
    c = scale * LOG2E
    out = np.zeros((Tq, D))
    lse = np.zeros(Tq)
    ntk = (Tk + TILE - 1) // TILE
    for q0 in range(0, Tq, block):
        if blocks is not None and q0 // block not in blocks:
            continue
        rows = np.arange(q0, min(q0 + block, Tq))
        kend = min(q0 + block + q_offset, Tk) if causal else Tk
        nall = (kend + TILE - 1) // TILE
        s_blk = (q[rows] @ k[:nall * TILE].T) * c  # log2 units
        if causal:
            vis = np.arange(s_blk.shape[1])[None, :] <= rows[:, None] + q_offset
            s_blk = np.where(vis, s_blk, -np.inf)
        parts = []
        for sp in range(S):
            j0, j1 = nall * sp // S, nall * (sp + 1) // S
            n = len(rows)
            mref = np.full(n, -np.inf)
            l = np.zeros(n)
            o = np.zeros((n, D))
            last = np.zeros((n, D))  # the previous tile's P V contribution
            for t in range(j0, min(j1, ntk)):
                kk = slice(t * TILE, min((t + 1) * TILE, Tk))
                st = s_blk[:, kk]
                msub = np.where(mref == -np.inf, 0.0, mref)
                w = _fp32(np.exp2(st - msub[:, None]))
                mt = st.max(axis=1)
                move = mt > mref + THRESHOLD
                if mutant == "never_move":
                    move &= mref == -np.inf
                if record is not None:
                    lane = ((np.arange(kk.start, kk.stop) - t * TILE) % 8) // 4
                    share = np.stack([w[:, lane == g].sum(axis=1) for g in (0, 1)], axis=1)
                    nvis = np.isfinite(st).sum(axis=1)
                    for r in np.nonzero(move & (mref > -np.inf))[0]:
                        record.append(dict(kind="move", row=int(rows[r]), tile=t, local=t - j0,
                                           chunk=sp, S=S, row_last=_row_last(rows[r], j0, j1, Tk,
                                                                             causal, q_offset),
                                           nkw=_nkw(rows[r], j0, j1, Tk, causal, q_offset)))
                    for r in np.nonzero(~move & (share.max(axis=1) > 2.0 ** THRESHOLD)
                                        & (nvis > 0))[0]:
                        record.append(dict(kind="checked", row=int(rows[r]), tile=t, chunk=sp))
                if move.any():
                    mnew = np.where(move, mt, mref)
                    with np.errstate(invalid="ignore"):
                        alpha = np.where(move, np.where(mref == -np.inf, 0.0,
                                                        np.exp2(np.minimum(mref - mnew, 0.0))), 1.0)
                    if mutant == "alpha_inverted":
                        alpha = np.where(move & (mref > -np.inf), np.exp2(mnew - mref), alpha)
                    if mutant != "no_l_rescale":
                        l = l * alpha
                    if mutant == "prev_tile_unscaled":
                        o = (o - last) * alpha[:, None] + last
                    elif mutant != "no_o_rescale":
                        o = o * alpha[:, None]
                    mref = mnew
                    if mutant != "stale_weights":
                        msub = np.where(mref == -np.inf, 0.0, mref)
                        w = _fp32(np.exp2(st - msub[:, None]))
                l = l + w.sum(axis=1)
                wp = w if round_p is None else round_p(w)
                last = wp @ v[kk]
                o = o + last
            parts.append((o, mref, l))
        M = np.max(np.stack([p[1] for p in parts]), axis=0)
        num = np.zeros((len(rows), D))
        den = np.zeros(len(rows))
        for o, m, l in parts:
            wgt = np.where(m == -np.inf, 0.0, np.exp2(np.where(m == -np.inf, 0.0, m - M)))
            num += wgt[:, None] * o
            den += wgt * l
        with np.errstate(invalid="ignore", divide="ignore"):
            out[rows] = num / den[:, None]
            lse[rows] = (M + np.log2(den)) / LOG2E
    return out, lse


def forward_head_all_rows(q, k, v, scale, causal, q_offset=0, round_p=None):
    """forward_head for the unsplit forward (S = 1, no mutant, no record),
    with every query row advanced through the tiles together in torch (CPU,
    float64, all host threads): the same loop, for sizes where forward_head
    takes minutes.  round_p takes and returns a float64 torch tensor."""
    import torch

    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64)) for a in (q, k, v))
    Tq, D = q.shape
    Tk = k.shape[0]
    c = scale * LOG2E
    rows = torch.arange(Tq, dtype=torch.float64)[:, None]
    mref = torch.full((Tq,), -np.inf, dtype=torch.float64)
    l = torch.zeros(Tq, dtype=torch.float64)
    o = torch.zeros(Tq, D, dtype=torch.float64)
    for t in range((Tk + TILE - 1) // TILE):
        k0, k1 = t * TILE, min((t + 1) * TILE, Tk)
        st = (qt @ kt[k0:k1].T) * c
        if causal:
            keys = torch.arange(k0, k1, dtype=torch.float64)[None, :]
            st = torch.where(keys <= rows + q_offset, st, torch.tensor(-np.inf, dtype=torch.float64))
        mt = st.max(dim=1).values
        move = mt > mref + THRESHOLD
        if bool(move.any()):
            mnew = torch.where(move, mt, mref)
            alpha = torch.where(move & (mref > -np.inf), torch.exp2(torch.clamp(mref - mnew, max=0.0)),
                                torch.where(move, torch.zeros_like(mref), torch.ones_like(mref)))
            l = l * alpha
            o = o * alpha[:, None]
            mref = mnew
        msub = torch.where(mref == -np.inf, torch.zeros_like(mref), mref)
        w = torch.exp2(st - msub[:, None])
        l = l + w.sum(dim=1)
        o = o + (w if round_p is None else round_p(w)) @ vt[k0:k1]
    out = (o / l[:, None]).numpy()
    lse = ((mref + torch.log2(l)) / LOG2E).numpy()
    return out, lse


def _row_last(i, j0, j1, Tk, causal, off):
    """Last tile of the chunk [j0, j1) with a key row i sees (-1: none)."""
    last_key = min(Tk - 1, i + off) if causal else Tk - 1
    return min(j1 - 1, last_key // TILE) if last_key >= j0 * TILE else -1


def _nkw(i, j0, j1, Tk, causal, off):
    """Tiles the wave of row i computes in the chunk [j0, j1): those some of
    its 32 rows see (the kernels' waves hold 32 consecutive rows)."""
    nkv = j1 - j0
    if not causal:
        return nkv
    qw = i - i % 32
    return min(nkv, max(0, (qw + 32 + off + TILE - 1) // TILE - j0))


def forward(q, k, v, scale, causal, q_offset=None, S=1, round_p=None, mutant=None, record=None,
            block=BLOCK):
    """O [B,Hq,Tq,D], lse [B,Hq,Tq] over all heads (GQA: kv head h // G)."""
    B, Hq, Tq, D = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    off = Tk - Tq if q_offset is None else q_offset
    G = Hq // Hkv
    o = np.zeros(q.shape)
    lse = np.zeros((B, Hq, Tq))
    for b in range(B):
        for h in range(Hq):
            rec = [] if record is not None else None
            o[b, h], lse[b, h] = forward_head(q[b, h], k[b, h // G], v[b, h // G], scale, causal,
                                              off if causal else 0, S, round_p, mutant, rec,
                                              block=block)
            if rec is not None:
                for e in rec:
                    e.update(b=b, h=h)
                record.extend(rec)
    return o, lse
