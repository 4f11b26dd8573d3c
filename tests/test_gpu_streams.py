"""Two steps at once on two streams.

The forward and backward entry points keep no state outside the buffers the
caller passes (outputs, split scratch, workspace), so a step of fa_fwd and
fa_bwd on one stream and another step on a second stream, each with its own
buffers, must not disturb each other: both results equal, bit for bit, those
of the same steps run one after the other (the kernels are deterministic).
The shapes split every stage, so the chunk partials and merges are in play.
Both streams have the default priority.
"""
import pytest
import torch

import exact_attention_30_amd as fa
from tests.gpu_util import say
from workloads import make_inputs

pytestmark = pytest.mark.gpu

# B, Hq, Hkv, T, D, causal
CASES = {
    "one_kv_group_d128": (1, 4, 1, 2048, 128, True),
    "mha_d64": (1, 4, 4, 1500, 64, True),
    "gqa_d96_noncausal": (1, 4, 2, 700, 96, False),
}


def _buffers(B, Hq, Hkv, T, D, dt):
    dev = "cuda"
    o = torch.empty(B, Hq, T, D, dtype=dt, device=dev)
    lse = torch.empty(B, Hq, T, dtype=torch.float32, device=dev)
    grads = (torch.empty(B, Hq, T, D, dtype=dt, device=dev), torch.empty(B, Hkv, T, D, dtype=dt, device=dev),
             torch.empty(B, Hkv, T, D, dtype=dt, device=dev))
    part = torch.empty(max(fa.fwd_split_bytes(B, Hq, Hkv, T, T, D, dt), 16), dtype=torch.uint8, device=dev)
    ws = torch.empty(max(fa.bwd_workspace_bytes(B, Hq, Hkv, T, D, dt), 16), dtype=torch.uint8, device=dev)
    return o, lse, grads, part, ws


def _step(x, bufs, scale, causal):
    o, lse, grads, part, ws = bufs
    fa.fwd(x["q"], x["k"], x["v"], scale=scale, causal=causal, out=o, lse=lse, partial=part)
    fa.bwd(x["q"], x["k"], x["v"], o, x["dout"], lse, scale=scale, causal=causal, workspace=ws, grads=grads)
    return [o, lse, *grads]


@pytest.mark.parametrize("name", list(CASES))
def test_two_streams_equal_sequential(name):
    B, Hq, Hkv, T, D, causal = CASES[name]
    dt = torch.bfloat16
    say(f"streams {name}: B={B} Hq={Hq} Hkv={Hkv} T={T} D={D} causal={causal}")
    scale = D ** -0.5
    x = {n: t.cuda() for n, t in make_inputs(B, Hq, Hkv, T, D, dt, seed=5151).items()}
    y = {n: t.cuda() for n, t in make_inputs(B, Hq, Hkv, T, D, dt, seed=5252).items()}
    assert fa.fwd_split_bytes(B, Hq, Hkv, T, T, D, dt) > 0 or fa.bwd_workspace_bytes(B, Hq, Hkv, T, D, dt) > 0

    bx, by = _buffers(B, Hq, Hkv, T, D, dt), _buffers(B, Hq, Hkv, T, D, dt)
    ref_x = [t.clone() for t in _step(x, bx, scale, causal)]
    ref_y = [t.clone() for t in _step(y, by, scale, causal)]
    torch.cuda.synchronize()
    assert any(not torch.equal(a, b) for a, b in zip(ref_x, ref_y))

    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    for r in range(3):
        for t in bx[:2] + by[:2]:
            t.zero_()
        for t in bx[2] + by[2]:
            t.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            got_x = _step(x, bx, scale, causal)
        with torch.cuda.stream(s2):
            got_y = _step(y, by, scale, causal)
        torch.cuda.synchronize()
        for n, g, want in zip(("o", "lse", "dq", "dk", "dv"), got_x, ref_x):
            assert torch.equal(g, want), f"round {r}: stream 1 {n} differs from the sequential result"
        for n, g, want in zip(("o", "lse", "dq", "dk", "dv"), got_y, ref_y):
            assert torch.equal(g, want), f"round {r}: stream 2 {n} differs from the sequential result"
