"""The forward and backward captured in a HIP graph and replayed.

A step of fa_fwd (split where the shapes call for it) and fa_bwd, captured
once on torch's capture stream, is replayed three times.  Between replays,
eager calls on other inputs overwrite the same output and scratch buffers and
the host synchronises, so every replay must recompute everything; each must
equal the eager result bit for bit (the kernels are deterministic).  The
library records no memset or allocation into the graph: its launch path is
kernels only.
"""
import pytest
import torch

import exact_attention_30_amd as fa
from tests.gpu_util import say
from workloads import make_inputs

pytestmark = pytest.mark.gpu

# B, Hq, Hkv, T, D, causal, dtype
CASES = {
    "c2_shape_split": (2, 8, 8, 512, 64, True, torch.bfloat16),
    "gqa_t1500_d128_split": (1, 4, 2, 1500, 128, True, torch.bfloat16),
    "full_t300_d64": (1, 4, 4, 300, 64, False, torch.bfloat16),
    "fp32_t150_d64": (1, 2, 1, 150, 64, True, torch.float32),
}


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replay_equals_eager(name):
    B, Hq, Hkv, T, D, causal, dt = CASES[name]
    say(f"graph {name}: B={B} Hq={Hq} Hkv={Hkv} T={T} D={D} causal={causal} {dt}")
    x = {n: t.cuda() for n, t in make_inputs(B, Hq, Hkv, T, D, dt, seed=4242).items()}
    y = {n: t.cuda() for n, t in make_inputs(B, Hq, Hkv, T, D, dt, seed=4343).items()}
    scale = D ** -0.5
    o = torch.empty_like(x["q"])
    lse = torch.empty(B, Hq, T, dtype=torch.float32, device="cuda")
    grads = (torch.empty_like(x["q"]), torch.empty_like(x["k"]), torch.empty_like(x["v"]))
    fpart = torch.empty(max(fa.fwd_split_bytes(B, Hq, Hkv, T, T, D, dt), 16), dtype=torch.uint8,
                        device="cuda")
    ws = torch.empty(max(fa.bwd_workspace_bytes(B, Hq, Hkv, T, D, dt), 16), dtype=torch.uint8,
                     device="cuda")

    def step(a):
        fa.fwd(a["q"], a["k"], a["v"], scale=scale, causal=causal, out=o, lse=lse, partial=fpart)
        fa.bwd(a["q"], a["k"], a["v"], o, a["dout"], lse, scale=scale, causal=causal, workspace=ws,
               grads=grads)

    step(x)
    torch.cuda.synchronize()
    ref = [t.clone() for t in (o, lse, *grads)]
    step(y)
    torch.cuda.synchronize()
    other = [t.clone() for t in (o, lse, *grads)]
    assert any(not torch.equal(a, b) for a, b in zip(ref, other))

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(x)
    for r in range(3):
        step(y)  # eager work on the same buffers between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n, got, want in zip(("o", "lse", "dq", "dk", "dv"), (o, lse, *grads), ref):
            assert torch.equal(got, want), f"replay {r}: {n} differs from the eager result"
