"""The single-kernel backward with atomic dQ (fa_bwd_atomic), the FA2
formulation of "L'attention fusionnée", «La passe arrière»: dK and dV stay in
the dK/dV kernel's registers and every query tile's share of dQ is added to
fp32 accumulators with atomic adds.

dK and dV come from the same kernel code as the two-kernel backward's dK/dV
stage and must equal it bit for bit; dQ sums the same bf16 dS times K in
another order (per 256-key block, then across blocks in whatever order the
atomics land), so it is held to the oracle at the bf16 tolerance (with the
rounding emulation where the method's own roundings exceed it) and to the
two-kernel backward's dQ within a few bf16 steps.
"""
import numpy as np
import pytest
import torch

import exact_attention_30_amd as fa
import oracle
from tests.gpu_util import assert_grad_close, emulated_fwd, emulated_grads, f64, say
from workloads import make_inputs

pytestmark = pytest.mark.gpu

bf16 = torch.bfloat16

# B, Hq, Hkv, T, causal
CASES = {
    "c2_shape": (2, 8, 8, 512, True),
    "gqa2_t1000_ragged": (1, 4, 2, 1000, True),
    "full_t300": (1, 4, 4, 300, False),
    "gqa3_t777_ragged": (2, 6, 2, 777, True),
}


@pytest.mark.parametrize("name", list(CASES))
def test_atomic_backward(name):
    B, Hq, Hkv, T, causal = CASES[name]
    D, scale = 64, 0.125
    say(f"atomic backward {name}: B={B} Hq={Hq} Hkv={Hkv} T={T} causal={causal}")
    x = make_inputs(B, Hq, Hkv, T, D, bf16, seed=900 + T)
    d = {n: t.cuda() for n, t in x.items()}
    o, lse = fa.fwd(d["q"], d["k"], d["v"], scale=scale, causal=causal)
    dq, dk, dv = fa.bwd_atomic(d["q"], d["k"], d["v"], o, d["dout"], lse, scale=scale, causal=causal)
    delta = fa.bwd_preprocess(o, d["dout"])
    dk0, dv0 = fa.bwd_dkdv(d["q"], d["k"], d["v"], d["dout"], lse, delta, scale=scale, causal=causal)
    dq0, _, _ = fa.bwd(d["q"], d["k"], d["v"], o, d["dout"], lse, scale=scale, causal=causal)
    torch.cuda.synchronize()
    assert torch.equal(dk, dk0) and torch.equal(dv, dv0)
    a, b = f64(dq), f64(dq0)
    assert np.all(np.abs(a - b) <= 2.0 ** -6 * np.abs(b) + 2e-3), float(np.max(np.abs(a - b)))
    xs = {n: t.double().numpy() for n, t in x.items()}
    rdq, _, _ = oracle.bwd(xs["q"], xs["k"], xs["v"], xs["dout"], scale, causal)
    _, rl = oracle.fwd(xs["q"], xs["k"], xs["v"], scale, causal)
    eo = emulated_fwd(xs, scale, causal)
    eq, _, _ = emulated_grads(xs, eo, rl, scale, causal)
    assert_grad_close(f"dQ atomic {name}", a, rdq, eq)
