"""fa_bwd_noalloc, the backward for callers that cannot allocate (its
workspace is the library's static per-GPU scratch), through the C ABI,
against fa_bwd_kv with a caller workspace: the same kernels, so the same bits.
Two calls in a row, the second smaller (the scratch keeps the first call's
contents), then fp32 and Tq != Tk; no device memory is allocated by the call;
shapes whose workspace exceeds the scratch are refused before any launch."""
import pytest
import torch

import exact_attention_30_amd as fa
from tests.gpu_util import say
from workloads import make_inputs

pytestmark = pytest.mark.gpu

bf16, fp32 = torch.bfloat16, torch.float32


def check(B, Hq, Hkv, Tq, Tk, D, dt, causal, q_offset, seed):
    say(f"noalloc B={B} Hq={Hq} Hkv={Hkv} Tq={Tq} Tk={Tk} D={D} {dt} causal={causal} "
        f"off={q_offset}")
    assert fa.bwd_workspace_bytes(B, Hq, Hkv, Tq, D, dt, Tk=Tk) <= fa.NOALLOC_SCRATCH_BYTES
    x = {n: t.cuda() for n, t in make_inputs(B, Hq, Hkv, Tq, D, dt, seed=seed, Tk=Tk).items()}
    kw = dict(causal=causal, q_offset=q_offset)
    o, lse = fa.fwd(x["q"], x["k"], x["v"], **kw)
    want = fa.bwd(x["q"], x["k"], x["v"], o, x["dout"], lse, **kw)
    grads = tuple(torch.full_like(t, float("nan")) for t in want)
    torch.cuda.synchronize()
    alloc0 = torch.cuda.memory_allocated()
    free0, _ = torch.cuda.mem_get_info()
    got = fa.bwd_noalloc(x["q"], x["k"], x["v"], o, x["dout"], lse, grads=grads, **kw)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert torch.cuda.memory_allocated() == alloc0
    assert free1 == free0
    for a, b in zip(got, want):
        assert torch.equal(a, b)


def setup_call():
    """The first call on a device looks up its scratch (the runtime may
    materialise the static array then); later calls allocate nothing."""
    x = {n: t.cuda() for n, t in make_inputs(1, 1, 1, 8, 64, bf16, seed=0).items()}
    o, lse = fa.fwd(x["q"], x["k"], x["v"])
    fa.bwd_noalloc(x["q"], x["k"], x["v"], o, x["dout"], lse)
    torch.cuda.synchronize()


def test_noalloc_equals_fa_bwd():
    setup_call()
    # bf16 whose dK/dV and dQ stages split: Delta and the partial sums in the scratch
    assert fa.dkdv_split_bytes(1, 4, 2, 1500, 1500, 128) > 0
    assert fa.dq_split_bytes(1, 4, 2, 1500, 1500, 128) > 0
    check(1, 4, 2, 1500, 1500, 128, bf16, True, None, 1)
    # a second, smaller call: the first call's contents are still in the scratch
    check(1, 4, 2, 700, 700, 64, bf16, False, None, 2)
    # fp32 (Delta from the preprocess kernel) and Tq != Tk with an offset
    check(1, 2, 1, 300, 300, 64, fp32, True, None, 3)
    check(1, 4, 2, 300, 900, 128, bf16, True, 250, 4)


def test_noalloc_refuses_workspace_past_the_scratch():
    """One kv group at T = 16384: its split dK/dV stage needs 128 MiB of fp32
    partial sums, past the 64 MiB scratch: FA_ERR_SCRATCH, nothing launched."""
    B, Hq, Hkv, T, D = 1, 4, 1, 16384, 128
    assert fa.bwd_workspace_bytes(B, Hq, Hkv, T, D) > fa.NOALLOC_SCRATCH_BYTES
    x = {n: t.cuda() for n, t in make_inputs(B, Hq, Hkv, T, D, bf16, seed=5).items()}
    lse = torch.zeros(B, Hq, T, device="cuda")
    say("noalloc refusal")
    with pytest.raises(fa.FAError) as e:
        fa.bwd_noalloc(x["q"], x["k"], x["v"], x["q"], x["dout"], lse)
    assert e.value.status == 6
