"""CPU checks of the Python binding's argument checks: a tensor of the wrong
shape or dtype is refused with ValueError before anything reaches the library
(the kernels read and write exactly the elements the shapes imply, so a
smaller tensor would be overrun)."""
import pytest
import torch

import exact_attention_30_amd as fa

B, Hq, Hkv, T, D = 1, 4, 2, 64, 64
SHAPE_ERR = r"must have shape|must be torch\."  # not the device check, which comes later


def t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


Q, K, V = t(B, Hq, T, D), t(B, Hkv, T, D), t(B, Hkv, T, D)
LSE = t(B, Hq, T, dtype=torch.float32)


@pytest.mark.parametrize("kw", [dict(out=t(B, Hq, T - 1, D)), dict(out=t(B, Hq, T, D - 1, dtype=torch.float32)),
                                dict(lse=t(B, Hq, T - 1, dtype=torch.float32)),
                                dict(lse=t(B, Hq, T))])
def test_fwd_outputs(kw):
    with pytest.raises(ValueError, match=SHAPE_ERR):
        fa.fwd(Q, K, V, **kw)


@pytest.mark.parametrize("o,dout,lse,grads", [
    (t(B, Hq, T - 1, D), Q, LSE, None),
    (Q, t(B, Hq, T, D - 8), LSE, None),
    (Q, Q, t(B, Hq, T + 1, dtype=torch.float32), None),
    (Q, Q, LSE, (t(B, Hq, T, D), t(B, Hkv, T - 1, D), V)),
    (Q, Q, LSE, (t(B, Hq - 1, T, D), K, V)),
    (Q, Q, LSE, (Q, K, t(B, Hkv, T, D, dtype=torch.float32))),
])
def test_bwd_operands(o, dout, lse, grads):
    with pytest.raises(ValueError, match=SHAPE_ERR):
        fa.bwd(Q, K, V, o, dout, lse, grads=grads)


@pytest.mark.parametrize("call", [
    lambda: fa.fwd(Q, K, V, out=t(B, Hq, T, D, dtype=torch.float16)),
    lambda: fa.fwd(Q, K, V, out_dtype=torch.float16),
    lambda: fa.fwd(Q, K, V, out=t(B, Hq, T, D), out_dtype=torch.float32),
    lambda: fa.fwd(Q.float(), K.float(), V.float(), out_dtype=torch.bfloat16),
    lambda: fa.bwd(Q.float(), K.float(), V.float(), Q, Q.float(), LSE),
    lambda: fa.bwd_dkdv(Q, K, V, Q, LSE, LSE, out_dtype=torch.float16),
    lambda: fa.bwd_dq(Q.float(), K.float(), V.float(), Q.float(), LSE, LSE, out_dtype=torch.bfloat16),
    lambda: fa.bwd_preprocess(Q, Q.float()),
])
def test_result_dtype_choices(call):
    """Results take the inputs' dtype, or float32 for bfloat16 inputs
    (FA_BF16_F32OUT); any other choice is a TypeError before the library."""
    with pytest.raises(TypeError):
        call()


def test_float32_results_of_bf16_inputs_pass_the_checks():
    """float32 O, gradients and preallocated results of bfloat16 inputs pass
    the dtype and shape checks and stop only at the device check (CPU
    tensors here)."""
    f = lambda *s: t(*s, dtype=torch.float32)  # noqa: E731
    for call in (lambda: fa.fwd(Q, K, V, out_dtype=torch.float32),
                 lambda: fa.fwd(Q, K, V, out=f(B, Hq, T, D)),
                 lambda: fa.bwd(Q, K, V, f(B, Hq, T, D), Q, LSE),
                 lambda: fa.bwd(Q, K, V, f(B, Hq, T, D), Q, LSE,
                                grads=(f(B, Hq, T, D), f(B, Hkv, T, D), f(B, Hkv, T, D))),
                 lambda: fa.bwd_preprocess(f(B, Hq, T, D), Q),
                 lambda: fa.bwd_dkdv(Q, K, V, Q, LSE, LSE, out_dtype=torch.float32),
                 lambda: fa.bwd_dq(Q, K, V, Q, LSE, LSE, dq=f(B, Hq, T, D))):
        with pytest.raises(ValueError, match="same GPU"):
            call()
    with pytest.raises(ValueError, match=SHAPE_ERR):  # grads must take o's dtype
        fa.bwd(Q, K, V, f(B, Hq, T, D), Q, LSE, grads=(Q, K, V))


def test_stage_operands():
    with pytest.raises(ValueError, match=SHAPE_ERR):
        fa.bwd_preprocess(Q, t(B, Hq, T - 1, D))
    with pytest.raises(ValueError, match=SHAPE_ERR):
        fa.bwd_preprocess(Q, Q, delta=t(B, Hq, T))
    with pytest.raises(ValueError, match=SHAPE_ERR):
        fa.bwd_dkdv(Q, K, V, Q, LSE, t(B, Hq, T - 1, dtype=torch.float32))
    with pytest.raises(ValueError, match=SHAPE_ERR):
        fa.bwd_dkdv(Q, K, V, Q, LSE, LSE, dk=t(B, Hkv, T - 1, D))
    with pytest.raises(ValueError, match=SHAPE_ERR):
        fa.bwd_dq(Q, K, V, Q, t(B, Hq, T), LSE)
    with pytest.raises(ValueError, match=SHAPE_ERR):
        fa.bwd_dq(Q, K, V, Q, LSE, LSE, dq=t(B, Hq, T, D - 1))
    with pytest.raises(ValueError, match=SHAPE_ERR):
        fa.bwd_dq_delta(Q, K, V, t(B, Hq, T - 2, D), Q, LSE)
    with pytest.raises(ValueError, match=SHAPE_ERR):
        fa.bwd_dq_delta(Q, K, V, Q, Q, LSE, delta=t(B, Hq - 1, T, dtype=torch.float32))


def test_fp8_outputs():
    q8 = torch.zeros(B, Hq, T, D, dtype=torch.float8_e4m3fn)
    k8 = torch.zeros(B, Hkv, T, D, dtype=torch.float8_e4m3fn)
    with pytest.raises(ValueError, match=SHAPE_ERR):
        fa.fwd_fp8(q8, k8, k8, 1.0, 1.0, 1.0, out=t(B, Hq, T - 1, D))
    with pytest.raises(ValueError, match=SHAPE_ERR):
        fa.fwd_fp8(q8, k8, k8, 1.0, 1.0, 1.0, lse=t(B, Hq, T))
