"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host (before any HIP call)
with the documented status codes.  CPU only."""
import ctypes
import os
import re

import pytest

import exact_attention_30_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

OK, NULL, SHAPE, UNSUP, ALIGN, HIP, SCRATCH = range(7)
BF16, FP32, BF16_F32OUT = 0, 1, 2


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIB_PATH):
        pytest.fail("libfa.so is not built (run __graft_entry__.build())")
    return fa.library()


def test_library_loads_with_all_symbols_resolved():
    # RTLD_NOW: every undefined symbol (e.g. a kernel handle) fails the load
    ctypes.CDLL(fa.LIB_PATH, mode=os.RTLD_NOW | os.RTLD_LOCAL)


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert {"fa_fwd", "fa_bwd", "fa_bwd_workspace_bytes", "fa_status_string"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/fa.h but not exported"
    assert set(names) == set(fa.SIGNATURES), "binding signatures and header disagree"


def test_status_strings(lib):
    for s in range(7):
        assert lib.fa_status_string(s)
    assert lib.fa_version().decode().count(".") == 2


# a fake, 16-byte aligned address that is never dereferenced: every call below
# must return before touching it
A = 1 << 20


def fwd(lib, q=A, k=A, v=A, o=A, lse=A, B=1, Hq=2, Hkv=1, T=64, D=128, scale=0.1, causal=1,
        dt=BF16):
    return lib.fa_fwd(q, k, v, o, lse, B, Hq, Hkv, T, D, scale, causal, dt, None)


def bwd(lib, ptrs=None, B=1, Hq=2, Hkv=1, T=64, D=128, scale=0.1, causal=1, dt=BF16):
    p = ptrs or [A] * 10
    return lib.fa_bwd(*p, B, Hq, Hkv, T, D, scale, causal, dt, None)


def test_shape_errors(lib):
    assert fwd(lib, Hq=3, Hkv=2) == SHAPE
    assert fwd(lib, Hkv=0) == SHAPE
    assert fwd(lib, Hq=0) == SHAPE
    assert fwd(lib, B=-1) == SHAPE
    assert fwd(lib, T=-5) == SHAPE
    # one head beyond the 2^31-byte range of a buffer resource
    assert fwd(lib, T=(1 << 23) + 1, D=128) == SHAPE
    assert bwd(lib, Hq=5, Hkv=2) == SHAPE


def test_unsupported_errors(lib):
    assert fwd(lib, D=96, dt=FP32) == UNSUP
    assert bwd(lib, D=96, dt=FP32) == UNSUP
    assert lib.fa_bwd_preprocess(A, A, A, 1, 2, 64, 96, FP32, None) == UNSUP
    assert fwd(lib, D=32) == UNSUP
    assert fwd(lib, dt=7) == UNSUP
    assert fwd(lib, scale=0.0) == UNSUP
    assert fwd(lib, scale=-0.5) == UNSUP
    assert fwd(lib, scale=float("inf")) == UNSUP
    assert fwd(lib, scale=float("nan")) == UNSUP
    assert bwd(lib, D=80) == UNSUP


def test_shape_checked_before_unsupported_and_null(lib):
    assert fwd(lib, Hq=3, Hkv=2, D=80, q=0) == SHAPE
    assert fwd(lib, D=80, q=0) == UNSUP


def test_head_dim_96_accepted_in_bf16(lib):
    # D = 96 passes the dimension check in bf16 and stops at the null pointer
    assert fwd(lib, D=96, q=0) == NULL
    p = [A] * 10
    p[0] = 0
    assert bwd(lib, p, D=96) == NULL
    assert lib.fa_bwd_preprocess(0, A, A, 1, 2, 64, 96, BF16, None) == NULL


def test_null_errors(lib):
    for name in ("q", "k", "v", "o", "lse"):
        assert fwd(lib, **{name: 0}) == NULL
    for i in range(10):
        p = [A] * 10
        p[i] = 0
        assert bwd(lib, p) == NULL
    assert lib.fa_bwd_preprocess(0, A, A, 1, 2, 64, 128, BF16, None) == NULL
    assert lib.fa_bwd_dkdv(A, A, A, A, A, A, 0, A, 1, 2, 1, 64, 128, 0.1, 1, BF16, None) == NULL
    assert lib.fa_bwd_dq(A, A, A, A, A, A, 0, 1, 2, 1, 64, 128, 0.1, 1, BF16, None) == NULL


def test_align_errors(lib):
    assert fwd(lib, q=A + 8) == ALIGN
    assert fwd(lib, o=A + 2) == ALIGN
    assert fwd(lib, lse=A + 2) == ALIGN
    p = [A] * 10
    p[9] = A + 4  # workspace
    assert bwd(lib, p) == ALIGN


def test_empty_inputs_are_no_ops(lib):
    # nothing to do: OK without pointers and without touching the GPU
    assert fwd(lib, q=0, k=0, v=0, o=0, lse=0, T=0) == OK
    assert fwd(lib, q=0, k=0, v=0, o=0, lse=0, B=0) == OK
    assert bwd(lib, [0] * 10, T=0) == OK
    assert lib.fa_bwd_preprocess(0, 0, 0, 0, 2, 64, 128, BF16, None) == OK


def test_workspace_bytes(lib):
    assert lib.fa_bwd_workspace_bytes(1, 32, 8, 16384, 128, BF16) == 32 * 16384 * 4
    assert lib.fa_bwd_workspace_bytes(2, 3, 1, 5, 64, BF16) == 256  # rounded up
    assert lib.fa_bwd_workspace_bytes(1, 3, 2, 5, 64, BF16) == 0  # invalid shape
    assert lib.fa_bwd_workspace_bytes(1, 2, 1, 0, 64, BF16) == 0


def test_binding_rejects_bad_tensors():
    import torch

    q = torch.zeros(1, 2, 8, 64)
    with pytest.raises(ValueError):
        fa.fwd(q, q, q)  # not on a GPU
    with pytest.raises(TypeError):
        fa.fwd(q.half(), q.half(), q.half())
    with pytest.raises(ValueError):
        fa.fwd(q, torch.zeros(1, 2, 9, 32), torch.zeros(1, 2, 9, 32))  # head sizes differ


def fwd_kv(lib, q=A, k=A, v=A, o=A, lse=A, B=1, Hq=2, Hkv=1, Tq=64, Tk=100, D=128, scale=0.1,
           causal=1, off=36, dt=BF16):
    return lib.fa_fwd_kv(q, k, v, o, lse, B, Hq, Hkv, Tq, Tk, D, scale, causal, off, dt, None)


def bwd_kv(lib, ptrs=None, B=1, Hq=2, Hkv=1, Tq=64, Tk=100, D=128, scale=0.1, causal=1, off=36,
           dt=BF16):
    p = ptrs or [A] * 10
    return lib.fa_bwd_kv(*p, B, Hq, Hkv, Tq, Tk, D, scale, causal, off, dt, None)


def test_kv_shape_errors(lib):
    assert fwd_kv(lib, off=-1) == SHAPE                    # a row would see no key
    assert fwd_kv(lib, Tk=0) == SHAPE                      # query rows without keys
    assert fwd_kv(lib, Tq=-1) == SHAPE
    assert fwd_kv(lib, Tk=-3) == SHAPE
    assert fwd_kv(lib, off=(1 << 31) - 100, Tq=64) == SHAPE  # key positions overflow
    assert fwd_kv(lib, Tk=(1 << 23) + 1) == SHAPE          # one K head beyond 2^31 bytes
    assert bwd_kv(lib, off=-5) == SHAPE
    assert bwd_kv(lib, Tk=0) == SHAPE
    assert fwd_kv(lib, off=-1, D=80) == SHAPE              # shape before unsupported
    assert fwd_kv(lib, D=80) == UNSUP
    for fn in (lib.fa_bwd_dkdv_kv, lib.fa_bwd_dq_kv):
        n = 8 if fn is lib.fa_bwd_dkdv_kv else 7
        assert fn(*([A] * n), 1, 2, 1, 64, 100, 128, 0.1, 1, -2, BF16, None) == SHAPE


def test_kv_null_and_align_errors(lib):
    for name in ("q", "k", "v", "o", "lse"):
        assert fwd_kv(lib, **{name: 0}) == NULL
    assert fwd_kv(lib, k=A + 4) == ALIGN
    for i in range(10):
        p = [A] * 10
        p[i] = 0
        assert bwd_kv(lib, p) == NULL
    # without query rows only k, v, dk, dv are needed, and they are checked
    p = [0] * 10
    p[1] = p[2] = p[8] = A  # k, v, dv; dk (index 7) missing
    assert bwd_kv(lib, p, Tq=0) == NULL
    p = [A] * 10
    p[2] = A + 8
    assert bwd_kv(lib, p) == ALIGN


def test_kv_empty_inputs_are_no_ops(lib):
    assert fwd_kv(lib, q=0, k=0, v=0, o=0, lse=0, Tq=0) == OK
    assert fwd_kv(lib, q=0, k=0, v=0, o=0, lse=0, B=0) == OK
    assert bwd_kv(lib, [0] * 10, Tq=0, Tk=0) == OK
    assert bwd_kv(lib, [0] * 10, B=0) == OK


def fwd_fp8(lib, q=A, k=A, v=A, qd=1.0, kd=1.0, vd=1.0, o=A, lse=A, ws=A, B=1, Hq=2, Hkv=1, Tq=64,
            Tk=64, D=128, scale=0.1, causal=1, off=0):
    return lib.fa_fwd_fp8(q, k, v, qd, kd, vd, o, lse, ws, B, Hq, Hkv, Tq, Tk, D, scale, causal, off,
                          None)


def test_fp8_validation(lib):
    assert fwd_fp8(lib, D=96) == UNSUP
    assert fwd_fp8(lib, D=32) == UNSUP
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        assert fwd_fp8(lib, qd=bad) == UNSUP
        assert fwd_fp8(lib, kd=bad) == UNSUP
        assert fwd_fp8(lib, vd=bad) == UNSUP
    assert fwd_fp8(lib, Hq=3, Hkv=2) == SHAPE
    assert fwd_fp8(lib, off=-1) == SHAPE
    assert fwd_fp8(lib, Tk=0) == SHAPE
    for name in ("q", "k", "v", "o", "lse", "ws"):
        assert fwd_fp8(lib, **{name: 0}) == NULL
    assert fwd_fp8(lib, q=A + 8) == ALIGN
    assert fwd_fp8(lib, ws=A + 4) == ALIGN
    assert fwd_fp8(lib, lse=A + 2) == ALIGN
    # nothing to compute: no pointer needed
    assert fwd_fp8(lib, q=0, k=0, v=0, o=0, lse=0, ws=0, Tq=0) == OK
    assert lib.fa_fp8_transpose_v(A, A, 1, 2, 64, 96, None) == UNSUP
    assert lib.fa_fp8_transpose_v(A, A, -1, 2, 64, 128, None) == SHAPE
    assert lib.fa_fp8_transpose_v(0, A, 1, 2, 64, 128, None) == NULL
    assert lib.fa_fp8_transpose_v(A, A + 8, 1, 2, 64, 128, None) == ALIGN
    assert lib.fa_fp8_transpose_v(0, 0, 1, 2, 0, 128, None) == OK
    # fa_fwd_fp8_vt: validation only (a valid call would launch on fake pointers)
    assert lib.fa_fwd_fp8_vt(A, A, A, 1.0, 1.0, 1.0, A, A, 1, 2, 1, 64, 64, 96, 0.1, 1, 0,
                             None) == UNSUP
    assert lib.fa_fwd_fp8_vt(A, A, 0, 1.0, 1.0, 1.0, A, A, 1, 2, 1, 64, 64, 64, 0.1, 1, 0,
                             None) == NULL
    assert lib.fa_fwd_fp8_vt(A, A, A, 1.0, 0.0, 1.0, A, A, 1, 2, 1, 64, 64, 64, 0.1, 1, 0,
                             None) == UNSUP


def test_fp8_workspace_bytes(lib):
    assert lib.fa_fwd_fp8_workspace_bytes(1, 8, 16384, 128) == 8 * 16384 * 128
    assert lib.fa_fwd_fp8_workspace_bytes(2, 3, 70, 64) == 2 * 3 * 128 * 64
    assert lib.fa_fwd_fp8_workspace_bytes(1, 1, 70, 96) == 0
    assert lib.fa_fwd_fp8_workspace_bytes(0, 1, 70, 64) == 0


def test_dq_delta_validation(lib):
    """fa_bwd_dq_delta: bf16 only, o required and aligned (validation only: a
    valid call would launch on fake pointers)."""
    def call(q=A, k=A, v=A, o=A, do=A, lse=A, delta=A, dq=A, Hq=2, Hkv=1, Tq=64, Tk=64, D=64,
             dt=BF16):
        return lib.fa_bwd_dq_delta(q, k, v, o, do, lse, delta, dq, None, 1, Hq, Hkv, Tq, Tk, D, 0.1,
                                   1, 0, dt, None)
    assert call(dt=FP32) == UNSUP
    assert call(D=80) == UNSUP
    assert call(Hq=3, Hkv=2) == SHAPE
    assert call(o=0) == NULL
    assert call(delta=0) == NULL
    assert call(o=A + 8) == ALIGN
    # no query row: nothing to compute, no query-side pointer needed
    assert call(q=0, o=0, do=0, lse=0, delta=0, dq=0, Tq=0) == OK


def test_noalloc_scratch_size_matches_the_header():
    text = open(HEADER).read()
    m = re.search(r"#define FA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == fa.NOALLOC_SCRATCH_BYTES


def noalloc(lib, B=1, Hq=4, Hkv=1, Tq=16384, Tk=16384, D=128, scale=0.1, causal=1, off=0,
            dt=BF16):
    return lib.fa_bwd_noalloc(*[A] * 9, B, Hq, Hkv, Tq, Tk, D, scale, causal, off, dt, None)


def test_noalloc_rejects_on_the_host(lib):
    """Shape and dtype errors come first, then the scratch limit; nothing is
    enqueued (these calls never reach the HIP runtime)."""
    assert noalloc(lib, Hq=5, Hkv=2) == SHAPE
    assert noalloc(lib, D=96, dt=FP32) == UNSUP
    assert noalloc(lib, scale=0.0) == UNSUP
    # one kv group at T = 16384 (its dK/dV stage splits: 2 x 8 chunks x 8 MiB
    # of fp32 partial sums, past the 64 MiB scratch)
    need = lib.fa_bwd_kv_workspace_bytes(1, 4, 1, 16384, 16384, 128, BF16)
    assert need > fa.NOALLOC_SCRATCH_BYTES
    assert noalloc(lib) == SCRATCH
    # Delta alone: 8 x 32 x 131072 rows x 4 bytes = 128 MiB
    assert noalloc(lib, B=8, Hq=32, Hkv=8, Tq=131072, Tk=131072) == SCRATCH


def test_block_rows_table(lib):
    """fa_block_rows reports the tile table documented in fa.h (host only)."""
    from tests import lazy_model

    lib.fa_block_rows.argtypes = [ctypes.c_int] * 6
    lib.fa_block_rows.restype = ctypes.c_int
    FWD, DQ, DKDV = 0, 1, 2
    BF16, FP32 = 0, 1
    # forward: 128 rows at D = 64 below 512 blocks of 256 rows
    assert lib.fa_block_rows(FWD, 2, 8, 4096, 64, BF16) == 128   # 256 blocks
    assert lib.fa_block_rows(FWD, 2, 16, 4096, 64, BF16) == 256  # 512 blocks
    assert lib.fa_block_rows(FWD, 1, 4, 1000, 128, BF16) == 256
    assert lib.fa_block_rows(FWD, 1, 4, 1000, 96, BF16) == 256
    # dQ and dK/dV: 128 at D = 64 below 256 blocks
    assert lib.fa_block_rows(DQ, 2, 8, 512, 64, BF16) == 128
    assert lib.fa_block_rows(DQ, 2, 8, 4096, 64, BF16) == 256
    assert lib.fa_block_rows(DKDV, 2, 8, 512, 64, BF16) == 128
    assert lib.fa_block_rows(DKDV, 2, 8, 4096, 64, BF16) == 256
    for st in (FWD, DQ, DKDV):
        assert lib.fa_block_rows(st, 1, 2, 100, 64, FP32) == 128
        assert lib.fa_block_rows(st, 1, 2, 100, 80, BF16) == 0   # unsupported D
        assert lib.fa_block_rows(st, -1, 2, 100, 64, BF16) == 0  # a shape error
    assert lib.fa_block_rows(3, 1, 2, 100, 64, BF16) == 0         # no such stage
    # the test-side model of the forward follows the same table
    for B, H, T, D in ((2, 8, 4096, 64), (2, 16, 4096, 64), (1, 4, 1500, 64), (1, 4, 700, 128)):
        assert lib.fa_block_rows(FWD, B, H, T, D, BF16) == lazy_model.block_rows(B, H, T, D)


def test_atomic_backward_validation(lib):
    """fa_bwd_atomic: bf16 at D = 64 only; other sizes or types are refused on
    the host before anything is enqueued (null pointers are never touched)."""
    f = lib.fa_bwd_atomic
    f.argtypes = ([ctypes.c_void_p] * 5 + [ctypes.c_void_p] + [ctypes.c_void_p] * 4 +
                  [ctypes.c_int] * 5 + [ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_void_p])
    f.restype = ctypes.c_int
    n = [None] * 10
    UNSUP = 3
    assert f(*n, 1, 4, 2, 100, 128, 0.1, 1, 0, None) == UNSUP   # D = 128
    assert f(*n, 1, 4, 2, 100, 96, 0.1, 1, 0, None) == UNSUP    # D = 96
    assert f(*n, 1, 4, 2, 100, 64, 0.1, 1, 1, None) == UNSUP    # fp32
    assert f(*n, 0, 4, 2, 100, 64, 0.1, 1, 0, None) == 0        # empty: a no-op
    g = lib.fa_bwd_atomic_workspace_bytes
    g.argtypes = [ctypes.c_int] * 5
    g.restype = ctypes.c_size_t
    assert g(2, 8, 512, 64, 0) == 2 * 8 * 512 * 4 + 2 * 8 * 512 * 64 * 4
    assert g(2, 8, 512, 128, 0) == 0 and g(2, 8, 512, 64, 1) == 0


def test_bf16_with_float32_results(lib):
    """FA_BF16_F32OUT: the bf16 kernels' checks, tile table and workspace
    sizes; D = 96 accepted; refused by the atomic backward only."""
    assert fwd(lib, D=96, q=0, dt=BF16_F32OUT) == NULL
    p = [A] * 10
    p[0] = 0
    assert bwd(lib, p, D=96, dt=BF16_F32OUT) == NULL
    assert lib.fa_bwd_preprocess(0, A, A, 1, 2, 64, 96, BF16_F32OUT, None) == NULL
    assert fwd(lib, D=80, dt=BF16_F32OUT) == UNSUP
    assert fwd(lib, Hq=3, Hkv=2, dt=BF16_F32OUT) == SHAPE
    for args in ((1, 32, 8, 16384, 128), (2, 3, 1, 5, 64), (1, 4, 1, 2048, 96)):
        assert (lib.fa_bwd_workspace_bytes(*args, BF16_F32OUT) ==
                lib.fa_bwd_workspace_bytes(*args, BF16))
    for args in ((1, 4, 1, 2048, 2048, 128), (2, 8, 8, 512, 512, 64)):
        assert lib.fa_fwd_split_bytes(*args, BF16_F32OUT) == lib.fa_fwd_split_bytes(*args, BF16)
        assert (lib.fa_bwd_dq_split_bytes(*args, BF16_F32OUT) ==
                lib.fa_bwd_dq_split_bytes(*args, BF16))
    for stage in range(3):
        for args in ((2, 8, 4096, 64), (1, 32, 16384, 128)):
            assert (lib.fa_block_rows(stage, *args, BF16_F32OUT) ==
                    lib.fa_block_rows(stage, *args, BF16))
    f = lib.fa_bwd_atomic
    f.argtypes = ([ctypes.c_void_p] * 10 + [ctypes.c_int] * 5 +
                  [ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_void_p])
    f.restype = ctypes.c_int
    assert f(*[None] * 10, 1, 4, 2, 100, 64, 0.1, 1, BF16_F32OUT, None) == UNSUP
