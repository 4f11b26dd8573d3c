"""Helpers shared by the GPU tests: device inputs, metrics, tolerances."""
import sys

import numpy as np
import torch

# Tolerances.  bf16 inputs: max-abs <= 1e-2 and relative L2 <= 5e-3 on O and
# the gradients; fp32 inputs: max-abs <= 1e-5, absolute.  The outputs of the
# bf16 path are bf16 numbers, which are 2^-5 apart between 4 and 8: rounding a
# value of that size can alone move it by more than 1e-2.  The bf16 max-abs
# bound is therefore read as |got - ref| <= tol * max(1, |ref|): absolute for
# values up to 1, relative above.
# lse (not fixed by the target): 1e-3 for bf16 inputs, 1e-5 for fp32 (scores
# of exactly-representable products accumulate in fp32 on both paths).
#
# With bf16 inputs the method itself rounds: P and dS enter the matrix
# products as bf16 ("L'attention fusionnée", «Sur les Tensor Cores»), the
# backward forms Delta from the stored bf16 O («La passe arrière»), and O is
# stored in bf16.  On shapes past the benchmark workloads (large scales, rows
# whose terms are large and of both signs) those roundings alone can exceed
# the target.  The tests then also compute `emul`, the method's result with
# exactly those roundings and otherwise exact arithmetic (the lazy-reference
# forward of tests/lazy_model.py with bf16 weights; the backward of
# tests/bf16_emulation.py), and an element passes if it meets the max-abs
# target against the oracle or against emul; the whole tensor passes the
# rel-L2 target against the oracle, or, where emul itself is past it, against
# emul.
BF16_MAX_ABS = 1e-2
BF16_REL_L2 = 5e-3
FP32_MAX_ABS = 1e-5
LSE_TOL = {torch.bfloat16: 1e-3, torch.float32: 1e-5}


def say(msg: str):
    """Name the case before a GPU step, flushed, so a fault can be traced."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(inputs: dict) -> dict:
    return {k: v.cuda() for k, v in inputs.items()}


def f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def metrics(got: np.ndarray, ref: np.ndarray):
    """(max over elements of |err| / max(1, |ref|), relative L2 error)."""
    err = got - ref
    max_abs = float(np.max(np.abs(err) / np.maximum(1.0, np.abs(ref)))) if err.size else 0.0
    den = float(np.linalg.norm(ref.ravel()))
    rel_l2 = float(np.linalg.norm(err.ravel()) / den) if den > 0 else float(np.linalg.norm(err.ravel()))
    return max_abs, rel_l2


def assert_close(name: str, got, ref, dtype, emul=None):
    """Check got against the oracle's ref at the target tolerance; for bf16
    with `emul` (the method's bf16 roundings in otherwise exact arithmetic),
    as stated above.  emul is an array of ref's shape, or a function that
    takes row indices (an int array [n, ref.ndim - 1]) and returns those rows
    ([n, ref.shape[-1]]), called only for rows that need it."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    max_abs, rel_l2 = metrics(got, ref)
    if dtype == torch.float32:
        abs_err = float(np.max(np.abs(got - ref))) if got.size else 0.0
        assert abs_err <= FP32_MAX_ABS, f"{name}: max-abs {abs_err:.3e} > {FP32_MAX_ABS}"
        return abs_err, rel_l2
    if emul is None or (max_abs <= BF16_MAX_ABS and rel_l2 <= BF16_REL_L2):
        assert rel_l2 <= BF16_REL_L2, f"{name}: rel-L2 {rel_l2:.3e} > {BF16_REL_L2}"
        assert max_abs <= BF16_MAX_ABS, f"{name}: max-abs {max_abs:.3e} > {BF16_MAX_ABS}"
        return max_abs, rel_l2
    scale = np.maximum(1.0, np.abs(ref))
    bad = np.abs(got - ref) / scale > BF16_MAX_ABS
    if rel_l2 > BF16_REL_L2:
        bad[...] = True  # the whole tensor is compared with the emulation
    rows = np.argwhere(bad.any(axis=-1))
    if callable(emul):
        em_rows = np.asarray(emul(rows), np.float64)
    else:
        em_rows = np.asarray(emul, np.float64)[tuple(rows.T)]
    sel = tuple(rows.T)
    g, r, sc = got[sel], ref[sel], scale[sel]
    err = np.where(bad[sel], np.minimum(np.abs(g - r), np.abs(g - em_rows)) / sc, 0.0)
    worst = float(np.max(err)) if err.size else 0.0
    print(f"[gpu] {name}: {int(bad.sum())} elements past max-abs against the oracle "
          f"(worst {max_abs:.3e}); against the emulation {worst:.3e}", flush=True)
    assert worst <= BF16_MAX_ABS, f"{name}: max-abs {worst:.3e} against oracle and emulation"
    if rel_l2 > BF16_REL_L2:  # rows = every row
        den = float(np.linalg.norm(ref.ravel()))
        predicted = float(np.linalg.norm((em_rows - r).ravel())) / den
        against = float(np.linalg.norm((g - em_rows).ravel())) / den
        print(f"[gpu] {name}: rel-L2 {rel_l2:.3e}; the bf16 roundings alone give {predicted:.3e}, "
              f"against them {against:.3e}", flush=True)
        assert predicted > BF16_REL_L2, f"{name}: rel-L2 {rel_l2:.3e} > {BF16_REL_L2}"
        assert against <= BF16_REL_L2, f"{name}: rel-L2 {against:.3e} against the emulation"
    return max_abs, rel_l2


def assert_lse_close(got, ref, dtype):
    err = float(np.max(np.abs(np.asarray(got, np.float64) - ref))) if np.size(ref) else 0.0
    assert err <= LSE_TOL[dtype], f"lse: max-abs {err:.3e} > {LSE_TOL[dtype]}"
    return err


class Emulation:
    """The method's result with its bf16 roundings and otherwise exact
    arithmetic, for one problem (fp64 inputs x: q, k, v, dout [B,H,T,D]):
      * O: the lazy-reference forward of tests/lazy_model.py with its weights
        rounded to bf16 for P V, then O rounded to bf16 (S chunks per query
        block as the split forward cuts them);
      * dQ, dK, dV: the backward of tests/bf16_emulation.py, with P from the
        oracle's lse and Delta from that emulated O (so that Delta follows
        the stored O that the kernels' backward reads).
    Rows are computed on demand; the emulated O of every row is computed once
    when first needed."""

    def __init__(self, x: dict, lse_ref, scale, causal, q_offset=None, S=1):
        """lse_ref: the oracle's lse of every row, or None to have the oracle
        compute it when first needed.  The query blocks are those the library
        picks for these shapes (lazy_model.block_rows)."""
        from tests import lazy_model as lm

        self.x = {n: np.asarray(a, np.float64) for n, a in x.items()}
        q, k = self.x["q"], self.x["k"]
        self.block = lm.block_rows(q.shape[0], q.shape[1], q.shape[2], q.shape[3])
        self.G = q.shape[1] // k.shape[1]
        self.off = k.shape[2] - q.shape[2] if q_offset is None else q_offset
        self._lse = None if lse_ref is None else np.asarray(lse_ref, np.float64)
        self.scale, self.causal, self.S = scale, causal, S
        self._o = None

    @property
    def lse(self) -> np.ndarray:
        if self._lse is None:
            import oracle

            self._lse = oracle.fwd(self.x["q"], self.x["k"], self.x["v"], self.scale, self.causal,
                                   q_offset=self.off)[1]
        return self._lse

    def o(self) -> np.ndarray:
        from tests import bf16_emulation as em
        from tests import lazy_model as lm

        if self._o is None:
            q, k, v = self.x["q"], self.x["k"], self.x["v"]
            if self.S == 1 and q.shape[2] * k.shape[2] > 1 << 22:  # large: all rows at once
                o = np.zeros(q.shape)
                for b in range(q.shape[0]):
                    for h in range(q.shape[1]):
                        o[b, h] = lm.forward_head_all_rows(q[b, h], k[b, h // self.G],
                                                           v[b, h // self.G], self.scale,
                                                           self.causal,
                                                           self.off if self.causal else 0,
                                                           round_p=em.bf16_torch)[0]
            else:
                o, _ = lm.forward(q, k, v, self.scale, self.causal, self.off, S=self.S,
                                  round_p=em.bf16, block=self.block)
            self._o = em.bf16(o)
        return self._o

    def o_rows(self, idx) -> np.ndarray:
        return self.o()[tuple(np.asarray(idx).T)]

    def dq_rows(self, idx) -> np.ndarray:
        """dq rows for (b, h, i) row indices."""
        from tests import bf16_emulation as em

        q, k, v, do = (self.x[n] for n in ("q", "k", "v", "dout"))
        o = self.o()
        out = np.zeros((len(idx), q.shape[-1]))
        for n, (b, h, i) in enumerate(np.asarray(idx).reshape(-1, 3)):
            hk = h // self.G
            out[n] = em.dq_rows(q[b, h], k[b, hk], v[b, hk], do[b, h], o[b, h], self.lse[b, h],
                                self.scale, self.causal, self.off, [i])[0]
        return out

    def dkdv_rows(self, idx):
        """(dk rows, dv rows) for (b, hk, j) key indices."""
        from tests import bf16_emulation as em

        q, k, v, do = (self.x[n] for n in ("q", "k", "v", "dout"))
        o = self.o()
        idx = np.asarray(idx).reshape(-1, 3)
        dk = np.zeros((len(idx), q.shape[-1]))
        dv = np.zeros((len(idx), q.shape[-1]))
        for n, (b, hk, j) in enumerate(idx):
            g = slice(hk * self.G, (hk + 1) * self.G)
            a, c = em.dkdv_rows(q[b, g], k[b, hk], v[b, hk], do[b, g], o[b, g], self.lse[b, g],
                                self.scale, self.causal, self.off, [j])
            dk[n], dv[n] = a[0], c[0]
        return dk, dv

    def dk_rows(self, idx):
        return self.dkdv_rows(idx)[0]

    def dv_rows(self, idx):
        return self.dkdv_rows(idx)[1]


def emulated_fwd(x: dict, scale, causal, q_offset=None, S=1):
    """The emulated bf16 O of every row (Emulation.o)."""
    return Emulation(x, None, scale, causal, q_offset, S).o()


def emulated_grads(x: dict, o_emul, lse_ref, scale, causal, q_offset=None):
    """dq, dk, dv of every row with the method's bf16 roundings (Emulation),
    with Delta from o_emul (the emulated bf16 O, emulated_fwd) and P from the
    oracle's lse."""
    from tests import bf16_emulation as em

    q, k, v, do = (np.asarray(x[n], np.float64) for n in ("q", "k", "v", "dout"))
    B, Hq, Tq, D = q.shape
    Hkv, Tk = k.shape[1], k.shape[2]
    G = Hq // Hkv
    off = Tk - Tq if q_offset is None else q_offset
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for b in range(B):
        for h in range(Hq):
            dq[b, h] = em.dq_rows(q[b, h], k[b, h // G], v[b, h // G], do[b, h], o_emul[b, h],
                                  lse_ref[b, h], scale, causal, off, range(Tq))
        for hk in range(Hkv):
            g = slice(hk * G, (hk + 1) * G)
            dk[b, hk], dv[b, hk] = em.dkdv_rows(q[b, g], k[b, hk], v[b, hk], do[b, g], o_emul[b, g],
                                                lse_ref[b, g], scale, causal, off, range(Tk))
    return dq, dk, dv


def assert_grad_close(name: str, got, ref, emul):
    """A bf16 gradient: assert_close with its emulation."""
    return assert_close(name, got, ref, torch.bfloat16, emul)
