"""Seeded synthetic inputs for exact attention.

This module only draws random numbers and names workload shapes; it holds none
of attention's arithmetic.  Both the oracle checks and the HIP library receive
the tensors it returns, so the two sides always see identical inputs.

Recipe: a CPU ``torch.Generator`` seeded with ``seed`` draws float32 standard
normals for q, k, v and dO, in that order; each is multiplied by
``input_scale`` (0.5 for the long non-causal workload, an exact power of two)
and then rounded to the compute dtype with round-to-nearest-even.

Workloads (layout [B, H, T, D], contiguous):
  C1  fp32, B=1, H=1,  T=128,   D=64,  causal, scale 1/8
  C2  bf16, B=2, H=8,  T=512,   D=64,  causal, scale 1/8
  C3  bf16, B=2, H=8,  T=4096,  D=64,  causal, scale 1/8 (the fp32 score tensor
      of the unfused form would be 1 GiB: "L'attention fusionnée",
      «Ce que l'attention écrit en mémoire»)
  C4  bf16, B=1, H=16, T=16384, D=64,  non-causal, scale 1/8, inputs x0.5,
      forward only (N = 16384 as in the cuTile page's memory example)
  C5  bf16, B=1, Hq=32, Hkv=8, T=16384, D=128, causal, scale 1/sqrt(128)
  C5-share  one kv group of C5 (B=1, Hq=4, Hkv=1), the part of C5 one GPU
      would own if C5 were split by kv group.
  C5-prefill  C5's heads with 4096 new query rows against 16384 keys (the
      last 4096 positions: causal offset Tk - Tq = 12288), a prefill step
      against cached keys.
  C5-d96  C5's shape with head dimension 96 (scale 1/sqrt(96)); the credited
      FLOP count uses D = 96.
  C5-fp8  C5's shape in e4m3 (forward only): q, k, v drawn as above in fp32,
      multiplied by 16 (exact) and rounded to e4m3 (RNE); each has descale
      1/16, so the real inputs are N(0,1) values on the e4m3 grid.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: torch.dtype
    B: int
    Hq: int
    Hkv: int
    T: int
    D: int
    causal: bool
    scale: float
    seed: int
    input_scale: float = 1.0
    backward: bool = True
    Tk: int = 0  # key rows; 0: the same as T (the query rows)

    @property
    def Tkv(self) -> int:
        return self.Tk or self.T

    @property
    def q_offset(self) -> int:
        """Position of query row 0 among the keys (last query on the last key)."""
        return self.Tkv - self.T

    @property
    def pairs(self) -> float:
        """(query, key) pairs of one head that the mask lets through; for
        T = Tk and causal, T^2/2 (the credited convention, not T(T+1)/2)."""
        if not self.causal:
            return float(self.T) * self.Tkv
        if self.Tkv == self.T:
            return self.T * self.T / 2.0
        # row i sees min(Tk, i + off + 1) keys (off >= 0: every row sees key 0)
        off, T, Tk = self.q_offset, self.T, self.Tkv
        assert off >= 0, "causal workloads have at least as many keys as query rows"
        full = max(0, min(T, T - (Tk - off - 1)))  # rows that see every key
        part = T - full
        return float(full) * Tk + part * (off + 1) + part * (part - 1) / 2.0

    @property
    def fwd_flop(self) -> float:
        """Credited forward FLOP: 4*B*Hq*D per visible pair (4*B*Hq*T^2*D,
        halved when causal, for one sequence)."""
        return 4.0 * self.B * self.Hq * self.D * self.pairs

    @property
    def bwd_flop(self) -> float:
        """Credited backward FLOP: 2.5x the forward."""
        return 2.5 * self.fwd_flop if self.backward else 0.0


WORKLOADS = {
    "C1": Workload("C1", torch.float32, 1, 1, 1, 128, 64, True, 1 / 8, 1000),
    "C2": Workload("C2", torch.bfloat16, 2, 8, 8, 512, 64, True, 1 / 8, 2000),
    "C3": Workload("C3", torch.bfloat16, 2, 8, 8, 4096, 64, True, 1 / 8, 3000),
    "C4": Workload("C4", torch.bfloat16, 1, 16, 16, 16384, 64, False, 1 / 8, 4000,
                   input_scale=0.5, backward=False),
    "C5": Workload("C5", torch.bfloat16, 1, 32, 8, 16384, 128, True, 1 / math.sqrt(128), 5000),
    "C5-share": Workload("C5-share", torch.bfloat16, 1, 4, 1, 16384, 128, True,
                         1 / math.sqrt(128), 5500),
    "C5-prefill": Workload("C5-prefill", torch.bfloat16, 1, 32, 8, 4096, 128, True,
                           1 / math.sqrt(128), 5700, Tk=16384),
    "C5-d96": Workload("C5-d96", torch.bfloat16, 1, 32, 8, 16384, 96, True, 1 / math.sqrt(96), 5900),
    "C5-fp8": Workload("C5-fp8", torch.float8_e4m3fn, 1, 32, 8, 16384, 128, True, 1 / math.sqrt(128),
                       6100, input_scale=16.0, backward=False),
}

FP8_AMP = 16.0  # fp8 inputs: codes = N(0,1) * FP8_AMP rounded to e4m3; descale 1 / FP8_AMP


def make_inputs(B: int, Hq: int, Hkv: int, T: int, D: int, dtype: torch.dtype, seed: int,
                input_scale: float = 1.0, with_dout: bool = True, Tk: int | None = None) -> dict:
    """Return CPU tensors q [B,Hq,T,D], k and v [B,Hkv,Tk,D] (Tk = T unless
    given) and (optionally) dout [B,Hq,T,D], drawn as described in the module
    docstring."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    Tk = T if Tk is None else Tk
    out = {}
    for name, h in (("q", Hq), ("k", Hkv), ("v", Hkv), ("dout", Hq)):
        if name == "dout" and not with_dout:
            break
        rows = T if name in ("q", "dout") else Tk
        x = torch.randn((B, h, rows, D), generator=g, dtype=torch.float32)
        if input_scale != 1.0:
            x = x * input_scale
        out[name] = x.to(dtype).contiguous()
    return out


def make_fp8_inputs(B: int, Hq: int, Hkv: int, T: int, D: int, seed: int, Tk: int | None = None,
                    amp: float = FP8_AMP) -> tuple[dict, float]:
    """e4m3 codes of q [B,Hq,T,D], k and v [B,Hkv,Tk,D] (CPU, torch.float8_e4m3fn)
    and their common descale 1/amp: the fp32 draws of make_inputs times amp (a
    power of two), rounded to nearest even."""
    x = make_inputs(B, Hq, Hkv, T, D, torch.float32, seed, with_dout=False, Tk=Tk)
    return {n: (t * amp).to(torch.float8_e4m3fn) for n, t in x.items()}, 1.0 / amp


def workload_inputs(w: Workload) -> dict:
    if w.dtype == torch.float8_e4m3fn:
        return make_fp8_inputs(w.B, w.Hq, w.Hkv, w.T, w.D, w.seed, Tk=w.Tkv, amp=w.input_scale)[0]
    return make_inputs(w.B, w.Hq, w.Hkv, w.T, w.D, w.dtype, w.seed, w.input_scale, w.backward,
                       Tk=w.Tkv)
