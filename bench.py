"""Benchmark: causal attention forward + backward on one MI355X.

One step = the whole hot path once: fa_fwd, then the three stages of fa_bwd
(Delta preprocess, dK/dV, dQ), on seeded synthetic inputs already resident in
HBM.  W untimed warm-up steps, then K timed steps bracketed by device
synchronisation, with nothing recorded between their kernels (--graph: each
the replay of one captured step, a HIP graph).  K more steps with HIP events
recorded on the launch stream between the kernels give the per-kernel
averages.

Throughput is credited FLOP / time with forward FLOP = 4*B*Hq*T^2*D (halved
when causal) and backward = 2.5x forward ("FlashAttention: l'attenzione che non
spreca memoria", «L'idea: lavorare a tessere»: 4N^2d forward, 10N^2d backward
with recomputation).

The roofline entry is for the slowest kernel, against the bf16 dense MFMA
peak; its "achieved" counts the GEMM FLOP that kernel's own math needs (see
KERNEL_GEMMS).  The CPU baseline times the fp64 oracle on a bounded sample of
the same workload (whole kv groups, or a causal prefix of one head).

Prints one JSON line.  Usage: python bench.py [--steps K] [--warmup W]
[--workload C5] [--no-cpu-baseline]; python bench.py --gemm-reference times a
large bf16 library GEMM on random data, a reference for the sustained
matrix-core rate of the chip.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_FP32_TFLOPS = 157.3    # MI355X dense fp32 MFMA, published
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA, published
METRIC = "causal attention fwd+bwd TFLOP/s on 1 MI355X; % of bf16 MFMA peak"

# GEMMs each kernel performs, in units of one T x T x D product over the
# visible (causal: lower-triangular) score entries: 2 FLOP per multiply-add.
#   fwd : S = Q K^T, O = P V                      -> 2
#   dkdv: S, dP = dO V^T, dV = P^T dO, dK = dS^T Q -> 4
#   dq  : S, dP, dQ = dS K                        -> 3
KERNEL_GEMMS = {"fwd": 2, "dkdv": 4, "dq": 3}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default="C5")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--atomic-bwd", action="store_true",
                   help="time fa_bwd against fa_bwd_atomic (dQ by atomic adds) on a D = 64 "
                        "workload; prints its own JSON line")
    p.add_argument("--graph", action="store_true",
                   help="time replays of a captured HIP graph of one step instead of eager steps")
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="target duration of the oracle sample")
    p.add_argument("--gemm-reference", action="store_true",
                   help="only time a large bf16 library GEMM (torch.matmul, random N(0,1) data) as a "
                        "reference for the matrix-core throughput reachable on this chip, and exit")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                   help="only run 5 plain device copies of BYTES bytes (a known-size reference "
                        "for the HBM byte counters) and exit")
    return p.parse_args()


def calibrate_copy(nbytes: int):
    """Five device-to-device copies of nbytes: each reads and writes nbytes, so
    FETCH_SIZE / WRITE_SIZE of these dispatches calibrate the counters."""
    import torch

    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibration_copy_bytes": nbytes, "copies": 5}), flush=True)


def gemm_reference():
    """Time torch.matmul (the vendor GEMM library) on 8192^3 bf16 products of
    random N(0,1) data: the sustained matrix-core rate a tuned library reaches
    here, with data-dependent power and clock included."""
    import torch

    n = 8192
    g = torch.Generator(device="cuda").manual_seed(7)
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=g)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=g)
    c = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)
    for _ in range(5):
        torch.matmul(a, b, out=c)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 50
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    print(json.dumps({"gemm_reference": f"torch.matmul bf16 {n}x{n}x{n}, random N(0,1)",
                      "ms": round(ms, 4), "tflops": round(tf, 1),
                      "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)}), flush=True)


def atomic_bwd_compare(args):
    """The two backward formulations of "L'attention fusionnée", «La passe
    arrière», on one D = 64 workload: fa_bwd (a dQ kernel that recomputes S and
    dP, then dK/dV) against fa_bwd_atomic (one dK/dV kernel that adds dQ with
    atomic adds), alternated over K rounds on the same inputs; prints one JSON
    line with each one's median time and credited TFLOP/s."""
    import statistics

    import torch

    import exact_attention_30_amd as fa
    from workloads import WORKLOADS, workload_inputs

    w = WORKLOADS[args.workload]
    if w.D != 64 or w.dtype != torch.bfloat16 or w.Tkv != w.T or not w.backward:
        sys.exit(f"bench.py --atomic-bwd: {w.name} is not a bf16 D = 64 fwd+bwd workload with "
                 "equal lengths (fa_bwd_atomic's scope)")
    d = {k: v.cuda() for k, v in workload_inputs(w).items()}
    q, k, v, do = d["q"], d["k"], d["v"], d["dout"]
    o, lse = fa.fwd(q, k, v, scale=w.scale, causal=w.causal)
    ws2 = torch.empty(max(fa.bwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.T, w.D), 16),
                      dtype=torch.uint8, device="cuda")
    wsa = torch.empty(max(fa.bwd_atomic_workspace_bytes(w.B, w.Hq, w.T, w.D), 16),
                      dtype=torch.uint8, device="cuda")
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v))
    runs = {
        "two_kernel": lambda: fa.bwd(q, k, v, o, do, lse, scale=w.scale, causal=w.causal,
                                     workspace=ws2, grads=grads),
        "atomic": lambda: fa.bwd_atomic(q, k, v, o, do, lse, scale=w.scale, causal=w.causal,
                                        workspace=wsa, grads=grads),
    }
    for f in runs.values():
        for _ in range(max(args.warmup, 1)):
            f()
    torch.cuda.synchronize()
    times = {n: [] for n in runs}
    for _ in range(args.steps):
        for n, f in runs.items():
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            f()
            e1.record()
            torch.cuda.synchronize()
            times[n].append(e0.elapsed_time(e1))
    out = {"atomic_bwd_compare": describe(w), "steps": args.steps}
    for n, t in times.items():
        ms = statistics.median(t)
        out[n] = {"ms": round(ms, 4), "credited_tflops": round(w.bwd_flop / (ms * 1e-3) / 1e12, 2)}
    print(json.dumps(out), flush=True)


def gemm_flop(w, n_gemm):
    """FLOP of n_gemm Tq x Tk x D products over the visible score entries."""
    return 2.0 * n_gemm * w.B * w.Hq * w.pairs * w.D


def source_hash(kernel_file: str) -> str:
    h = hashlib.sha256()
    for f in ("fa_device.hpp", "fa_pipe.hpp", kernel_file):
        with open(os.path.join(ROOT, "exact_attention_30_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_for(kernel: str, kernel_file: str, workload: str):
    """HBM bytes per launch from the committed counter summary, if it was taken
    on the current source of that kernel; otherwise None."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    e = data.get(f"{kernel}:{workload}")
    if not e or e.get("source_hash") != source_hash(kernel_file):
        return None
    return e.get("hbm_bytes_per_launch")


def describe(w) -> str:
    rows = f"T={w.T}" if w.Tkv == w.T else f"Tq={w.T} Tk={w.Tkv} q_offset={w.q_offset}"
    return (f"{w.name}: {'causal' if w.causal else 'non-causal'} {'GQA' if w.Hq != w.Hkv else 'MHA'} "
            f"attention {'fwd+bwd' if w.backward else 'fwd'}, B={w.B} Hq={w.Hq} Hkv={w.Hkv} "
            f"{rows} D={w.D}, scale={w.scale:.6g}")


def forward_only(args, w, x, q, k, v, o, lse):
    """A forward-only workload: one step is one fa_fwd; the line reports the
    forward's credited TFLOP/s (no backward exists for it)."""
    import torch

    import exact_attention_30_amd as fa

    for _ in range(args.warmup):
        fa.fwd(q, k, v, scale=w.scale, causal=w.causal, out=o, lse=lse)
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for ev in events:
        ev[0].record()
        fa.fwd(q, k, v, scale=w.scale, causal=w.causal, out=o, lse=lse)
        ev[1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = sum(ev[0].elapsed_time(ev[1]) for ev in events) / args.steps
    ms_per_step = max(wall * 1e3 / args.steps, events[0][0].elapsed_time(events[-1][1]) / args.steps)
    bf = w.dtype == torch.bfloat16
    peak = PEAK_BF16_TFLOPS if bf else PEAK_FP32_TFLOPS
    value = w.fwd_flop / (ms_per_step * 1e-3) / 1e12
    achieved = gemm_flop(w, KERNEL_GEMMS["fwd"]) / (per * 1e-3) / 1e12
    kfile = "fa_fwd_bf16.hip" if bf else "fa_fwd.hip"
    out = {
        "metric": "attention fwd TFLOP/s on 1 MI355X; % of bf16 MFMA peak (forward-only workload)",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16" if bf else "fp32",
        "data": "synthetic (seeded N(0,1) inputs of the workload's shape)",
        "config": {"workload": describe(w), "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "T": w.T, "D": w.D,
                   "causal": w.causal, "parallelism": "single GPU",
                   **({"Tk": w.Tkv, "q_offset": w.q_offset} if w.Tkv != w.T else {})},
        "pct_of_peak": round(100 * value / peak, 2),
        "roofline": {
            "kernel": "fwd_bf16_kernel" if bf else "fwd_kernel", "bound": "mfma",
            "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4), "traffic": traffic_for("fwd", kfile, w.name),
            "avg_launch_ms": round(per, 4),
            "algorithmic_flop_per_launch": gemm_flop(w, KERNEL_GEMMS["fwd"]),
        },
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def forward_only_fp8(args, w, q, k, v, lse):
    """The e4m3 forward-only workload: one step is one fa_fwd_fp8 (the V
    transpose pre-pass and the forward); the roofline is the forward kernel
    alone (fa_fwd_fp8_vt, timed by its own events) against the dense fp8 MFMA
    peak."""
    import torch

    import exact_attention_30_amd as fa

    ds = 1.0 / w.input_scale
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=q.device)
    ws = torch.empty(max(fa.fwd_fp8_workspace_bytes(w.B, w.Hkv, w.Tkv, w.D), 16), dtype=torch.uint8,
                     device=q.device)

    def step(ev=None):
        if ev:
            ev[0].record()
        fa.fp8_transpose_v(v, ws)
        if ev:
            ev[1].record()
        fa.fwd_fp8_vt(q, k, ws, v.shape, ds, ds, ds, scale=w.scale, causal=w.causal, out=o, lse=lse)
        if ev:
            ev[2].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for ev in events:
        step(ev)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    vt_ms = sum(ev[0].elapsed_time(ev[1]) for ev in events) / args.steps
    per = sum(ev[1].elapsed_time(ev[2]) for ev in events) / args.steps
    ms_per_step = max(wall * 1e3 / args.steps, events[0][0].elapsed_time(events[-1][2]) / args.steps)
    value = w.fwd_flop / (ms_per_step * 1e-3) / 1e12
    achieved = gemm_flop(w, KERNEL_GEMMS["fwd"]) / (per * 1e-3) / 1e12
    out = {
        "metric": "attention fwd TFLOP/s on 1 MI355X; % of fp8 MFMA peak (forward-only e4m3 workload)",
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8",
        "data": "synthetic (seeded N(0,1) inputs of the workload's shape, x16 and rounded to e4m3, "
                "descale 1/16)",
        "config": {"workload": describe(w), "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "T": w.T, "D": w.D,
                   "causal": w.causal, "parallelism": "single GPU"},
        "pct_of_peak": round(100 * value / PEAK_FP8_TFLOPS, 2),
        "breakdown": {"transpose_v_ms": round(vt_ms, 4), "fwd_ms": round(per, 4)},
        "roofline": {
            "kernel": "fwd_fp8_kernel", "bound": "mfma", "achieved": round(achieved, 2),
            "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP8_TFLOPS, 4),
            "traffic": traffic_for("fwd_fp8", "fa_fwd_fp8.hip", w.name),
            "avg_launch_ms": round(per, 4),
            "algorithmic_flop_per_launch": gemm_flop(w, KERNEL_GEMMS["fwd"]),
        },
        "cpu_baseline": None,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(w, x, target_s: float):
    """Time the oracle's fwd + bwd on a bounded sample of the workload, sized
    to take about target_s seconds: whole kv groups (all their query heads,
    every position) when one group takes at most twice that, else a causal
    prefix of query head 0 and its kv head.  Returns (record, outputs): for whole kv
    groups, outputs holds the oracle's O, lse, dQ, dK, dV of groups
    0 .. n-1 of batch 0 (for the parity errors), else None."""
    import oracle

    orc = oracle.default()
    G = w.Hq // w.Hkv
    outputs = None

    def run(ngroups, tp):
        nonlocal outputs
        sl = (slice(0, 1), slice(0, ngroups * G), slice(0, tp))
        kl = (slice(0, 1), slice(0, ngroups), slice(0, tp))
        q, do = x["q"][sl].double().numpy(), x["dout"][sl].double().numpy()
        k, v = x["k"][kl].double().numpy(), x["v"][kl].double().numpy()
        t0 = time.perf_counter()
        o, lse = orc.fwd(q, k, v, w.scale, w.causal)
        dq, dk, dv = orc.bwd(q, k, v, do, w.scale, w.causal)
        elapsed = time.perf_counter() - t0
        outputs = {"ngroups": ngroups, "o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}
        return elapsed

    # calibrate on one query head (one kv head, G = 1 slice) and a short prefix
    def run_head(tp):
        q, do = x["q"][:1, :1, :tp].double().numpy(), x["dout"][:1, :1, :tp].double().numpy()
        k, v = x["k"][:1, :1, :tp].double().numpy(), x["v"][:1, :1, :tp].double().numpy()
        t0 = time.perf_counter()
        orc.fwd(q, k, v, w.scale, w.causal)
        orc.bwd(q, k, v, do, w.scale, w.causal)
        return time.perf_counter() - t0

    run_head(min(256, w.T))  # the first call starts the oracle's thread pool
    cal = min(4096, w.T)
    t_cal = run_head(cal)
    t_head = t_cal * (w.T / cal) ** 2  # work grows as T^2
    # whole kv groups (the parity slice) while one fits in twice the target
    if t_head * G <= 2 * target_s:
        ngroups = max(1, min(w.B * w.Hkv, int(target_s / (t_head * G))))
        ngroups = min(ngroups, w.Hkv)
        tp, nheads = w.T, ngroups * G
        elapsed = run(ngroups, tp)
        what = (f"all {tp} positions of query heads 0-{nheads - 1} and kv heads 0-{ngroups - 1} "
                f"of {w.name}")
    else:
        tp = int(cal * math.sqrt(max(target_s, 0.1) / max(t_cal, 1e-3)))
        tp = max(cal, min(w.T, tp // 128 * 128))
        nheads = 1
        elapsed = run_head(tp)
        what = f"the first {tp} positions of query head 0 and its kv head of {w.name}"
    credited = 3.5 * 4.0 * nheads * tp * tp * w.D * (0.5 if w.causal else 1.0)  # fwd + 2.5x fwd
    return {
        "value": credited / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": orc.threads(),
        "kind": "oracle",
        "sample": f"fp64 oracle fwd+bwd on {what} ({elapsed:.1f} s)",
        "seconds": round(elapsed, 2),
    }, (outputs if tp == w.T else None)


def parity_errors(w, gpu: dict, ref: dict) -> dict:
    """Errors of the GPU outputs of the timed steps against the oracle's on
    every element of kv groups 0 .. n-1 of batch 0: max-abs (relative above
    |ref| = 1, as the bf16 target reads it; absolute for fp32) and rel-L2 for
    O, dQ, dK, dV, max-abs for lse, with the target tolerance."""
    import numpy as np
    import torch

    n = ref["ngroups"]
    G = w.Hq // w.Hkv
    bf = w.dtype == torch.bfloat16
    out = {"slice": f"batch 0, kv heads 0-{n - 1}, query heads 0-{n * G - 1}, every position",
           "tolerance": ("max-abs <= 1e-2 (relative above |ref| = 1) and rel-L2 <= 5e-3; "
                         "lse max-abs <= 1e-3" if bf else "max-abs <= 1e-5")}
    ok = True
    for name, heads in (("o", n * G), ("lse", n * G), ("dq", n * G), ("dk", n), ("dv", n)):
        got = gpu[name][:1, :heads].double().cpu().numpy()
        r = ref[name]
        err = got - r
        if name == "lse":
            m = float(np.max(np.abs(err)))
            out[name] = {"max_abs": m}
            ok &= m <= (1e-3 if bf else 1e-5)
            continue
        m = float(np.max(np.abs(err) / (np.maximum(1.0, np.abs(r)) if bf else 1.0)))
        rel = float(np.linalg.norm(err) / np.linalg.norm(r))
        out[name] = {"max_abs": m, "rel_l2": rel}
        ok &= (m <= 1e-2 and rel <= 5e-3) if bf else m <= 1e-5
    out["pass"] = bool(ok)
    return out


def float32_results_errors(w, q, k, v, do, fpart, ref: dict) -> dict:
    """One more forward and backward of the same inputs with float32 results
    (FA_BF16_F32OUT: the same kernels, O and the gradients stored without the
    final rounding to bf16), after the timed region, against the oracle's
    outputs on the same kv groups: the stated target read literally, max |err|
    absolute and rel-L2."""
    import numpy as np
    import torch

    import exact_attention_30_amd as fa

    o, lse = fa.fwd(q, k, v, scale=w.scale, causal=w.causal, partial=fpart, out_dtype=torch.float32)
    dq, dk, dv = fa.bwd(q, k, v, o, do, lse, scale=w.scale, causal=w.causal)
    torch.cuda.synchronize()
    n = ref["ngroups"]
    G = w.Hq // w.Hkv
    out = {"slice": f"batch 0, kv heads 0-{n - 1}, query heads 0-{n * G - 1}, every position",
           "tolerance": "max |err| <= 1e-2 absolute and rel-L2 <= 5e-3; lse max-abs <= 1e-3"}
    ok = True
    for name, t, heads in (("o", o, n * G), ("lse", lse, n * G), ("dq", dq, n * G), ("dk", dk, n),
                           ("dv", dv, n)):
        err = t[:1, :heads].double().cpu().numpy() - ref[name]
        m = float(np.max(np.abs(err)))
        if name == "lse":
            out[name] = {"max_abs": m}
            ok &= m <= 1e-3
            continue
        rel = float(np.linalg.norm(err) / np.linalg.norm(ref[name]))
        out[name] = {"max_abs": m, "rel_l2": rel, "elements_past_1e-2": int(np.sum(np.abs(err) > 1e-2)),
                     "elements": int(err.size)}
        ok &= m <= 1e-2 and rel <= 5e-3
    out["pass"] = bool(ok)
    return out


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    if args.atomic_bwd:
        atomic_bwd_compare(args)
        return
    if args.gemm_reference:
        gemm_reference()
        return
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU only (asked for --gpus {args.gpus}); "
              "sharding by kv group across GPUs is not built.", file=sys.stderr)
        sys.exit(2)

    import torch

    import exact_attention_30_amd as fa
    from workloads import WORKLOADS, workload_inputs

    w = WORKLOADS[args.workload]
    print(f"[bench] workload {w.name}: B={w.B} Hq={w.Hq} Hkv={w.Hkv} T={w.T} D={w.D} "
          f"causal={w.causal} {w.dtype}", file=sys.stderr, flush=True)
    x = workload_inputs(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    d = {k: v.to(dev) for k, v in x.items()}
    q, k, v, do = d["q"], d["k"], d["v"], d.get("dout")
    if w.dtype == torch.float8_e4m3fn:
        forward_only_fp8(args, w, q, k, v,
                         torch.empty(w.B, w.Hq, w.T, dtype=torch.float32, device=dev))
        return
    o = torch.empty_like(q)
    lse = torch.empty(w.B, w.Hq, w.T, dtype=torch.float32, device=dev)
    delta = torch.empty(w.B, w.Hq, w.T, dtype=torch.float32, device=dev)
    if not w.backward:
        forward_only(args, w, x, q, k, v, o, lse)
        return
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    # scratch of the dK/dV stage when the shapes split its query side (as in fa_bwd)
    part = torch.empty(max(fa.dkdv_split_bytes(w.B, w.Hq, w.Hkv, w.T, w.Tkv, w.D, w.dtype),
                           fa.dq_split_bytes(w.B, w.Hq, w.Hkv, w.T, w.Tkv, w.D, w.dtype), 16),
                       dtype=torch.uint8, device=dev)

    fpart = torch.empty(max(fa.fwd_split_bytes(w.B, w.Hq, w.Hkv, w.T, w.Tkv, w.D, w.dtype), 16),
                        dtype=torch.uint8, device=dev)

    # bf16: the backward as fa_bwd runs it (the dQ kernel forms Delta, then
    # dK/dV); fp32: preprocess, dK/dV, dQ
    fused = w.dtype == torch.bfloat16
    names = ["fwd", "dq", "dkdv"] if fused else ["fwd", "pre", "dkdv", "dq"]

    def step(ev=None):
        if ev:
            ev[0].record()
        fa.fwd(q, k, v, scale=w.scale, causal=w.causal, out=o, lse=lse, partial=fpart)
        if ev:
            ev[1].record()
        if fused:
            fa.bwd_dq_delta(q, k, v, o, do, lse, scale=w.scale, causal=w.causal, dq=dq, delta=delta,
                            partial=part)
            if ev:
                ev[2].record()
            fa.bwd_dkdv(q, k, v, do, lse, delta, scale=w.scale, causal=w.causal, dk=dk, dv=dv,
                        partial=part)
            if ev:
                ev[3].record()
            return
        fa.bwd_preprocess(o, do, delta)
        if ev:
            ev[2].record()
        fa.bwd_dkdv(q, k, v, do, lse, delta, scale=w.scale, causal=w.causal, dk=dk, dv=dv,
                    partial=part)
        if ev:
            ev[3].record()
        fa.bwd_dq(q, k, v, do, lse, delta, scale=w.scale, causal=w.causal, dq=dq, partial=part)
        if ev:
            ev[4].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] warm-up done ({args.warmup} steps)", file=sys.stderr, flush=True)

    # The timed region: K steps with nothing between their kernels (events
    # between kernels leave the GPU idle for a few microseconds each), eager,
    # or with --graph each the replay of one captured step (a HIP graph: the
    # kernels of a step go to the GPU in one launch).
    run, launch = step, "eager"
    if args.graph:
        try:
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                step()
            run, launch = graph.replay, "graph"
        except RuntimeError as e:
            print(f"[bench] graph capture failed ({e}); timing eager steps", file=sys.stderr,
                  flush=True)
    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_span = e0.elapsed_time(e1) / args.steps
    ms_per_step = max(wall * 1e3 / args.steps, gpu_span)
    print(f"[bench] timed {args.steps} steps ({launch}) in {wall:.3f} s", file=sys.stderr,
          flush=True)

    # Kernel durations: K more eager steps with events between the kernels
    nev = len(names) + 1
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    per = {n: 0.0 for n in names}
    for ev in events:
        for i, n in enumerate(names):
            per[n] += ev[i].elapsed_time(ev[i + 1])
    per = {n: t / args.steps for n, t in per.items()}
    bwd_ms = sum(per[n] for n in names if n != "fwd")
    if fused:
        # the preprocess kernel on its own, after the timed region (its HBM rate)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        pre_delta = torch.empty_like(delta)
        fa.bwd_preprocess(o, do, pre_delta)
        e0.record()
        for _ in range(20):
            fa.bwd_preprocess(o, do, pre_delta)
        e1.record()
        torch.cuda.synchronize()
        per["pre"] = e0.elapsed_time(e1) / 20

    fwd_flop, bwd_flop = w.fwd_flop, w.bwd_flop
    value = (fwd_flop + bwd_flop) / (ms_per_step * 1e-3) / 1e12
    fwd_tflops = fwd_flop / (per["fwd"] * 1e-3) / 1e12
    bwd_tflops = bwd_flop / (bwd_ms * 1e-3) / 1e12
    pre_bytes = 2 * w.B * w.Hq * w.T * w.D * q.element_size() + 4 * w.B * w.Hq * w.T

    dom = max(("fwd", "dkdv", "dq"), key=lambda n: per[n])
    bf = w.dtype == torch.bfloat16
    kfile = {"fwd": "fa_fwd_bf16.hip" if bf else "fa_fwd.hip",
             "dkdv": "fa_bwd_bf16.hip" if bf else "fa_bwd.hip",
             "dq": "fa_bwd_bf16.hip" if bf else "fa_bwd.hip"}[dom]
    achieved = gemm_flop(w, KERNEL_GEMMS[dom]) / (per[dom] * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == torch.bfloat16 else PEAK_FP32_TFLOPS
    roofline = {
        "kernel": ({"fwd": "fwd_bf16_kernel", "dkdv": "dkdv_bf16_kernel", "dq": "dq_bf16_kernel"} if bf else
                   {"fwd": "fwd_kernel", "dkdv": "bwd_dkdv_kernel", "dq": "bwd_dq_kernel"})[dom],
        "bound": "mfma",
        "achieved": round(achieved, 2),
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": round(achieved / peak, 4),
        "traffic": traffic_for(dom, kfile, w.name),
        "avg_launch_ms": round(per[dom], 4),
        "algorithmic_flop_per_launch": gemm_flop(w, KERNEL_GEMMS[dom]),
    }

    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == torch.bfloat16 else "fp32",
        "data": "synthetic (seeded N(0,1) inputs of the workload's shape)",
        "config": {
            "workload": describe(w),
            "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "T": w.T, "D": w.D, "causal": w.causal,
            "parallelism": "single GPU",
            **({"Tk": w.Tkv, "q_offset": w.q_offset} if w.Tkv != w.T else {}),
        },
        "pct_of_peak": round(100 * value / peak, 2),
        "breakdown": {
            "fwd_ms": round(per["fwd"], 4), "pre_ms": round(per["pre"], 4),
            "dkdv_ms": round(per["dkdv"], 4), "dq_ms": round(per["dq"], 4),
            "fwd_tflops": round(fwd_tflops, 2), "fwd_pct_peak": round(100 * fwd_tflops / peak, 2),
            "bwd_tflops": round(bwd_tflops, 2), "bwd_pct_peak": round(100 * bwd_tflops / peak, 2),
            "pre_gbps": round(pre_bytes / (per["pre"] * 1e-3) / 1e9, 1),
            "bwd_path": ("dQ kernel forms Delta, then dK/dV (as fa_bwd); pre_ms: the preprocess "
                         "kernel timed on its own" if fused else "preprocess, dK/dV, dQ"),
            "step_launch": launch,
            "kernel_ms": "events between the kernels of K eager steps after the timed region",
        },
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline and w.Tkv == w.T:  # the sample takes prefixes of one sequence
        print("[bench] timing the oracle on a bounded sample", file=sys.stderr, flush=True)
        out["cpu_baseline"], ref = cpu_baseline(w, x, args.cpu_seconds)
        if ref is not None:
            out["parity"] = parity_errors(w, {"o": o, "lse": lse, "dq": dq, "dk": dk, "dv": dv}, ref)
            if fused:
                out["parity_float32_results"] = float32_results_errors(w, q, k, v, do, fpart, ref)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
