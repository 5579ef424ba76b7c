#!/usr/bin/env python3
"""Benchmark of the S2-Attn hot path on one MI355X: forward + backward per step.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--range W1,W2,..]

A step is one forward (s2attn_fwd) and one backward (its two launches, as
s2attn_bwd runs them: prep fused into dQ, then dK/dV) over one batch of seeded
synthetic inputs already resident in HBM.  Untimed steps for half a second
(the clock ramp, so the engine clock has left its idle state), W untimed
warm-up steps, then K steps between two device synchronisations; the wall time of those K
steps gives ``value`` (effective TFLOP/s: group-local causal pairs only, 4d
FLOP per pair forward, 10d backward).  HIP events recorded on the launch
stream around every kernel launch give each kernel's average duration; the
longest one is the roofline kernel.  Afterwards a vendor bf16 GEMM on
standard-normal operands is timed as the practical matrix-core ceiling for
data of this distribution, and the float64 CPU oracle is timed on a bounded
sample of the same workload (rank 0, one GPU only).  The other workloads of
the metric's N range (8k, 100k, and the 70B GQA shape at 32k), Table 7's 1/6
group at 8k and full causal attention at 100k (G = N) are then timed and
reported under "range" (outside the timed region): each is warmed up for
at least half a second, so the clock has left the idle state the CPU timing
leaves it in, and timed over at least a quarter second of steps.

Prints one JSON line.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "shifted_sparse_attention_s2attn_amd", "csrc")


def _code_only(text):
    """C++ source without its comments and blank lines, each line stripped, so
    that an edit of a comment does not count as a change of the kernels."""
    import re
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*", "", line).strip() for line in text.splitlines())
    return "\n".join(line for line in lines if line)


def kernel_source_hash():
    """Hash of the device code and its launchers: every csrc file except
    s2attn_api.hip, which only validates arguments before calling them;
    comments and layout are ignored."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name == "s2attn_api.hip":
            continue
        with open(os.path.join(CSRC, name), encoding="utf-8") as f:
            h.update(name.encode())
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def read_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if current.

    The summary lists FETCH_SIZE / WRITE_SIZE (KiB per dispatch) of the kernel,
    the same counters for a plain copy kernel of known size, and the hash of the
    kernel sources they were taken with.  Returns None when absent or stale.
    """
    path = os.path.join(PROFILES, f"{kernel}_{workload}_hbm_counters.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        line = line.strip()
        if line and not line.startswith("#") and "=" in line:
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_hash") != kernel_source_hash():
        return None
    fetch_scale = float(vals["copy_bytes_read"]) / (float(vals["copy_fetch_kib"]) * 1024)
    write_scale = float(vals["copy_bytes_written"]) / (float(vals["copy_write_kib"]) * 1024)
    return (float(vals["kernel_fetch_kib"]) * 1024 * fetch_scale +
            float(vals["kernel_write_kib"]) * 1024 * write_scale)


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return max(n)
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def cpu_baseline(w, t, seconds, wrap="roll"):
    """Time the float64 oracle (fwd + bwd) on whole (batch, head, group) slices of the inputs."""
    import numpy as np
    from oracle import s2attn_oracle as orc
    r = w.H // w.Hkv
    done, flop, el = 0, 0, 0.0
    for h in range(w.H):
        c = h // r
        q = t["q"][:, :, h:h + 1].float().cpu().numpy().astype(np.float64)
        k = t["k"][:, :, c:c + 1].float().cpu().numpy().astype(np.float64)
        v = t["v"][:, :, c:c + 1].float().cpu().numpy().astype(np.float64)
        do = t["do"][:, :, h:h + 1].float().cpu().numpy().astype(np.float64)
        S1 = 1 if h >= w.H - w.shift_heads else 0
        groups = w.N // w.G
        for g in range(groups):
            t0 = time.perf_counter()
            orc.head_group_forward(q, k, v, w.G, S1, 0, 0, g, wrap)
            orc.head_group_backward(q, k, v, do, w.G, S1, 0, 0, g, wrap)
            el += time.perf_counter() - t0
            done += 1
            pairs = w.G * (w.G + 1) // 2
            if wrap == "split" and S1 and g == groups - 1 and w.N % w.G == 0:
                pairs -= (w.G - w.G // 2) * (w.G // 2)   # the wrap group cut in two
            flop += 14 * w.d * pairs
            if el >= seconds:
                break
        if el >= seconds:
            break
    return {
        "value": flop / el / 1e12,
        "unit": "TFLOP/s",
        "cores": blas_threads(),
        "kind": "oracle",
        "sample": f"{done} (batch, head, group) slices of {w.G} query rows, forward + backward, "
                  f"float64 NumPy, {el:.1f} s",
    }


def device_peak():
    """The bf16 dense matrix-core peak recomputed from what rocminfo reports for
    the GPU agent (compute units x max engine clock x 4096 FLOP per CU-clock),
    next to the nominal figure; None where rocminfo is not available."""
    import re
    import subprocess
    try:
        out = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except (OSError, subprocess.SubprocessError):
        return None
    for block in out.split("Agent ")[1:]:
        if not re.search(r"Name:\s+gfx9", block):
            continue
        cu = re.search(r"Compute Unit:\s+(\d+)", block)
        mhz = re.search(r"Max Clock Freq\. \(MHz\):\s+(\d+)", block)
        if cu and mhz:
            n, f = int(cu.group(1)), int(mhz.group(1))
            return {"compute_units": n, "max_clock_mhz": f, "bf16_peak_tflops": round(n * f * 1e6 * 4096 / 1e12, 1)}
    return None


def gemm_reference(torch, dev, n=16384, reps=5):
    """A vendor bf16 GEMM (torch.matmul, i.e. hipBLASLt) of n x n x n on seeded
    standard-normal operands: the rate a tuned dense contraction sustains on this
    chip with data of the inputs' distribution.  The matrix cores' throughput
    depends on the operand bits (the clock drops under random data), so this,
    not the nominal peak, is the practical ceiling of an MFMA-bound kernel."""
    g = torch.Generator(device=dev).manual_seed(0)
    a = torch.randn((n, n), generator=g, device=dev, dtype=torch.bfloat16)
    b = torch.randn((n, n), generator=g, device=dev, dtype=torch.bfloat16)
    c = torch.empty((n, n), device=dev, dtype=torch.bfloat16)
    for _ in range(2):
        torch.matmul(a, b, out=c)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b, c
    return {"tflops": round(2 * n ** 3 / ms / 1e9, 1), "ms": round(ms, 4), "shape": f"{n}x{n}x{n}",
            "operands": "bf16, seeded standard normal", "library": "torch.matmul (hipBLASLt)"}


WARM_S, TIMED_S = 0.5, 0.25


def time_workload(torch, w, wrap, steps, warmup):
    """Forward and backward of one more workload (the same launches as the timed
    step), HIP events on the launch stream; per-kernel and per-pass averages."""
    from shifted_sparse_attention_s2attn_amd import (s2attn_bwd_dkdv, s2attn_bwd_prep_dq,
                                                     s2attn_bwd_workspace_bytes, s2attn_fwd)
    from shifted_sparse_attention_s2attn_amd import flops as F
    from shifted_sparse_attention_s2attn_amd.inputs import make_inputs
    dev = torch.device("cuda:0")
    t = make_inputs(w, seed=0, device="cuda")
    q, k, v, do = t["q"], t["k"], t["v"], t["do"]
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(s2attn_bwd_workspace_bytes(w.B, w.H, w.Hkv, w.N, w.d, w.G, w.shift_heads, q.dtype),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        s2attn_fwd(q, k, v, w.G, w.shift_heads, out=o, lse=lse, wrap=wrap)
        if ev:
            ev[1].record(stream)
        s2attn_bwd_prep_dq(q, k, v, o, lse, do, dq, ws, w.G, w.shift_heads, wrap=wrap)
        if ev:
            ev[2].record(stream)
        s2attn_bwd_dkdv(q, k, v, do, dk, dv, ws, w.G, w.shift_heads, wrap=wrap)
        if ev:
            ev[3].record(stream)

    # Warm-up: at least `warmup` steps and at least WARM_S seconds of them, so
    # the engine clock has left its idle state (the host-side oracle timing
    # before this leaves the GPU idle for seconds); then at least `steps`
    # steps and at least TIMED_S seconds' worth, so that short workloads are
    # not timed over a few hundred microseconds.
    torch.cuda.synchronize()
    t0, n = time.perf_counter(), 0
    while n < warmup or time.perf_counter() - t0 < WARM_S:
        step()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    per_step = (time.perf_counter() - t0) / n
    steps = max(steps, min(int(TIMED_S / per_step) + 1, 2000))
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    ms = [sum(ev[j].elapsed_time(ev[j + 1]) for ev in events) / steps for j in range(3)]
    fwd_f = F.fwd_flops(w.B, w.H, w.N, w.G, w.d, w.shift_heads, wrap)
    bwd_f = F.bwd_flops(w.B, w.H, w.N, w.G, w.d, w.shift_heads, wrap)
    peak = F.MI355X_BF16_PEAK_TFLOPS if w.dtype == "bf16" else F.MI355X_F32_PEAK_TFLOPS
    bwd_ms = ms[1] + ms[2]
    del t, q, k, v, do, o, lse, dq, dk, dv, ws
    torch.cuda.empty_cache()
    return {"N": w.N, "G": w.G, "H": w.H, "Hkv": w.Hkv, "steps": steps,
            "ms_per_step": round(ms[0] + bwd_ms, 4),
            "tflops": round((fwd_f + bwd_f) / (ms[0] + bwd_ms) / 1e9, 1),
            "frac_of_peak": round((fwd_f + bwd_f) / (ms[0] + bwd_ms) / 1e9 / peak, 4),
            "fwd": {"ms": round(ms[0], 4), "frac_of_peak": round(fwd_f / ms[0] / 1e9 / peak, 4)},
            "bwd": {"ms": round(bwd_ms, 4), "frac_of_peak": round(bwd_f / bwd_ms / 1e9 / peak, 4),
                    "prep_dq_ms": round(ms[1], 4), "dkdv_ms": round(ms[2], 4)}}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama2-7b-32k")
    ap.add_argument("--wrap", default="roll", choices=["roll", "split", "swap"],
                    help="wrap handling of the shifted heads (split, swap: Table 8's Variants 2, 3)")
    ap.add_argument("--rope", action="store_true",
                    help="also time the rotary embedding with Position Interpolation on q and k (and its inverse "
                         "on dq and dk), the step before the attention, and a whole step with the rotary passes "
                         "stand-alone against one with them fused into the attention kernels (k's pass kept); "
                         "reported apart from the step")
    ap.add_argument("--range", default="llama2-7b-8k,llama2-7b-100k,llama2-70b-gqa-32k,llama2-7b-8k-g1365,"
                                       "llama2-7b-100k-fullattn",
                    help="comma-separated workloads also timed (forward and backward only, a few steps each) and "
                         "reported under \"range\", so the metric's whole N range is measured in one run; empty = none")
    ap.add_argument("--range-steps", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gemm-reference", action="store_true")
    ap.add_argument("--hbm-copy-bytes", type=int, default=0,
                    help="after timing, run one plain device-to-device copy of this many bytes; under "
                         "rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE it calibrates the HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "attention units (batch, head, group) are independent, so several GPUs would each "
              "run this same kernel on their own share of heads or batch.", file=sys.stderr)
        sys.exit(2)

    import torch
    from shifted_sparse_attention_s2attn_amd import (s2attn_bwd_dkdv, s2attn_bwd_prep_dq,
                                                     s2attn_bwd_workspace_bytes, s2attn_fwd)
    from shifted_sparse_attention_s2attn_amd import flops as F
    from shifted_sparse_attention_s2attn_amd.inputs import WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    range_names = [n for n in args.range.split(",") if n and n != w.name]
    for n in range_names:
        if n not in WORKLOADS:
            ap.error(f"unknown workload in --range: {n}")
    t = make_inputs(w, seed=0, device="cuda")
    q, k, v, do = t["q"], t["k"], t["v"], t["do"]
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(s2attn_bwd_workspace_bytes(w.B, w.H, w.Hkv, w.N, w.d, w.G, w.shift_heads, q.dtype),
                     dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    # the backward as the library's s2attn_bwd runs it: prep fused into dq, then dK/dV
    names = ["fwd", "bwd_prep_dq", "bwd_dkdv"]

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        s2attn_fwd(q, k, v, w.G, w.shift_heads, out=o, lse=lse, wrap=args.wrap)
        if ev:
            ev[1].record(stream)
        s2attn_bwd_prep_dq(q, k, v, o, lse, do, dq, ws, w.G, w.shift_heads, wrap=args.wrap)
        if ev:
            ev[2].record(stream)
        s2attn_bwd_dkdv(q, k, v, do, dk, dv, ws, w.G, w.shift_heads, wrap=args.wrap)
        if ev:
            ev[3].record(stream)

    # Clock ramp: untimed steps for at least WARM_S seconds, so the engine clock
    # has left its idle state before the W warm-up steps (a short workload's
    # few warm-up steps would otherwise be timed on a clock still rising);
    # their count is reported as "clock_ramp_steps".
    torch.cuda.synchronize()
    t_ramp, ramp_steps = time.perf_counter(), 0
    while time.perf_counter() - t_ramp < WARM_S:
        step()
        ramp_steps += 1
        if ramp_steps % 8 == 0:
            torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    ms_step = el * 1e3 / args.steps

    kern_all = {n: sorted(ev[j].elapsed_time(ev[j + 1]) for ev in events) for j, n in enumerate(names)}
    kern_ms = {n: sum(v) / len(v) for n, v in kern_all.items()}
    fwd_f = F.fwd_flops(w.B, w.H, w.N, w.G, w.d, w.shift_heads, args.wrap)
    bwd_f = F.bwd_flops(w.B, w.H, w.N, w.G, w.d, w.shift_heads, args.wrap)
    peak = F.MI355X_BF16_PEAK_TFLOPS if w.dtype == "bf16" else F.MI355X_F32_PEAK_TFLOPS
    # algorithmic FLOP per launch: the backward's five contractions are S, dP, dV, dK
    # (the dK/dV kernel, 8d per pair) and dQ (the dQ kernel, 2d per pair; that kernel
    # also recomputes S and dP, which are not counted again)
    pairs = F.allowed_pairs(w.B, w.H, w.N, w.G, w.shift_heads, args.wrap)
    kern_flops = {"fwd": fwd_f, "bwd_dkdv": 8 * w.d * pairs, "bwd_prep_dq": 2 * w.d * pairs}
    dominant = max(kern_ms, key=kern_ms.get)
    kernels = {}
    for n, ms in kern_ms.items():
        times = kern_all[n]
        kernels[n] = {"ms": round(ms, 4), "ms_min": round(times[0], 4),
                      "ms_median": round(times[len(times) // 2], 4), "ms_max": round(times[-1], 4)}
        if n in kern_flops:
            kernels[n]["tflops"] = round(kern_flops[n] / ms / 1e9, 1)
            kernels[n]["frac_of_peak"] = round(kern_flops[n] / ms / 1e9 / peak, 4)
    kernels["bwd_prep_dq"]["executed_tflops"] = round(6 * w.d * pairs / kern_ms["bwd_prep_dq"] / 1e9, 1)
    fwd_ms = kern_ms["fwd"]
    bwd_ms = kern_ms["bwd_prep_dq"] + kern_ms["bwd_dkdv"]
    achieved = kern_flops[dominant] / kern_ms[dominant] / 1e9    # every launch is a contraction
    roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak, "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4)}
    roof["kernel"] = dominant
    # the committed counter summaries were taken with the main method's row map
    roof["traffic"] = read_traffic(dominant, w.name) if args.wrap == "roll" else None

    result = {
        "metric": "S2-Attn fwd+bwd effective TFLOP/s (group-local causal pairs), % of bf16 MFMA peak",
        "value": round((fwd_f + bwd_f) / (ms_step / 1e3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "clock_ramp_steps": ramp_steps,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Hkv": w.Hkv, "d": w.d, "N": w.N, "G": w.G,
                   "shift_heads": w.shift_heads, "wrap": args.wrap, "parallelism": "none"},
        "fwd": {"ms": round(fwd_ms, 4), "tflops": round(fwd_f / fwd_ms / 1e9, 1),
                "frac_of_peak": round(fwd_f / fwd_ms / 1e9 / peak, 4)},
        "bwd": {"ms": round(bwd_ms, 4), "tflops": round(bwd_f / bwd_ms / 1e9, 1),
                "frac_of_peak": round(bwd_f / bwd_ms / 1e9 / peak, 4)},
        "frac_of_peak": round((fwd_f + bwd_f) / (ms_step / 1e3) / 1e12 / peak, 4),
        "kernels": kernels,
        "roofline": roof,
        "cpu_baseline": None,
    }
    if args.hbm_copy_bytes > 0:
        src = torch.empty(args.hbm_copy_bytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.add(src, 1.0, out=dst)            # one elementwise kernel: reads and writes N bytes
        torch.cuda.synchronize()
        result["hbm_copy_bytes"] = src.numel() * 4
        del src, dst
    if args.rope:
        from shifted_sparse_attention_s2attn_amd import s2attn_bwd_rope, s2attn_fwd_rope, s2attn_rope
        pi = 4096 / w.N                          # Position Interpolation from a 4k model to this context
        qr, kr = torch.empty_like(q), torch.empty_like(k)

        def rope_step():
            s2attn_rope(q, pi, out=qr)
            s2attn_rope(k, pi, out=kr)
            s2attn_rope(dq, pi, inverse=True, out=qr)
            s2attn_rope(dk, pi, inverse=True, out=kr)

        def unfused_step():                      # rotary passes around the plain attention step
            s2attn_rope(q, pi, out=qr)
            s2attn_rope(k, pi, out=kr)
            s2attn_fwd(qr, kr, v, w.G, w.shift_heads, out=o, lse=lse, wrap=args.wrap)
            s2attn_bwd_prep_dq(qr, kr, v, o, lse, do, dq, ws, w.G, w.shift_heads, wrap=args.wrap)
            s2attn_bwd_dkdv(qr, kr, v, do, dk, dv, ws, w.G, w.shift_heads, wrap=args.wrap)
            s2attn_rope(dq, pi, inverse=True, out=dq)
            s2attn_rope(dk, pi, inverse=True, out=dk)

        qrot = torch.empty_like(q)

        def fused_step():                        # k's pass only; q, dq, dk turned inside the kernels
            s2attn_rope(k, pi, out=kr)
            s2attn_fwd_rope(q, kr, v, w.G, w.shift_heads, pi, wrap=args.wrap, out=o, lse=lse, q_rot=qrot)
            s2attn_bwd_rope(qrot, kr, v, o, lse, do, w.G, w.shift_heads, pi, wrap=args.wrap, workspace=ws,
                            grads=(dq, dk, dv))

        def timed(fn, reps):
            for _ in range(3):
                fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for _ in range(reps):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / reps

        ms = timed(rope_step, args.steps)
        nbytes = 2 * 2 * (q.numel() + k.numel()) * q.element_size()   # read + write, forward and inverse
        result["rope"] = {"ms": round(ms, 4), "gbps": round(nbytes / ms / 1e6, 1), "bytes": nbytes,
                          "pos_scale": pi, "bound": "hbm", "frac_of_8tbs": round(nbytes / ms / 1e6 / 8000, 4)}
        # the two routes alternated, so both see the same clock
        un, fu = [], []
        for _ in range(3):
            un.append(timed(unfused_step, args.steps))
            fu.append(timed(fused_step, args.steps))
        result["rope"]["step_ms_standalone"] = round(sorted(un)[1], 4)
        result["rope"]["step_ms_fused"] = round(sorted(fu)[1], 4)
    result["device_peak"] = device_peak()
    if w.dtype == "bf16" and not args.no_gemm_reference:
        ref = gemm_reference(torch, dev)
        ref["fwd_frac"] = round(fwd_f / fwd_ms / 1e9 / ref["tflops"], 4)
        ref["roofline_kernel_frac"] = round(roof["achieved"] / ref["tflops"], 4)
        result["gemm_reference"] = ref
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, t, args.cpu_seconds, args.wrap)
    if range_names:
        del t, q, k, v, do, o, lse, dq, dk, dv, ws
        torch.cuda.empty_cache()
        result["range"] = {n: time_workload(torch, WORKLOADS[n], args.wrap, args.range_steps, 3) for n in range_names}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
