#!/usr/bin/env python3
"""Benchmark of the exact-attention forward on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--pass fwd|bwd]
                    [--pv-dtype bf16|e4m3]

``--pv-dtype e4m3`` (fp8 workloads) times the P.V product in e4m3 on the
8-bit matrix instructions instead of bf16.  ``--pass bwd`` measures the
backward instead (dQ, dK, dV after one forward;
2.5x the forward's flop, the five products S, dP, dV, dK, dQ) with the float64
gradient oracle as the CPU baseline.

Prints ONE JSON line.  A step is one forward call over the whole workload
(inputs already resident in HBM): ``value`` is the whole-job throughput in
TFLOP/s over K timed steps bracketed by device synchronisation, counting only
visible (unmasked) query/key pairs at 4*d flop each.  ``roofline`` prices the
kernel's own average duration (HIP events on the launch stream) against the
MI355X dense MFMA peak of its input type.  ``cpu_baseline`` times the float64
oracle (the checker of the tests, not a tuned CPU kernel) on a bounded sample
of the same workload's heads, on the host cores.  For the short workloads
(under 1e11 flop) ``short_sequence`` adds the per-launch time of launches the
GPU runs back to back (queued behind a spin kernel, so none waits on the
host's launch path), HBM GB/s from it, and a cold-cache kernel time.

The default workload is the causal bf16 d=128 N=4096 case (B=4, H=32).  The
warm-up / timed step counts default to the pages' protocol of 10 warm-up calls
and 100 timed calls ("Flash Attention | Hermes Skill", Workflow 2, Step 4).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s and % of MFMA peak (bf16 causal d=128, N=4096)"
# MI355X dense MFMA peaks (256 CUs x 2.4 GHz): 16-bit 4096 flop/CU/clk, fp8 8192.
PEAK_TFLOPS = {"f16": 2516.6, "bf16": 2516.6, "fp8": 5033.2}
HBM_PEAK_GBS = 8000.0
# the forward and backward kernels' sources (a recorded traffic measurement is valid only for these)
KERNEL_SRCS = [os.path.join(ROOT, "exact_attention_04_amd", "csrc", f) for f in ("fwd_kernel.hip", "kernel_common.h")]
BWD_KERNEL_SRCS = [os.path.join(ROOT, "exact_attention_04_amd", "csrc", f) for f in ("bwd_kernel.hip", "kernel_common.h")]


def visible_pairs_per_head(w) -> int:
    """Number of (query, key) pairs the mask leaves visible in one head."""
    n = w.seqlen
    i = np.arange(n, dtype=np.int64)
    hi = np.full(n, n - 1, dtype=np.int64)
    if w.causal:
        hi = np.minimum(hi, i)
    if w.window_right >= 0:
        hi = np.minimum(hi, i + w.window_right)
    lo = np.maximum(0, i - w.window_left) if w.window_left >= 0 else np.zeros(n, dtype=np.int64)
    return int(np.maximum(hi - lo + 1, 0).sum())


def workload_flops(w) -> float:
    return 4.0 * w.headdim * visible_pairs_per_head(w) * w.batch * w.heads


def workload_bytes(w) -> float:
    """One read of Q, K, V plus one write of O (16-bit) and of the fp32 LSE."""
    esz = 1 if w.dtype == "fp8" else 2
    q_elems = w.batch * w.heads * w.seqlen * w.headdim
    kv_elems = w.batch * w.kv_heads * w.seqlen * w.headdim
    return float((q_elems + 2 * kv_elems) * esz + 2 * q_elems + 4 * w.batch * w.heads * w.seqlen)


def kernel_code(text: str) -> str:
    """Kernel source without `//` comments and blank lines: edits to the
    comments leave a recorded measurement valid."""
    lines = (re.sub(r"//.*$", "", line).rstrip() for line in text.splitlines())
    return "\n".join(line for line in lines if line.strip())


def kernel_hash(srcs=None) -> str:
    h = hashlib.sha256()
    for path in srcs or KERNEL_SRCS:
        with open(path, encoding="utf-8") as f:
            h.update(kernel_code(f.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, pv8: bool = False, bwd: bool = False):
    """HBM bytes per launch (per backward call with `bwd`) from a committed
    counter summary, if still current."""
    name = f"traffic_bwd_{workload}" if bwd else f"traffic_{workload}{'_pv8' if pv8 else ''}"
    path = os.path.join(ROOT, "profiles", name + ".json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_sha256_16") != kernel_hash(BWD_KERNEL_SRCS if bwd else None):
        return None
    return rec.get("hbm_bytes_per_launch")


def time_gpu(w, steps: int, warmup: int, pv8: bool = False):
    import torch
    from exact_attention_04_amd import attention, plan
    from exact_attention_04_amd.workloads import make_inputs

    inp = make_inputs(w)
    dev = torch.device("cuda", 0)
    q, k, v = (t.to(dev) for t in (inp.q, inp.k, inp.v))
    o = torch.empty(q.shape, dtype=torch.bfloat16 if w.dtype == "fp8" else q.dtype, device=dev)
    lse = torch.empty((w.batch, w.heads, w.seqlen), dtype=torch.float32, device=dev)
    kw = dict(causal=w.causal, window_size=(w.window_left, w.window_right), softmax_scale=w.softmax_scale,
              layout=w.layout, descale=inp.descale if w.dtype == "fp8" else None)
    if pv8:
        kw["pv_dtype"] = torch.float8_e4m3fn
    info = plan(q, k, v, o, lse, **kw)
    for _ in range(warmup):
        attention(q, k, v, out=o, lse=lse, **kw)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)   # the stream the kernel is launched on
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        attention(q, k, v, out=o, lse=lse, **kw)
        ends[i].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kern_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]

    def run_once():
        attention(q, k, v, out=o, lse=lse, **kw)

    return {
        "run": run_once,
        "ms_per_step": (t1 - t0) * 1e3 / steps,
        "kernel_ms_avg": float(np.mean(kern_ms)),
        "kernel_ms_median": float(np.median(kern_ms)),
        "kernel_ms_min": float(np.min(kern_ms)),
        "plan": info,
    }


def time_gpu_bwd(w, steps: int, warmup: int):
    """Time the backward (both kernels) after one forward for O and LSE."""
    import torch
    from exact_attention_04_amd import attention, attention_backward
    from exact_attention_04_amd.workloads import make_inputs

    inp = make_inputs(w)
    dev = torch.device("cuda", 0)
    q, k, v = (t.to(dev) for t in (inp.q, inp.k, inp.v))
    g = torch.Generator(device=dev).manual_seed(w.seed + 7)
    do = torch.randn(q.shape, device=dev, generator=g).to(q.dtype)
    kw = dict(causal=w.causal, window_size=(w.window_left, w.window_right), softmax_scale=w.softmax_scale,
              layout=w.layout)
    o, lse = attention(q, k, v, **kw)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty_like(lse)
    for _ in range(warmup):
        attention_backward(q, k, v, o, do, lse, dq=dq, dk=dk, dv=dv, delta=delta, **kw)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        attention_backward(q, k, v, o, do, lse, dq=dq, dk=dk, dv=dv, delta=delta, **kw)
        ends[i].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    kern_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]

    def run_once():
        attention_backward(q, k, v, o, do, lse, dq=dq, dk=dk, dv=dv, delta=delta, **kw)

    return {"run": run_once, "ms_per_step": (t1 - t0) * 1e3 / steps, "kernel_ms_avg": float(np.mean(kern_ms)),
            "kernel_ms_median": float(np.median(kern_ms)), "kernel_ms_min": float(np.min(kern_ms))}


def cpu_baseline_bwd(w, target_s: float = 12.0, max_procs: int = 16):
    """Time the float64 gradient oracle on whole heads of the workload."""
    import torch
    import oracle
    from oracle.sdpa_fp64 import make_pool
    from oracle.sdpa_bwd_fp64 import attention_backward_parallel
    from exact_attention_04_amd.workloads import make_inputs

    inp = make_inputs(w)
    cores = max(1, min(len(os.sched_getaffinity(0)), max_procs))
    rng = np.random.default_rng(w.seed + 7)

    def head(b, h):
        g = oracle.kv_head_of(h, w.heads, w.kv_heads)
        out = []
        for t, hh in zip((inp.q, inp.k, inp.v), (h, g, g)):
            x = t[b, :, hh, :] if w.layout == "bshd" else t[b, hh, :, :]
            out.append(x.float().numpy())
        out.append(rng.standard_normal(out[0].shape))
        return tuple(out)

    order = [(b, h) for h in range(w.heads) for b in range(w.batch)]
    pool = make_pool(cores)
    try:
        list(pool.map(abs, range(cores)))
        done, elapsed = 0, 0.0
        while done < len(order) and elapsed < target_s:
            batch = [head(b, h) for (b, h) in order[done:done + cores]]
            t0 = time.perf_counter()
            attention_backward_parallel(batch, w.softmax_scale, w.causal, (w.window_left, w.window_right), pool)
            elapsed += time.perf_counter() - t0
            done += len(batch)
    finally:
        pool.shutdown()
    flops = 2.5 * workload_flops(w) * done / (w.batch * w.heads)
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} of {w.batch * w.heads} (batch, head) pairs, all rows, float64 numpy gradients, "
                      f"one process per core; {elapsed:.1f} s wall", "seconds": elapsed}


def cold_cache_us(run_once, reps: int = 20, flush_bytes: int = 512 << 20):
    """Median kernel time with L2 and the MALL flushed before each call (a
    512 MB device write between calls, outside the timed events)."""
    import torch
    buf = torch.empty(flush_bytes // 4, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    times = []
    for i in range(reps):
        buf.fill_(float(i))
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record(stream)
        run_once()
        e.record(stream)
        torch.cuda.synchronize()
        times.append(s.elapsed_time(e) * 1e3)
    del buf
    return float(np.median(times))


def queued_us(run_once, reps: int = 50):
    """Per-launch time of `reps` launches that the GPU runs back to back: they
    are queued behind a spin kernel that lasts longer than the host takes to
    issue them, so no launch waits on the host (for the short workloads the
    host's launch path is longer than the kernel)."""
    import torch
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        run_once()
    issue_s = time.perf_counter() - t0
    torch.cuda.synchronize()
    # cycles of the spin kernel per second of wall time
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    torch.cuda._sleep(1_000_000)
    b.record(stream)
    torch.cuda.synchronize()
    cycles_per_s = 1_000_000 / max(a.elapsed_time(b) * 1e-3, 1e-9)
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(3.0 * issue_s * cycles_per_s) + 100_000)
    s.record(stream)
    for _ in range(reps):
        run_once()
    e.record(stream)
    torch.cuda.synchronize()
    return s.elapsed_time(e) * 1e3 / reps


def sample_clock(run_once, kernel_ms: float, cap_s: float = 15.0):
    """GFX clock of each XCD and socket power while the kernel runs back to
    back: three `amd-smi metric` samples one second apart, after a second of
    load; medians over the samples (None when the tool is unavailable)."""
    import shutil
    import subprocess
    import threading

    import torch
    exe = shutil.which("amd-smi") or "/opt/rocm/bin/amd-smi"
    if not os.path.exists(exe):
        return None
    out = {}

    def sampler():
        try:
            time.sleep(1.0)   # clocks settle under load first
            r = subprocess.run([exe, "metric", "-g", "0", "-c", "-p", "-w", "1", "-i", "3", "--json"],
                               capture_output=True, text=True, timeout=30)
            out["raw"] = r.stdout
        except Exception as e:   # the measurement is optional
            out["err"] = repr(e)

    batch = max(8, int(25.0 / max(kernel_ms, 1e-3)))   # >= 25 ms of work between host syncs
    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    t0 = time.time()
    while th.is_alive() and time.time() - t0 < cap_s:
        for _ in range(batch):
            run_once()
        torch.cuda.synchronize()
    th.join(timeout=1.0)
    try:
        raw, dec, pos, samples = out["raw"], json.JSONDecoder(), 0, []
        while True:
            i = raw.find("{", pos)
            if i < 0:
                break
            obj, pos = dec.raw_decode(raw, i)
            samples.append(obj["gpu_data"][0])
        mhz = [[float(g["clock"][f"gfx_{x}"]["clk"]["value"]) for x in range(8)] for g in samples]
        watts = [float(g["power"]["socket_power"]["value"]) for g in samples]
        per_xcd = [float(v) for v in np.median(np.array(mhz), axis=0)]
        return {"gfx_mhz": per_xcd, "gfx_mhz_mean": round(float(np.mean(per_xcd)), 1),
                "socket_power_w": float(np.median(watts)), "samples": len(samples),
                "tool": "amd-smi metric -g 0 -c -p -w 1 -i 3 while the kernel runs back to back (medians)"}
    except Exception:
        return None


def copy_calibration(nbytes: int = 1 << 30):
    """A plain device copy of known size, for scaling HBM byte counters."""
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    return nbytes


def cpu_baseline(w, target_s: float = 12.0, max_procs: int = 16):
    """Time the float64 oracle on whole heads of the workload, batch by batch."""
    import torch
    import oracle
    from oracle.sdpa_fp64 import make_pool
    from exact_attention_04_amd.workloads import make_inputs

    inp = make_inputs(w)
    cores = max(1, min(len(os.sched_getaffinity(0)), max_procs))

    def head(b, h):
        out = []
        g = oracle.kv_head_of(h, w.heads, w.kv_heads)   # the K/V head query head h reads
        for t, s, hh in zip((inp.q, inp.k, inp.v), inp.descale, (h, g, g)):
            x = t[b, :, hh, :] if w.layout == "bshd" else t[b, hh, :, :]
            if x.dtype == torch.float8_e4m3fn:
                out.append(oracle.dequantize_e4m3(x.contiguous().view(torch.uint8).numpy(), s))
            else:
                out.append(x.float().numpy())   # exact for fp16/bf16 values
        return tuple(out)

    order = [(b, h) for h in range(w.heads) for b in range(w.batch)]
    pool = make_pool(cores)
    try:
        list(pool.map(abs, range(cores)))   # start the workers before timing
        done, elapsed = 0, 0.0
        while done < len(order) and elapsed < target_s:
            batch = [head(b, h) for (b, h) in order[done:done + cores]]
            t0 = time.perf_counter()
            oracle.attention_parallel(batch, w.softmax_scale, w.causal, (w.window_left, w.window_right), pool=pool)
            elapsed += time.perf_counter() - t0
            done += len(batch)
    finally:
        pool.shutdown()
    flops = workload_flops(w) * done / (w.batch * w.heads)
    return {
        "value": flops / elapsed / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{done} of {w.batch * w.heads} (batch, head) pairs, all {w.seqlen} query rows each, "
                  f"float64 numpy, one process per core; {elapsed:.1f} s wall",
        "seconds": elapsed,
    }


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--pass", dest="which", choices=("fwd", "bwd"), default="fwd",
                    help="fwd: the forward (the headline metric); bwd: the backward (dQ, dK, dV)")
    ap.add_argument("--pv-dtype", choices=("bf16", "e4m3"), default="bf16",
                    help="fp8 workloads: number format of P and V in the P.V product")
    ap.add_argument("--no-clock", action="store_true", help="skip the amd-smi clock and power sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB device copy (for HBM counter scaling)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this forward path has no multi-GPU mode "
              "(a head-sharded launch needs no exchange; see the design notes). Run with --gpus 1.",
              file=sys.stderr)
        return 2

    from exact_attention_04_amd.workloads import HEADLINE, WORKLOADS
    name = args.workload or HEADLINE
    w = WORKLOADS[name]
    if args.which == "bwd":
        return main_bwd(args, name, w)
    pv8 = args.pv_dtype == "e4m3"
    if pv8 and w.dtype != "fp8":
        print("--pv-dtype e4m3 applies to fp8 workloads only", file=sys.stderr)
        return 2
    flops = workload_flops(w)

    g = time_gpu(w, args.steps, args.warmup, pv8)
    if args.copy_calibration:
        copy_calibration()
    short = flops < 1e11   # the short-sequence workloads: launch- or latency-bound
    extra = {}
    if short:
        bytes_ = workload_bytes(w)
        q_us = queued_us(g["run"])
        extra["short_sequence"] = {
            "queued_us_per_launch": round(q_us, 2),
            "queued_algorithmic_GBps": round(bytes_ / (q_us * 1e-6) / 1e9, 1),
            "kernel_us_median": round(g["kernel_ms_median"] * 1e3, 2),
            "kernel_us_min": round(g["kernel_ms_min"] * 1e3, 2),
            "back_to_back_us": round(g["ms_per_step"] * 1e3, 2),
            "cold_cache_kernel_us_median": round(cold_cache_us(g["run"]), 2),
            "algorithmic_GBps_median": round(bytes_ / (g["kernel_ms_median"] * 1e-3) / 1e9, 1),
        }
    clock = None if args.no_clock else sample_clock(g["run"], g["kernel_ms_median"])
    value = flops / (g["ms_per_step"] * 1e-3) / 1e12
    achieved = flops / (g["kernel_ms_avg"] * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    traffic = measured_traffic(name, pv8)
    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(g["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": name, "batch": w.batch, "heads": w.heads, "kv_heads": w.kv_heads, "seqlen": w.seqlen, "headdim": w.headdim,
            "causal": w.causal, "window": [w.window_left, w.window_right], "layout": w.layout,
            "softmax_scale": w.softmax_scale,
            **({"pv_dtype": "e4m3"} if pv8 else {}),
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": traffic,
            "kernel": g["plan"].kernel.decode(),
            "kernel_ms_avg": round(g["kernel_ms_avg"], 5),
            "kernel_ms_median": round(g["kernel_ms_median"], 5),
            "kernel_ms_min": round(g["kernel_ms_min"], 5),
            "flop_per_launch": flops,
            "algorithmic_bytes_per_launch": workload_bytes(w),
            "algorithmic_GBps": round(workload_bytes(w) / (g["kernel_ms_avg"] * 1e-3) / 1e9, 1),
        },
        "cpu_baseline": None,
        **extra,
        "clock": clock,
    }
    if w.dtype == "fp8" and not pv8:
        # Q.K^T on the fp8 MFMA, P.V on the bf16 MFMA: half the flop at each rate
        mixed = 1.0 / (0.5 / PEAK_TFLOPS["fp8"] + 0.5 / PEAK_TFLOPS["bf16"])
        rec["roofline"]["peak_mixed"] = round(mixed, 1)
        rec["roofline"]["frac_mixed"] = round(achieved / mixed, 4)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, target_s=args.cpu_seconds)
    print(json.dumps(rec), flush=True)
    return 0


def main_bwd(args, name, w):
    """One JSON line for the backward pass on workload `w` (16-bit inputs)."""
    flops = 2.5 * workload_flops(w)   # five products of the forward's size: S, dP, dV, dK, dQ
    g = time_gpu_bwd(w, args.steps, args.warmup)
    if args.copy_calibration:
        copy_calibration()
    achieved = flops / (g["kernel_ms_avg"] * 1e-3) / 1e12
    peak = PEAK_TFLOPS[w.dtype]
    esz = 2
    q_el = w.batch * w.heads * w.seqlen * w.headdim
    kv_el = w.batch * w.kv_heads * w.seqlen * w.headdim
    nbytes = float(esz * (3 * q_el + 2 * kv_el) + esz * (q_el + 2 * kv_el) + 8 * w.batch * w.heads * w.seqlen)
    rec = {
        "metric": "attention bwd TFLOP/s (dQ, dK, dV; 2.5x the forward's flop)",
        "value": round(flops / (g["ms_per_step"] * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(g["ms_per_step"], 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": name, "pass": "bwd", "batch": w.batch, "heads": w.heads, "kv_heads": w.kv_heads,
                   "seqlen": w.seqlen, "headdim": w.headdim, "causal": w.causal,
                   "window": [w.window_left, w.window_right], "layout": w.layout, "softmax_scale": w.softmax_scale},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": measured_traffic(name, bwd=True),
                     "kernel": "attn_bwd_dq + attn_bwd_dkdv", "kernel_ms_avg": round(g["kernel_ms_avg"], 5),
                     "kernel_ms_median": round(g["kernel_ms_median"], 5), "flop_per_launch": flops,
                     "algorithmic_bytes_per_launch": nbytes,
                     "algorithmic_GBps": round(nbytes / (g["kernel_ms_avg"] * 1e-3) / 1e9, 1)},
        "cpu_baseline": None,
    }
    if not args.no_clock:
        rec["clock"] = sample_clock(g["run"], g["kernel_ms_median"])
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline_bwd(w, target_s=args.cpu_seconds)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
