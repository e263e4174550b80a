"""Benchmark: attention forward + JVP throughput on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one attn_jvp_fwd call over the whole workload (inputs resident in
HBM, outputs preallocated).  The default workload is the 32760-token video
self-attention layer (B=1, H=40, Lq=Lk=32760, d=128, bf16).  Throughput counts
the nominal 12*B*H*Lq*Lk*d flops of the six dense products.  Prints ONE JSON
line on stdout.

Other modes:
  --proj NAME          time attn_jvp_proj, the projection of hidden states into
                       attention heads with its tangent, on a projection workload
                       (qkv_video_bf16: 32760 tokens, D = 5120 -> 3 x 40 x 128);
                       throughput counts 2*B*L*D*F flops per product (two with a
                       tangent).  Same JSON contract.
  --norm-rope NAME     time attn_jvp_rmsnorm_rope, the RMS normalisation and rotary
                       embedding of queries or keys with the tangent (q_video_bf16:
                       40 heads x 32760 rows of 128); bound by HBM traffic, so the
                       roofline is in GB/s of its algorithmic bytes.
  --copy-calibration   time/profile a plain device copy of known size (HBM
                       counter calibration) instead of the kernel.
  --trace-summary DIR  summarise a rocprofv3 kernel-trace (or counter) CSV
                       under DIR: per-kernel dispatch statistics, skipping the
                       first --skip dispatches of each kernel (the warm-ups).

The default run also times the other attention workloads (tiny fp32, image
self-attention, text cross-attention with and without the frozen-context path,
the video cross-attention stress case) and reports them under "per_workload".
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, vendor figure
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 matrix/vector, vendor figure
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, vendor figure
METRIC = "attention-JVP TFLOP/s (12*B*H*Lq*Lk*d) + % bf16 MFMA peak, 1 MI355X"
METRIC_FROZEN = "attention-JVP executed TFLOP/s, frozen context (8*B*H*Lq*Lk*d) + % bf16 MFMA peak, 1 MI355X"
METRIC_NORM_ROPE = "RMS-norm + rotary embedding JVP, HBM GB/s of algorithmic bytes (% of 8 TB/s), 1 MI355X"
METRIC_PROJ = "projection-JVP TFLOP/s (2*B*L*D*F per product, X and TX) + % bf16 MFMA peak, 1 MI355X"
# The sources of each kernel whose HBM traffic profiles/ records: a change to
# any of them makes the recorded traffic stale (reported as null).
_CSRC = "attention_forward_mode_attn_amd/csrc/"
KERNEL_SOURCES = {
    "attention": [_CSRC + "kernel_bf16.hip", _CSRC + "device_common.h", _CSRC + "launch.h"],
    "attention_fp32": [_CSRC + "kernel_fp32.hip", _CSRC + "device_common.h", _CSRC + "launch.h"],
    "proj": [_CSRC + "proj_bf16.hip", _CSRC + "device_common.h", _CSRC + "launch.h"],
    "norm_rope": [_CSRC + "norm_rope.hip", _CSRC + "device_common.h", _CSRC + "launch.h"],
    "merge": [_CSRC + "merge.hip", _CSRC + "device_common.h", _CSRC + "launch.h"],
}


def proj_kernel_name(w) -> str:
    """The projection kernel instantiation a launch of workload ``w`` runs: grids
    of at most 128 workgroups of 256 features use 128-feature tiles (without a
    tangent with a 128-wide hidden step, when D % 128 == 0)."""
    wide = -(-w.n_out * w.H * w.d // 256) * -(-w.L // 128) * w.B
    if wide <= 128 and (w.tangent or w.D % 128 == 0):
        return f"proj_bf16_kernel<{str(w.tangent).lower()}, 128, {64 if w.tangent else 128}>"
    return f"proj_bf16_kernel<{str(w.tangent).lower()}, 256, 64>"


def kernel_source_hash(kernel: str = "attention") -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel: str = "attention"):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, or None
    when there is none for this workload or the kernel changed since."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_src = re.search(r"kernel_source_sha256:\s*([0-9a-f]+)", txt)
    m_b = re.search(r"traffic_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m_src or not m_b or m_src.group(1) != kernel_source_hash(kernel):
        return None
    return float(m_b.group(1))


def sclk_path(torch):
    """The sysfs `pp_dpm_sclk` file of the card that torch's device 0 is on
    (matched by PCI domain and bus), or None where there is none."""
    import glob

    props = torch.cuda.get_device_properties(0)
    bus, dom = getattr(props, "pci_bus_id", None), getattr(props, "pci_domain_id", 0)
    for dev in sorted(glob.glob("/sys/class/drm/card*/device")):
        try:
            uevent = open(os.path.join(dev, "uevent")).read()
        except OSError:
            continue
        m = re.search(r"PCI_SLOT_NAME=([0-9a-fA-F]+):([0-9a-fA-F]+):", uevent)
        path = os.path.join(dev, "pp_dpm_sclk")
        if m and bus is not None and int(m.group(2), 16) == bus and int(m.group(1), 16) == dom \
                and os.path.exists(path):
            return path
    return None


def read_sclk_mhz(path):
    """The current shader clock: the entry marked '*' in pp_dpm_sclk."""
    try:
        m = re.search(r"(\d+)\s*Mhz\s*\*", open(path).read(), re.I)
    except OSError:
        return None
    return int(m.group(1)) if m else None


def wait_sampling_sclk(path, done, period_s: float = 0.01, min_samples: int = 20):
    """Wait for the event `done` while sampling the shader clock; returns the
    sclk summary for the JSON line.  None with fewer than `min_samples` samples:
    the firmware's figure trails the load, so a timed region much shorter than
    0.2 s does not show the clock it ran at."""
    samples = []
    while not done.query():
        if path:
            v = read_sclk_mhz(path)
            if v:
                samples.append(v)
        time.sleep(period_s)
    if len(samples) < min_samples:
        return None
    samples.sort()
    return {"median": samples[len(samples) // 2], "min": samples[0], "max": samples[-1],
            "samples": len(samples), "source": "pp_dpm_sclk, sampled while the timed launches ran"}


def _blas_cores() -> int:
    try:
        from threadpoolctl import threadpool_info

        return max((int(x.get("num_threads", 1)) for x in threadpool_info()), default=1)
    except Exception:  # pragma: no cover
        return os.cpu_count() or 1


def cpu_baseline(w, budget_s: float = 30.0, rows_per_head: int = 1024):
    """Time the fp64 oracle on sampled query rows of the same workload.

    Every head contributes ``rows_per_head`` query rows (both tile edges, the
    ragged tail and seeded random rows) against all of its keys; heads are
    added until the time budget is spent."""
    import numpy as np

    from oracle import attention_jvp_head
    from workloads import TENSORS, head_array, sample_rows

    cores = _blas_cores()
    rows_done = 0
    t_total = 0.0
    heads = 0
    for b in range(w.B):
        for h in range(w.H):
            a = {t: head_array(w, t, b, h) for t in TENSORS}
            rows = sample_rows(w, b, h, n_random=max(0, rows_per_head - 32))
            t0 = time.perf_counter()
            attention_jvp_head(a["q"], a["k"], a["v"], a["tq"], a["tk"], a["tv"], w.scale, rows=rows)
            t_total += time.perf_counter() - t0
            rows_done += rows.size
            heads += 1
            if t_total >= budget_s:
                break
        if t_total >= budget_s:
            break
    flops = 12.0 * rows_done * w.Lk * w.d
    full_s = t_total / rows_done * (w.B * w.H * w.Lq)
    return {
        "value": flops / t_total / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": f"{rows_done} query rows ({rows.size} per head x {heads} heads) of {w.name}, "
                  f"all {w.Lk} keys; {t_total:.1f} s; full workload extrapolates to {full_s:.0f} s",
        "float": "f64",
        "_np": np.__version__,
    }


def cpu_baseline_proj(w, h, budget_s: float = 30.0):
    """Time the fp64 projection oracle on growing blocks of tokens (all
    features) until the budget is spent; ``h`` holds the host inputs."""
    from oracle import projection_jvp

    n = 64
    rows_done, t_total = 0, 0.0
    while t_total < budget_s and rows_done < w.L:
        rows = list(range(rows_done, min(w.L, rows_done + n)))
        t0 = time.perf_counter()
        projection_jvp(h["x"], h["tx"], h["w"], h["bias"], w.n_out, w.H, w.d, rows=rows)
        t_total += time.perf_counter() - t0
        rows_done += len(rows)
        n *= 2
    tok = rows_done * w.B
    flops = 2.0 * (2 if w.tangent else 1) * tok * w.D * w.F
    full_s = t_total / tok * (w.B * w.L)
    return {
        "value": flops / t_total / 1e12,
        "unit": "TFLOP/s",
        "cores": _blas_cores(),
        "kind": "oracle",
        "sample": f"{tok} tokens ({rows_done} per batch x {w.B}) of {w.name}, all {w.F} features; "
                  f"{t_total:.1f} s; full workload extrapolates to {full_s:.0f} s",
        "float": "f64",
    }


def time_launches(step, stream, warmup: int, n: int):
    """Run ``step`` warmup + n times on ``stream``; per-launch HIP-event times
    (ms) of the last n, sorted."""
    import torch

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) for a, b in ev)


# The workloads timed beside the headline one in the default run: name, whether
# the frozen-context path (tk = tv = NULL) is used, timed launches.
PER_WORKLOAD = (
    ("tiny_self_fp32", False, 50),
    ("image_self_bf16", False, 20),
    ("text_cross_bf16", False, 50),
    ("text_cross_bf16", True, 50),
    ("video_cross_stress_bf16", False, 20),
)


def per_workload(warmup: int = 3):
    """Timed figures of the other attention workloads: average, median
    and minimum launch time over the timed launches (HIP events on the launch
    stream, after ``warmup`` untimed launches), TFLOP/s of the nominal
    12*B*H*Lq*Lk*d flops (of the executed 8*B*H*Lq*Lk*d on the frozen-context
    path) and the fraction of the dtype's peak."""
    import torch

    import attention_forward_mode_attn_amd as A
    from workloads import WORKLOADS
    from workloads.device import device_inputs

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    out = {}
    cache = {}
    for name, frozen, n in PER_WORKLOAD:
        w = WORKLOADS[name]
        print(f"bench: per-workload {name}{' (frozen context)' if frozen else ''}", file=sys.stderr, flush=True)
        if name not in cache:
            cache.clear()
            cache[name] = device_inputs(w)
        x = cache[name]
        o, to = torch.empty_like(x["q"]), torch.empty_like(x["q"])
        lse = torch.empty((w.B, w.H, w.Lq), dtype=torch.float32, device=dev)
        tk, tv = (None, None) if frozen else (x["tk"], x["tv"])

        def step():
            A.fwd(x["q"], x["k"], x["v"], x["tq"], tk, tv, scale=w.scale, out=(o, to, lse), stream=stream)

        ms = time_launches(step, stream, warmup, n)
        avg = sum(ms) / len(ms)
        flops = w.flops * (8.0 / 12.0 if frozen else 1.0)
        peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
        tf = flops / (avg * 1e-3) / 1e12
        out[name + ("_frozen" if frozen else "")] = {
            "B": w.B, "H": w.H, "Lq": w.Lq, "Lk": w.Lk, "d": w.d, "dtype": w.dtype,
            "path": "frozen context (tk = tv = NULL), executed 8 flops per logit and head dim" if frozen
                    else "full JVP, 12 flops per logit and head dim",
            "launches": n, "warmup": warmup,
            "avg_launch_ms": round(avg, 5), "median_launch_ms": round(ms[len(ms) // 2], 5),
            "min_launch_ms": round(ms[0], 5),
            "flops_per_launch": flops, "tflops": round(tf, 2), "peak": peak, "frac": round(tf / peak, 4),
        }
    return out


def trace_summary(directory: str, skip: int, kernel_filter: str = ""):
    """Per-kernel dispatch statistics of a rocprofv3 CSV run under
    ``directory``: the kernel trace (``*kernel_trace.csv``) gives durations from
    the dispatch timestamps; a counter run (``*counter_collection.csv``) gives
    each dispatch's counters.  The first ``skip`` dispatches of every kernel are
    left out (the untimed warm-up launches of the run)."""
    import csv
    import glob

    out = {}
    for path in sorted(glob.glob(os.path.join(directory, "**", "*kernel_trace.csv"), recursive=True)):
        with open(path) as f:
            rows = list(csv.DictReader(f))
        per = {}
        for r in rows:
            name = r.get("Kernel_Name", "")
            if kernel_filter and kernel_filter not in name:
                continue
            per.setdefault(name, []).append((int(r["Dispatch_Id"]),
                                             int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
        for name, ds in per.items():
            ds.sort()
            dur = [t for _, t in ds[skip:]]
            if not dur:
                continue
            s = sorted(dur)
            out.setdefault("kernel_trace", {})[name] = {
                "dispatches": len(ds), "skipped": min(skip, len(ds)), "counted": len(dur),
                "avg_ns": sum(dur) / len(dur), "median_ns": s[len(s) // 2], "min_ns": s[0], "max_ns": s[-1],
                "durations_ns": dur,
            }
    for path in sorted(glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)):
        with open(path) as f:
            rows = list(csv.DictReader(f))
        per = {}
        for r in rows:
            name = r.get("Kernel_Name", "")
            if kernel_filter and kernel_filter not in name:
                continue
            d = per.setdefault(name, {}).setdefault(int(r["Dispatch_Id"]), {})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            if "Start_Timestamp" in r and "End_Timestamp" in r:
                d["_duration_ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        for name, ds in per.items():
            keys = sorted(ds)[skip:]
            out.setdefault("counters", {})[name] = [dict(dispatch=k, **ds[k]) for k in keys]
    return out


def bench_norm_rope(args):
    import torch

    import attention_forward_mode_attn_amd as A
    from workloads import NORM_ROPE_WORKLOADS
    from workloads.device import device_norm_rope_inputs

    w = NORM_ROPE_WORKLOADS[args.norm_rope]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"bench: {w.name} B{w.B} H{w.H} L{w.L} d{w.d} {w.dtype} tangent={w.tangent} rope={w.rope}: "
          "generating inputs", file=sys.stderr, flush=True)
    x = device_norm_rope_inputs(w)
    y = torch.empty_like(x["x"])
    ty = torch.empty_like(x["x"]) if w.tangent else None
    stream = torch.cuda.current_stream(dev)

    def step():
        A.rmsnorm_rope(x["x"], x["tx"], x["gamma"], x["cos"], x["sin"], eps=w.eps, out=(y, ty), stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    per = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    print(f"bench: timing {args.steps} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for a, b in per:
        a.record(stream)
        step()
        b.record(stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    launch_ms = sorted(a.elapsed_time(b) for a, b in per)
    avg_launch_ms = sum(launch_ms) / len(launch_ms)
    value = w.algorithmic_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = w.algorithmic_bytes / (avg_launch_ms * 1e-3) / 1e9
    out = {
        "metric": METRIC_NORM_ROPE,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) rows and tangents, gain 1 + N(0, 0.1^2), rotary tables of positions 0..L-1)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "L": w.L, "d": w.d, "tangent": w.tangent,
                   "rope": w.rope, "gain": w.gain, "eps": w.eps, "parallelism": "single GPU"},
        "wall_s_timed_region": round(wall, 3),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": measured_traffic(w.name, "norm_rope"),
            "kernel": f"norm_rope_kernel<{str(w.dtype == 'bf16').lower()}, {w.d}>",
            "avg_launch_ms": round(avg_launch_ms, 5),
            "median_launch_ms": round(launch_ms[len(launch_ms) // 2], 5),
            "min_launch_ms": round(launch_ms[0], 5),
            "algorithmic_bytes_per_launch": w.algorithmic_bytes,
        },
    }
    if not args.no_cpu_baseline:
        print("bench: timing the fp64 oracle on whole heads (cpu_baseline)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline_norm_rope(w, args.cpu_budget)
    print(json.dumps(out), flush=True)


def cpu_baseline_norm_rope(w, budget_s: float = 30.0):
    """Time the fp64 oracle over whole heads until the budget is spent, in GB/s
    of the same algorithmic bytes per row."""
    from oracle import norm_rope_jvp
    from workloads import norm_rope_array, rope_tables

    c, s = rope_tables(w)
    g = norm_rope_array(w, "gamma") if w.gain else None
    rows, t_total, heads = 0, 0.0, 0
    for b in range(w.B):
        for h in range(w.H):
            x = norm_rope_array(w, "x", b, h)
            tx = norm_rope_array(w, "tx", b, h) if w.tangent else None
            t0 = time.perf_counter()
            norm_rope_jvp(x, tx, g, c, s, w.eps)
            t_total += time.perf_counter() - t0
            rows += w.L
            heads += 1
            if t_total >= budget_s:
                break
        if t_total >= budget_s:
            break
    per_row = w.algorithmic_bytes / w.rows
    return {
        "value": rows * per_row / t_total / 1e9,
        "unit": "GB/s",
        "cores": _blas_cores(),
        "kind": "oracle",
        "sample": f"{heads} heads x {w.L} rows of {w.name}; {t_total:.2f} s; full workload extrapolates to "
                  f"{t_total / rows * w.rows:.1f} s",
        "float": "f64",
    }


def bench_proj(args):
    import torch

    import attention_forward_mode_attn_amd as A
    from workloads import PROJ_WORKLOADS, proj_host_inputs
    from workloads.device import device_proj_inputs

    w = PROJ_WORKLOADS[args.proj]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"bench: {w.name} B{w.B} L{w.L} D{w.D} n_out{w.n_out} H{w.H} d{w.d} tangent={w.tangent}: "
          "generating inputs", file=sys.stderr, flush=True)
    x = device_proj_inputs(w)
    y = torch.empty(w.out_shape, dtype=torch.bfloat16, device=dev)
    ty = torch.empty_like(y) if w.tangent else None
    stream = torch.cuda.current_stream(dev)

    def step():
        A.proj(x["x"], x["tx"], x["w"], x["bias"], n_out=w.n_out, heads=w.H, out=(y, ty), stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    per = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    print(f"bench: timing {args.steps} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for a, b in per:
        a.record(stream)
        step()
        b.record(stream)
    ev1.record(stream)
    sclk = wait_sampling_sclk(sclk_path(torch), ev1)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = ev0.elapsed_time(ev1) / args.steps
    launch_ms = sorted(a.elapsed_time(b) for a, b in per)
    avg_launch_ms = sum(launch_ms) / len(launch_ms)
    value = w.flops / (ms_per_step * 1e-3) / 1e12
    achieved = w.flops / (avg_launch_ms * 1e-3) / 1e12
    out = {
        "metric": METRIC_PROJ,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) hidden states and tangents, N(0,1/D) weights, N(0,0.1^2) bias)",
        "config": {"workload": w.name, "B": w.B, "L": w.L, "D": w.D, "n_out": w.n_out, "H": w.H, "d": w.d,
                   "tangent": w.tangent, "bias": w.bias, "parallelism": "single GPU"},
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "wall_s_timed_region": round(wall, 3),
        "sclk_mhz": sclk,
        "roofline": {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": measured_traffic(w.name, "proj"),
            "kernel": proj_kernel_name(w),
            "avg_launch_ms": round(avg_launch_ms, 4),
            "median_launch_ms": round(launch_ms[len(launch_ms) // 2], 4),
            "min_launch_ms": round(launch_ms[0], 4),
            "algorithmic_flops_per_launch": w.flops,
            "algorithmic_bytes_per_launch": w.algorithmic_bytes,
        },
    }
    if not args.no_cpu_baseline:
        print("bench: timing the fp64 oracle on a block of tokens (cpu_baseline)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline_proj(w, proj_host_inputs(w), args.cpu_budget)
    print(json.dumps(out), flush=True)


def main():
    from workloads import WORKLOADS

    ap = argparse.ArgumentParser(description="Attention forward + JVP (or projection) throughput on one MI355X; "
                                             "prints one JSON line.")
    ap.add_argument("--gpus", type=int, default=1, help="must be 1: the library runs on one GPU")
    ap.add_argument("--steps", type=int, default=20, help="timed launches")
    ap.add_argument("--warmup", type=int, default=3, help="untimed launches before them")
    ap.add_argument("--workload", default="video_self_bf16", choices=sorted(WORKLOADS),
                    help="attention workload (default: the 32760-token video self-attention layer)")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip timing the fp64 oracle on the host")
    ap.add_argument("--cpu-budget", type=float, default=30.0, help="seconds of oracle work for the CPU baseline")
    ap.add_argument("--cpu-rows-per-head", type=int, default=1024,
                    help="query rows per head that the CPU baseline times (then extrapolated)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a plain 1 GiB device copy instead (HBM counter calibration)")
    ap.add_argument("--split", type=int, default=0,
                    help="time the key-sharded path: N attn_jvp_fwd_part passes plus attn_jvp_merge; "
                         "the roofline object then covers the merge launch (HBM bound)")
    ap.add_argument("--f32-partials", action="store_true",
                    help="with --split: bf16 shards write float32 partial O and tO (dtype 2), which the merge "
                         "rounds to bf16 once")
    ap.add_argument("--frozen-context", action="store_true",
                    help="pass tk = tv = NULL (workloads whose key tangents are zero); "
                         "value is then executed TFLOP/s at 8 flops per logit and head dim")
    ap.add_argument("--proj", default=None,
                    help="time the projection into attention heads (attn_jvp_proj) on this projection workload")
    ap.add_argument("--norm-rope", default=None,
                    help="time the RMS normalisation + rotary embedding of queries/keys (attn_jvp_rmsnorm_rope) "
                         "on this workload")
    ap.add_argument("--no-per-workload", action="store_true",
                    help="skip timing the other attention workloads (the per_workload object)")
    ap.add_argument("--trace-summary", default=None, metavar="DIR",
                    help="print per-kernel statistics of the rocprofv3 CSV output under DIR as JSON and exit")
    ap.add_argument("--skip", type=int, default=0,
                    help="with --trace-summary: dispatches of each kernel left out at the start (warm-ups)")
    ap.add_argument("--kernel", default="", help="with --trace-summary: only kernels whose name contains this")
    args = ap.parse_args()

    if args.trace_summary is not None:
        print(json.dumps(trace_summary(args.trace_summary, args.skip, args.kernel)))
        return

    if args.split and not 1 <= args.split <= 16:
        print("bench.py: --split must be in 1 .. 16 (ATTN_JVP_MAX_MERGE_PARTS)", file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(f"bench.py: this library runs on one GPU; --gpus {args.gpus} is not supported "
              "(the attention JVP shards by (batch, head) with no exchange: run one process per GPU)",
              file=sys.stderr)
        sys.exit(2)

    if args.norm_rope is not None:
        from workloads import NORM_ROPE_WORKLOADS

        if args.norm_rope not in NORM_ROPE_WORKLOADS or args.split or args.frozen_context or args.proj:
            print(f"bench.py: --norm-rope takes one of {sorted(NORM_ROPE_WORKLOADS)} (alone)", file=sys.stderr)
            sys.exit(2)
        bench_norm_rope(args)
        return

    if args.proj is not None:
        from workloads import PROJ_WORKLOADS

        if args.proj not in PROJ_WORKLOADS or args.split or args.frozen_context:
            print(f"bench.py: --proj takes one of {sorted(PROJ_WORKLOADS)} (without --split or --frozen-context)",
                  file=sys.stderr)
            sys.exit(2)
        bench_proj(args)
        return

    import torch

    import attention_forward_mode_attn_amd as A
    from workloads.device import device_inputs

    w = WORKLOADS[args.workload]
    if args.frozen_context and (w.std.get("tk", 1.0) != 0.0 or w.std.get("tv", 1.0) != 0.0):
        print(f"bench.py: --frozen-context needs a workload with tK = tV = 0 ({w.name} has key tangents)",
              file=sys.stderr)
        sys.exit(2)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(args.warmup + args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": args.warmup + args.steps}))
        return

    print(f"bench: {w.name} B{w.B} H{w.H} Lq{w.Lq} Lk{w.Lk} d{w.d} {w.dtype}: generating inputs",
          file=sys.stderr, flush=True)
    x = device_inputs(w)
    o = torch.empty_like(x["q"])
    to = torch.empty_like(x["q"])
    lse = torch.empty((w.B, w.H, w.Lq), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    tk, tv = (None, None) if args.frozen_context else (x["tk"], x["tv"])
    if args.split:
        bounds = A.shard_bounds(w.Lk, args.split)
        pdt = torch.float32 if args.f32_partials else o.dtype
        parts = [(torch.empty(o.shape, dtype=pdt, device=dev), torch.empty(o.shape, dtype=pdt, device=dev),
                  torch.empty_like(lse), torch.empty_like(lse)) for _ in bounds]
        tlse = torch.empty_like(lse)
        merge_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                    for _ in range(args.warmup + args.steps)]
        n_step = [0]

    def step():
        if not args.split:
            A.fwd(x["q"], x["k"], x["v"], x["tq"], tk, tv, scale=w.scale, out=(o, to, lse), stream=stream)
            return
        for (k0, k1), part in zip(bounds, parts):
            A.fwd_part(x["q"], x["k"], x["v"], x["tq"], tk, tv, k0, k1, scale=w.scale, out=part, stream=stream,
                       f32_out=args.f32_partials)
        a, b = merge_ev[n_step[0]]
        n_step[0] += 1
        a.record(stream)
        A.merge(parts, out=(o, to, lse, tlse), stream=stream, out_dtype=o.dtype)
        b.record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    per = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    print(f"bench: timing {args.steps} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for a, b in per:
        a.record(stream)
        step()
        b.record(stream)
    ev1.record(stream)
    sclk = wait_sampling_sclk(sclk_path(torch), ev1)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = ev0.elapsed_time(ev1)
    launch_ms = sorted(a.elapsed_time(b) for a, b in per)
    avg_launch_ms = sum(launch_ms) / len(launch_ms)
    ms_per_step = total_ms / args.steps

    # executed work: the frozen-context path skips the tK Q^T and tV P^T products
    flops = w.flops * (8.0 / 12.0 if args.frozen_context else 1.0)
    value = flops / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    achieved = flops / (avg_launch_ms * 1e-3) / 1e12
    if args.split:
        # the merge launch: n partial (O, tO, lse, tlse) rows read, one written
        timed = merge_ev[args.warmup:]
        merge_ms = sorted(a.elapsed_time(b) for a, b in timed)
        avg_merge_ms = sum(merge_ms) / len(merge_ms)
        rows = w.B * w.H * w.Lq
        part_bytes = 2 * w.d * (4 if args.f32_partials else w.elem_bytes) + 8
        merge_bytes = float(rows * (part_bytes * len(bounds) + 2 * w.d * w.elem_bytes + 8))
        roofline = {
            "bound": "hbm",
            "achieved": round(merge_bytes / (avg_merge_ms * 1e-3) / 1e9, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(merge_bytes / (avg_merge_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "traffic": None,
            "kernel": (f"merge_kernel<{str(w.dtype == 'bf16' and not args.f32_partials).lower()}, "
                       f"{str(w.dtype == 'bf16').lower()}, {w.d}>"),
            "avg_launch_ms": round(avg_merge_ms, 4),
            "median_launch_ms": round(merge_ms[len(merge_ms) // 2], 4),
            "min_launch_ms": round(merge_ms[0], 4),
            "algorithmic_bytes_per_launch": merge_bytes,
            "shard_bounds": bounds,
        }
    else:
        roofline = {
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(achieved / peak, 4),
            "traffic": None if args.frozen_context else measured_traffic(w.name),
            "kernel": (f"attn_jvp_bf16_kernel<{w.d}, {str(args.frozen_context).lower()}>" if w.dtype == "bf16"
                       else f"attn_jvp_fp32_kernel<{w.d}>"),
            "avg_launch_ms": round(avg_launch_ms, 4),
            "median_launch_ms": round(launch_ms[len(launch_ms) // 2], 4),
            "min_launch_ms": round(launch_ms[0], 4),
            "algorithmic_flops_per_launch": flops,
            "algorithmic_bytes_per_launch": w.algorithmic_bytes,
        }
    out = {
        "metric": METRIC_FROZEN if args.frozen_context else METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) inputs of the workload's shape)",
        "config": {"workload": w.name, "B": w.B, "H": w.H, "Lq": w.Lq, "Lk": w.Lk, "d": w.d,
                   "scale": w.scale, "parallelism": "single GPU",
                   "path": ("frozen context (tk = tv = NULL; 8 executed flops per logit and head dim)"
                            if args.frozen_context else "full JVP (12 flops per logit and head dim)")
                   + (f"; {args.split} key shards + exact merge" if args.split else "")
                   + ("; float32 partials" if args.split and args.f32_partials else "")},
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "wall_s_timed_region": round(wall, 3),
        "sclk_mhz": sclk,
        "roofline": roofline,
    }
    if args.workload == "video_self_bf16" and not (args.split or args.frozen_context or args.no_per_workload):
        del x, o, to, lse
        out["per_workload"] = per_workload()
    if not args.no_cpu_baseline:
        print("bench: timing the fp64 oracle on sampled rows (cpu_baseline)", file=sys.stderr, flush=True)
        cb = cpu_baseline(w, args.cpu_budget, args.cpu_rows_per_head)
        cb.pop("_np", None)
        out["cpu_baseline"] = cb
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
