"""The bench line's JSON contract, checked on small runs on the GPU (one
process per bench run, as the benchmark is used): the required keys and
types, a roofline object whose fraction is achieved / peak, and a CPU
baseline that names its sample and thread count."""
import json
import os
import subprocess
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def bench(*args):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("case bench", " ".join(args), flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                       timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout
    return json.loads(lines[0])


def check_common(d, steps, warmup, workload, dtype):
    for k, t in (("metric", str), ("value", float), ("unit", str), ("n_gpus", int), ("steps", int),
                 ("warmup", int), ("ms_per_step", float), ("higher_is_better", bool), ("scaling", str),
                 ("dtype", str), ("data", str), ("config", dict), ("roofline", dict)):
        assert isinstance(d[k], t), (k, d.get(k))
    assert "vs_baseline" in d and d["vs_baseline"] is None
    assert d["n_gpus"] == 1 and d["steps"] == steps and d["warmup"] == warmup
    assert d["higher_is_better"] is True and d["scaling"] in ("weak", "strong")
    assert d["dtype"] == dtype and d["config"]["workload"] == workload
    assert d["value"] > 0 and d["ms_per_step"] > 0
    rf = d["roofline"]
    assert rf["bound"] in ("mfma", "hbm", "alu") and rf["unit"] in ("TFLOP/s", "GB/s")
    assert rf["achieved"] > 0 and rf["peak"] > 0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert "traffic" in rf


def test_attention_bench_line():
    d = bench("--workload", "tiny_self_fp32", "--steps", "3", "--warmup", "1", "--cpu-budget", "2")
    check_common(d, 3, 1, "tiny_self_fp32", "fp32")
    assert d["roofline"]["peak"] == 157.3
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]


def test_projection_bench_line():
    d = bench("--proj", "kv_text_frozen_bf16", "--steps", "3", "--warmup", "1", "--cpu-budget", "2")
    check_common(d, 3, 1, "kv_text_frozen_bf16", "bf16")
    assert d["roofline"]["peak"] == 2500.0
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]


def test_split_bench_line_reports_the_merge():
    d = bench("--workload", "text_cross_bf16", "--split", "4", "--steps", "3", "--warmup", "1", "--no-cpu-baseline")
    check_common(d, 3, 1, "text_cross_bf16", "bf16")
    assert d["roofline"]["bound"] == "hbm" and d["roofline"]["unit"] == "GB/s"
    assert "cpu_baseline" not in d


def test_default_bench_line_carries_every_workload():
    """The default run (the video self-attention headline) also times the other
    attention workloads and reports each under per_workload."""
    d = bench("--steps", "2", "--warmup", "1", "--no-cpu-baseline")
    check_common(d, 2, 1, "video_self_bf16", "bf16")
    pw = d["per_workload"]
    assert sorted(pw) == ["image_self_bf16", "text_cross_bf16", "text_cross_bf16_frozen", "tiny_self_fp32",
                          "video_cross_stress_bf16"]
    for name, e in pw.items():
        assert e["launches"] >= 10 and e["avg_launch_ms"] > 0 and e["tflops"] > 0, name
        assert abs(e["frac"] - e["tflops"] / e["peak"]) < 1e-3, name
        assert abs(e["tflops"] - e["flops_per_launch"] / (e["avg_launch_ms"] * 1e-3) / 1e12) < 1e-2 * e["tflops"]
    assert pw["tiny_self_fp32"]["peak"] == 157.3 and pw["image_self_bf16"]["peak"] == 2500.0
    assert pw["text_cross_bf16_frozen"]["flops_per_launch"] * 1.5 == pw["text_cross_bf16"]["flops_per_launch"]


def test_norm_rope_bench_line():
    d = bench("--norm-rope", "q_image_bf16", "--steps", "3", "--warmup", "1", "--cpu-budget", "1")
    check_common(d, 3, 1, "q_image_bf16", "bf16")
    assert d["roofline"]["bound"] == "hbm" and d["roofline"]["peak"] == 8000.0
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1 and cb["sample"]
