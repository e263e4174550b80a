"""bench.py argument guard rails (CPU): runs that this build does not support
exit with status 2 and a message before touching a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_frozen_context_needs_zero_key_tangents():
    r = bench("--workload", "video_self_bf16", "--frozen-context")
    assert r.returncode == 2
    assert "tK = tV = 0" in r.stderr


def test_split_part_count_is_checked():
    r = bench("--split", "17")
    assert r.returncode == 2
    assert "--split" in r.stderr


def test_projection_workload_is_checked():
    r = bench("--proj", "no_such_projection")
    assert r.returncode == 2
    assert "qkv_video_bf16" in r.stderr
    r = bench("--proj", "qkv_video_bf16", "--split", "2")
    assert r.returncode == 2


def test_sclk_parsing_and_sampling(tmp_path):
    """The shader clock is the entry marked '*' of pp_dpm_sclk, in either of its
    layouts (a separate current-clock line, or a marked level); the sampler
    summarises what it read while the event was pending."""
    sys.path.insert(0, ROOT)
    import bench

    f = tmp_path / "pp_dpm_sclk"
    f.write_text("S: 1843Mhz *\n0: 500Mhz\n1: 2400Mhz\n")
    assert bench.read_sclk_mhz(str(f)) == 1843
    f.write_text("0: 500Mhz\n1: 1500Mhz *\n2: 2100Mhz\n")
    assert bench.read_sclk_mhz(str(f)) == 1500
    f.write_text("0: 500Mhz\n1: 2400Mhz\n")
    assert bench.read_sclk_mhz(str(f)) is None
    assert bench.read_sclk_mhz(str(tmp_path / "missing")) is None

    class Pending:
        def __init__(self, n):
            self.n = n

        def query(self):
            self.n -= 1
            return self.n < 0

    f.write_text("S: 1700Mhz *\n")
    s = bench.wait_sampling_sclk(str(f), Pending(3), period_s=0.0, min_samples=3)
    assert s["samples"] == 3 and s["median"] == s["min"] == s["max"] == 1700
    assert bench.wait_sampling_sclk(str(f), Pending(2), period_s=0.0, min_samples=3) is None  # too short a run
    assert bench.wait_sampling_sclk(None, Pending(3), period_s=0.0) is None
    assert bench.wait_sampling_sclk(str(f), Pending(0), period_s=0.0) is None


def test_trace_summary_skips_warmups(tmp_path):
    """--trace-summary reads rocprofv3's kernel-trace and counter CSVs and
    leaves out the first --skip dispatches of each kernel."""
    sys.path.insert(0, ROOT)
    import bench

    d = tmp_path / "host" / "run"
    d.mkdir(parents=True)
    hdr = "Kind,Agent_Id,Queue_Id,Dispatch_Id,Kernel_Id,Kernel_Name,Start_Timestamp,End_Timestamp\n"
    rows = [(1, "k<a>", 0, 900), (2, "other", 0, 5), (3, "k<a>", 1000, 1100), (4, "k<a>", 2000, 2120),
            (5, "k<a>", 3000, 3110)]
    (d / "run_kernel_trace.csv").write_text(
        hdr + "".join(f"KERNEL_DISPATCH,1,1,{i},7,\"{n}\",{s},{e}\n" for i, n, s, e in rows))
    chdr = "Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value,Start_Timestamp,End_Timestamp\n"
    crow = [(1, "k<a>", "X", 3.0, 0, 50), (1, "k<a>", "X", 4.0, 0, 50), (3, "k<a>", "X", 5.0, 60, 80)]
    (d / "run_counter_collection.csv").write_text(
        chdr + "".join(f"{i},\"{n}\",{c},{v},{s},{e}\n" for i, n, c, v, s, e in crow))
    out = bench.trace_summary(str(tmp_path), skip=1, kernel_filter="k<")
    k = out["kernel_trace"]["k<a>"]
    assert k["dispatches"] == 4 and k["counted"] == 3 and k["durations_ns"] == [100, 120, 110]
    assert k["avg_ns"] == 110 and k["min_ns"] == 100 and k["max_ns"] == 120
    assert "other" not in out["kernel_trace"]
    c = out["counters"]["k<a>"]
    assert c == [{"dispatch": 3, "X": 5.0, "_duration_ns": 20}]


def test_norm_rope_workload_is_checked():
    r = bench("--norm-rope", "nope")
    assert r.returncode == 2
    assert "q_video_bf16" in r.stderr


def test_projection_kernel_name_follows_the_tile_switch():
    """The bench line names the projection instantiation a launch runs: 128-feature
    tiles when the 256-feature grid has at most 128 workgroups (without a
    tangent only when D % 128 == 0), else 256-feature tiles."""
    import bench
    from workloads import PROJ_WORKLOADS, custom_proj

    assert bench.proj_kernel_name(PROJ_WORKLOADS["qkv_video_bf16"]) == "proj_bf16_kernel<true, 256, 64>"
    assert bench.proj_kernel_name(PROJ_WORKLOADS["qkv_image_bf16"]) == "proj_bf16_kernel<true, 256, 64>"
    assert bench.proj_kernel_name(PROJ_WORKLOADS["kv_text_frozen_bf16"]) == "proj_bf16_kernel<false, 128, 128>"
    # 42 token tiles x 3 feature tiles = 126 workgroups: narrow; 43 x 3 = 129: wide
    assert bench.proj_kernel_name(custom_proj(1, 5376, 64, 3, 2, 128)) == "proj_bf16_kernel<true, 128, 64>"
    assert bench.proj_kernel_name(custom_proj(1, 5504, 64, 3, 2, 128)) == "proj_bf16_kernel<true, 256, 64>"
    assert bench.proj_kernel_name(custom_proj(1, 200, 192, 2, 2, 64, tangent=False)) == \
        "proj_bf16_kernel<false, 256, 64>"
