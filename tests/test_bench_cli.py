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
