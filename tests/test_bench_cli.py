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
