"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU, no GPU).

attn_jvp_api.hip holds only host code: it is compiled here as plain C++ with
g++, linked against stub launchers that record the problem they would launch
(tests/abi_sanitize/), and driven by abi_check.cpp over the argument matrix of
the header's limits, one past them and 64-bit extremes.  Any signed overflow,
out-of-bounds read of the caller's pointer arrays, or other undefined
behaviour aborts the run.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "abi_sanitize")
CSRC = os.path.join(ROOT, "attention_forward_mode_attn_amd", "csrc")


def test_c_abi_host_code_is_clean_under_asan_and_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None or not os.path.isdir("/opt/rocm/include"):
        pytest.skip("needs g++ and the HIP headers")
    # the product source, as C++ (it has no device code)
    api = tmp_path / "attn_jvp_api.cpp"
    shutil.copy(os.path.join(CSRC, "attn_jvp_api.hip"), api)
    exe = tmp_path / "abi_check"
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I/opt/rocm/include", f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}", f"-I{HERE}",
           str(api), os.path.join(HERE, "stub_launch.cpp"), os.path.join(HERE, "abi_check.cpp"),
           "-pthread", "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300, env=env)
    print(r.stdout[-3000:])
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "ALL OK" in r.stdout
