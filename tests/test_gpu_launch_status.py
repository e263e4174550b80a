"""GPU: each entry point reports the status of its own launch.

An error that an unrelated earlier HIP call left pending on the calling thread
(here an invalid hipSetDevice) must neither fail a correct launch nor be
consumed by it: the call returns ATTN_JVP_OK and the outputs match the oracle.
"""
import ctypes

import numpy as np
import pytest
import torch

from workloads import custom_proj, custom_workload, proj_host_inputs
from workloads.device import device_proj_inputs

from _parity import LSE_TOL, TOL, compare, device_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def A():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_forward_mode_attn_amd as A

    A.load_library()
    return A


def leave_pending_error():
    """A failed HIP call on this thread: hipSetDevice with an ordinal far past
    the device count returns hipErrorInvalidDevice and changes nothing else."""
    hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch and the library share
    hip.hipSetDevice.argtypes = [ctypes.c_int]
    hip.hipSetDevice.restype = ctypes.c_int
    rc = hip.hipSetDevice(9999)
    assert rc != 0, "hipSetDevice(9999) unexpectedly succeeded"
    return hip


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_pending_error_does_not_fail_attention(A, dtype):
    w = custom_workload(1, 2, 150, 90, 64, dtype, seed_id=5151)
    print(f"case pending-error fwd {w.name} {dtype}", flush=True)
    x = device_inputs(w)
    torch.cuda.synchronize()
    leave_pending_error()
    o, to, lse = A.fwd(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], scale=w.scale)
    torch.cuda.synchronize()
    res = compare(w, o, to, lse)
    assert res["O"] <= TOL[dtype] and res["tO"] <= TOL[dtype] and res["lse"] <= LSE_TOL[dtype], res


def test_pending_error_does_not_fail_merge_or_projection(A):
    w = custom_workload(1, 2, 130, 200, 128, "bf16", seed_id=5152)
    print(f"case pending-error split+merge {w.name}", flush=True)
    x = device_inputs(w)
    torch.cuda.synchronize()
    leave_pending_error()
    o, to, lse, _ = A.fwd_split(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], 3, scale=w.scale)
    torch.cuda.synchronize()
    res = compare(w, o, to, lse)
    assert res["O"] <= TOL["bf16"] and res["tO"] <= TOL["bf16"], res

    from oracle import projection_jvp

    pw = custom_proj(1, 70, 128, 3, 2, 64, seed_id=5153)
    print(f"case pending-error projection {pw.name}", flush=True)
    h = proj_host_inputs(pw)
    xp = device_proj_inputs(pw, device="cuda:0")
    torch.cuda.synchronize()
    leave_pending_error()
    y, ty = A.proj(xp["x"], xp["tx"], xp["w"], xp["bias"], n_out=3, heads=2)
    torch.cuda.synchronize()
    Y, TY = projection_jvp(h["x"], h["tx"], h["w"], h["bias"], 3, 2, 64)
    for got, ref in ((y, Y), (ty, TY)):
        err = np.abs(got.float().cpu().numpy() - ref)
        assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 2e-4 * np.abs(ref).max())
