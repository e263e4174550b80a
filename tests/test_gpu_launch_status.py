"""GPU: each entry point reports the status of its own launch.

An error that an unrelated earlier HIP call left pending on the calling thread
(here an invalid hipSetDevice) must neither fail a correct launch nor be
consumed by it: the call returns ATTN_JVP_OK, the caller still finds its own
error pending afterwards (read here with hipGetLastError, which also clears it
before torch's next call would report it), and the outputs match the oracle.
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


HIP_ERROR_INVALID_DEVICE = 101


def _hip():
    hip = ctypes.CDLL("libamdhip64.so.7")  # the runtime torch and the library share
    hip.hipSetDevice.argtypes = [ctypes.c_int]
    hip.hipSetDevice.restype = ctypes.c_int
    hip.hipGetLastError.argtypes = []
    hip.hipGetLastError.restype = ctypes.c_int
    return hip


def leave_pending_error():
    """A failed HIP call on this thread: hipSetDevice with an ordinal far past
    the device count returns hipErrorInvalidDevice and changes nothing else."""
    hip = _hip()
    hip.hipGetLastError()  # start from a clean state
    rc = hip.hipSetDevice(9999)
    assert rc == HIP_ERROR_INVALID_DEVICE, rc


def pending_error_survived():
    """The planted error is still the thread's last error (and is cleared now)."""
    return _hip().hipGetLastError() == HIP_ERROR_INVALID_DEVICE


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_pending_error_does_not_fail_attention(A, dtype):
    w = custom_workload(1, 2, 150, 90, 64, dtype, seed_id=5151)
    print(f"case pending-error fwd {w.name} {dtype}", flush=True)
    x = device_inputs(w)
    o, to = torch.empty_like(x["q"]), torch.empty_like(x["q"])
    lse = torch.empty((w.B, w.H, w.Lq), dtype=torch.float32, device=x["q"].device)
    torch.cuda.synchronize()
    leave_pending_error()
    A.fwd(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], scale=w.scale, out=(o, to, lse))  # raises if not OK
    assert pending_error_survived()
    torch.cuda.synchronize()
    res = compare(w, o, to, lse)
    assert res["O"] <= TOL[dtype] and res["tO"] <= TOL[dtype] and res["lse"] <= LSE_TOL[dtype], res


def test_pending_error_does_not_fail_merge_or_projection(A):
    w = custom_workload(1, 2, 130, 200, 128, "bf16", seed_id=5152)
    print(f"case pending-error split+merge {w.name}", flush=True)
    x = device_inputs(w)
    bounds = A.shard_bounds(w.Lk, 3)
    lse_shape = (w.B, w.H, w.Lq)

    def four():
        return (torch.empty_like(x["q"]), torch.empty_like(x["q"]),
                torch.empty(lse_shape, dtype=torch.float32, device=x["q"].device),
                torch.empty(lse_shape, dtype=torch.float32, device=x["q"].device))

    parts = [four() for _ in bounds]
    merged = four()
    torch.cuda.synchronize()
    for (k0, k1), part in zip(bounds, parts):
        leave_pending_error()
        A.fwd_part(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], k0, k1, scale=w.scale, out=part)
        assert pending_error_survived()
    leave_pending_error()
    A.merge(parts, out=merged)
    assert pending_error_survived()
    torch.cuda.synchronize()
    o, to, lse, _ = merged
    res = compare(w, o, to, lse)
    assert res["O"] <= TOL["bf16"] and res["tO"] <= TOL["bf16"], res

    from oracle import projection_jvp

    pw = custom_proj(1, 70, 128, 3, 2, 64, seed_id=5153)
    print(f"case pending-error projection {pw.name}", flush=True)
    h = proj_host_inputs(pw)
    xp = device_proj_inputs(pw, device="cuda:0")
    y = torch.empty((3, 1, 2, 70, 64), dtype=torch.bfloat16, device="cuda:0")
    ty = torch.empty_like(y)
    torch.cuda.synchronize()
    leave_pending_error()
    A.proj(xp["x"], xp["tx"], xp["w"], xp["bias"], n_out=3, heads=2, out=(y, ty))
    assert pending_error_survived()
    torch.cuda.synchronize()
    Y, TY = projection_jvp(h["x"], h["tx"], h["w"], h["bias"], 3, 2, 64)
    for got, ref in ((y, Y), (ty, TY)):
        err = np.abs(got.float().cpu().numpy() - ref)
        assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 2e-4 * np.abs(ref).max())
