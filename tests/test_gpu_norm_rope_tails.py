"""GPU: the normalisation/rotary kernel at every length up to 70, against its oracle.

The kernel spreads one row over d*e/16 lanes and a workgroup over 2048/d rows
(bf16) or 1024/d (float32); rows past L leave before the row shuffles.  This
sweep covers every length 1 .. 70 (past two workgroups of the bf16 d = 64
layout), over two heads, both head dims and element types, toggling the
tangent, the gain and the rotation from case to case; every element is checked
against the bound of the module's other tests (2^-8 |ref| + 2e-5 max|ref| for
bf16, 1e-5 max|ref| for float32).
"""
import numpy as np
import pytest
import torch

from oracle import norm_rope_jvp
from workloads import custom_norm_rope, norm_rope_array, rope_tables
from workloads.device import device_norm_rope_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def A():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_forward_mode_attn_amd as A

    A.load_library()
    return A


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("fp32", 64), ("fp32", 128)])
def test_every_length(A, dtype, d):
    bad = []
    for L in range(1, 71):
        tangent, gain, rope = L % 2 == 1, L % 3 != 0, L % 5 != 0
        w = custom_norm_rope(1, 2, L, d, dtype, tangent=tangent, rope=rope, gain=gain, seed_id=9100 + L)
        print(f"case norm_rope tail L{L} d{d} {dtype} tangent={tangent} gain={gain} rope={rope}", flush=True)
        x = device_norm_rope_inputs(w)
        y, ty = A.rmsnorm_rope(x["x"], x["tx"], x["gamma"], x["cos"], x["sin"], eps=w.eps)
        torch.cuda.synchronize()
        c, s = rope_tables(w)
        g = norm_rope_array(w, "gamma") if gain else None
        for h in range(2):
            Y, TY = norm_rope_jvp(norm_rope_array(w, "x", 0, h),
                                  norm_rope_array(w, "tx", 0, h) if tangent else None, g, c, s, w.eps)
            for got, ref in ((y[0, h], Y), (ty[0, h] if tangent else None, TY)):
                if ref is None:
                    continue
                err = np.abs(got.float().cpu().numpy().astype(np.float64) - ref)
                bound = (2.0 ** -8 * np.abs(ref) + 2e-5 * np.abs(ref).max()) if dtype == "bf16" \
                    else 1e-5 * np.abs(ref).max()
                if not np.all(err <= bound):
                    print(f"  h{h}: max error {err.max():.3e}", flush=True)
                    bad.append((L, h))
    assert not bad, bad[:10]
