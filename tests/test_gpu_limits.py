"""GPU parity at the size limits the C ABI states, where the 32-bit byte
offsets inside the kernels come closest to overflowing.

  * attention: Lq*d and Lk*d below 2^29 elements per head (bf16 at d = 128,
    and fp32 at d = 64, whose byte offsets then approach 2^31);
  * projection: L*D below 2^31 elements.

Each case checks sampled rows (both ends, the middle, seeded random rows)
against the fp64 oracle with the tolerances of the other parity tests.
"""
import numpy as np
import pytest
import torch

from oracle import projection_jvp
from workloads import bf16_bits_to_f32, custom_proj, custom_workload, proj_array, proj_upload

from _parity import LSE_TOL, TOL, compare, device_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def A():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_forward_mode_attn_amd as A

    A.load_library()
    return A


def rows_of(L, n_random=48, seed=0):
    """Rows 0-7, the 8 middle rows, the last 8 and n_random seeded rows of [0, L)."""
    fixed = set(range(min(8, L))) | set(range(max(0, L - 8), L))
    fixed |= set(r for r in range(L // 2 - 4, L // 2 + 4) if 0 <= r < L)
    rnd = np.random.default_rng(seed).choice(L, size=min(n_random, L), replace=False)
    return np.array(sorted(fixed | set(int(r) for r in rnd)), dtype=np.int64)


LIMIT_SHAPES = [
    # (Lq, Lk, d, dtype): the largest per-head sequence the ABI accepts (L*d = 2^29 - d)
    ((1 << 29) // 128 - 1, 97, 128, "bf16"),
    (1, (1 << 29) // 128 - 1, 128, "bf16"),
    ((1 << 29) // 64 - 1, 70, 64, "fp32"),
]


@pytest.mark.parametrize("Lq,Lk,d,dtype", LIMIT_SHAPES)
def test_attention_at_the_sequence_limit(A, Lq, Lk, d, dtype):
    w = custom_workload(1, 1, Lq, Lk, d, dtype, seed_id=8000 + d)
    print(f"case limit attention Lq{Lq} Lk{Lk} d{d} {dtype}", flush=True)
    assert Lq * d < (1 << 29) and Lk * d < (1 << 29)
    x = device_inputs(w)
    o, to, lse = A.fwd(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], scale=w.scale)
    torch.cuda.synchronize()
    del x
    rows = rows_of(Lq)
    res = compare(w, o, to, lse, rows_fn=lambda b, h: rows, threads=1)
    print(f"  O {res['O']:.3e} tO {res['tO']:.3e} lse {res['lse']:.3e}", flush=True)
    assert res["O"] <= TOL[dtype] and res["tO"] <= TOL[dtype] and res["lse"] <= LSE_TOL[dtype]


def test_projection_near_the_token_limit(A):
    """L*D = 2^31 - 8192 (the largest multiple of 64 under the limit at D = 8192),
    frozen input (the tangent shares the X addressing and is tested elsewhere)."""
    L, D = (1 << 18) - 1, 8192
    w = custom_proj(1, L, D, 1, 2, 128, tangent=False, bias=True, seed_id=8100)
    print(f"case limit projection L{L} D{D} (L*D = {L * D})", flush=True)
    assert L * D < (1 << 31)
    bits = proj_upload(w, "x", 0)  # generated once: 2.1e9 values
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to("cuda").view(1, L, D)
    wt = torch.from_numpy(proj_upload(w, "w").view(np.int16)).view(torch.bfloat16).to("cuda")
    bs = torch.from_numpy(proj_upload(w, "bias").view(np.int16)).view(torch.bfloat16).to("cuda")
    y, ty = A.proj(x, None, wt, bs, n_out=1, heads=2)
    torch.cuda.synchronize()
    assert ty is None
    del x
    rows = rows_of(L, seed=1)
    xr = bf16_bits_to_f32(bits[rows])[None]
    del bits
    Y, _ = projection_jvp(xr, None, proj_array(w, "w"), proj_array(w, "bias"), 1, 2, 128)
    got = y[:, :, :, torch.as_tensor(rows, device=y.device)].float().cpu().numpy()
    err = np.abs(got - Y)
    bound = 2.0 ** -8 * np.abs(Y) + 2e-4 * np.abs(Y).max()
    print(f"  Y: max err {err.max():.3e}, worst err/bound {(err / bound).max():.3f}", flush=True)
    assert np.all(err <= bound)
