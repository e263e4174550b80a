"""GPU parity on seeded random shapes, away from the hand-picked cases: the
attention pass (both dtypes, d 64/128, sometimes a frozen context, sometimes
split into key shards and merged) and the projection (with and without
tangent and bias), every output row against the fp64 oracle.
"""
import numpy as np
import pytest
import torch

from oracle import projection_jvp
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


def attention_cases(n=24, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        B, H = int(rng.integers(1, 4)), int(rng.integers(1, 5))
        Lq, Lk = int(rng.integers(1, 700)), int(rng.integers(1, 900))
        d = int(rng.choice([64, 128]))
        dtype = str(rng.choice(["bf16", "fp32"], p=[0.7, 0.3]))
        frozen = bool(rng.random() < 0.3)
        n_split = int(rng.choice([1, 1, 2, 3, 4])) if Lk >= 4 else 1
        out.append((i, B, H, Lq, Lk, d, dtype, frozen, n_split))
    return out


@pytest.mark.parametrize("i,B,H,Lq,Lk,d,dtype,frozen,n_split", attention_cases())
def test_attention_random_shape(A, i, B, H, Lq, Lk, d, dtype, frozen, n_split):
    std = {"q": 1.0, "k": 1.0, "v": 1.0, "tq": 1.0, "tk": 0.0 if frozen else 1.0, "tv": 0.0 if frozen else 1.0}
    w = custom_workload(B, H, Lq, Lk, d, dtype, seed_id=9000 + i, std=std)
    print(f"case random attention {i}: B{B} H{H} Lq{Lq} Lk{Lk} d{d} {dtype} frozen={frozen} split={n_split}",
          flush=True)
    x = device_inputs(w)
    tk, tv = (None, None) if frozen else (x["tk"], x["tv"])
    if n_split == 1:
        o, to, lse = A.fwd(x["q"], x["k"], x["v"], x["tq"], tk, tv, scale=w.scale)
    else:
        o, to, lse, _ = A.fwd_split(x["q"], x["k"], x["v"], x["tq"], tk, tv, n_split, scale=w.scale)
    torch.cuda.synchronize()
    res = compare(w, o, to, lse)
    print(f"  O {res['O']:.3e} tO {res['tO']:.3e} lse {res['lse']:.3e}", flush=True)
    assert res["O"] <= TOL[dtype] and res["tO"] <= TOL[dtype] and res["lse"] <= LSE_TOL[dtype]


def projection_cases(n=12, seed=20261204):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        out.append((i, int(rng.integers(1, 4)), int(rng.integers(1, 400)), 64 * int(rng.integers(1, 11)),
                    int(rng.integers(1, 4)), int(rng.integers(1, 5)), int(rng.choice([64, 128])),
                    bool(rng.random() < 0.7), bool(rng.random() < 0.7)))
    return out


@pytest.mark.parametrize("i,B,L,D,n_out,H,d,tangent,bias", projection_cases())
def test_projection_random_shape(A, i, B, L, D, n_out, H, d, tangent, bias):
    w = custom_proj(B, L, D, n_out, H, d, tangent=tangent, bias=bias, seed_id=9100 + i)
    print(f"case random projection {i}: B{B} L{L} D{D} n_out{n_out} H{H} d{d} tangent={tangent} bias={bias}",
          flush=True)
    h = proj_host_inputs(w)
    x = device_proj_inputs(w)
    y, ty = A.proj(x["x"], x["tx"], x["w"], x["bias"], n_out=n_out, heads=H)
    torch.cuda.synchronize()
    Y, TY = projection_jvp(h["x"], h["tx"], h["w"], h["bias"], n_out, H, d)
    for got, ref in ((y, Y), (ty, TY)):
        if ref is None:
            assert got is None
            continue
        err = np.abs(got.float().cpu().numpy() - ref)
        assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 2e-4 * np.abs(ref).max()), float(err.max())


def distribution_cases(n=24, seed=20261205):
    """Seeded shapes with varied value distributions: operand std (logit std is
    its square at the default scale), tangent std, softmax scale, key shards up
    to 16, and fp32 over long key ranges."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        dtype = str(rng.choice(["bf16", "fp32"]))
        d = int(rng.choice([64, 128]))
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
        Lq = int(rng.integers(1, 600))
        Lk = int(rng.integers(1, 9000 if dtype == "fp32" else 12000))
        sq = float(rng.choice([0.3, 1.0, 2.0] if dtype == "fp32" else [0.3, 1.0, 2.0, 2.83]))
        st = float(rng.choice([0.01, 0.5, 1.0, 10.0]))
        scale = float(10 ** rng.uniform(-2.5, -0.5))
        n_split = int(rng.choice([1, 1, 2, 5, 16])) if Lk >= 16 else 1
        frozen = bool(rng.random() < 0.25)
        out.append((i, B, H, Lq, Lk, d, dtype, sq, st, scale, n_split, frozen))
    return out


@pytest.mark.parametrize("i,B,H,Lq,Lk,d,dtype,sq,st,scale,n_split,frozen", distribution_cases())
def test_attention_random_distribution(A, i, B, H, Lq, Lk, d, dtype, sq, st, scale, n_split, frozen):
    std = {"q": sq, "k": sq, "v": 1.0, "tq": st, "tk": 0.0 if frozen else st, "tv": 0.0 if frozen else st}
    w = custom_workload(B, H, Lq, Lk, d, dtype, seed_id=9500 + i, std=std)
    # the oracle reads the softmax scale from the workload: give this one its own
    w = _with_scale(w, scale)
    print(f"case random distribution {i}: B{B} H{H} Lq{Lq} Lk{Lk} d{d} {dtype} sq={sq} st={st} "
          f"scale={scale:.4g} split={n_split} frozen={frozen}", flush=True)
    x = device_inputs(w)
    tk, tv = (None, None) if frozen else (x["tk"], x["tv"])
    if n_split == 1:
        o, to, lse = A.fwd(x["q"], x["k"], x["v"], x["tq"], tk, tv, scale=scale)
    else:
        o, to, lse, _ = A.fwd_split(x["q"], x["k"], x["v"], x["tq"], tk, tv, n_split, scale=scale)
    torch.cuda.synchronize()
    res = compare(w, o, to, lse)
    print(f"  O {res['O']:.3e} tO {res['tO']:.3e} lse {res['lse']:.3e}", flush=True)
    assert res["O"] <= TOL[dtype] and res["tO"] <= TOL[dtype] and res["lse"] <= LSE_TOL[dtype]


def _with_scale(w, scale):
    """A copy of workload ``w`` whose softmax scale is ``scale``."""
    import copy

    class Scaled(type(w)):
        @property
        def scale(self):
            return self._scale

    w2 = copy.copy(w)
    object.__setattr__(w2, "__class__", Scaled)
    object.__setattr__(w2, "_scale", scale)
    return w2
