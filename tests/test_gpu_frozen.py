"""GPU parity of the frozen-context path (tk = tv = NULL: zero key-side
tangents, the text cross-attention case), through the C ABI.

The oracle runs on the same inputs with tK = tV = 0.  The frozen path skips
the tK Q^T and tV P^T products; on zero-filled tk, tv the full path adds exact
zeros to the same accumulators, so the two agree exactly.
"""
import pytest
import torch

from workloads import WORKLOADS, custom_workload, sample_rows

from _parity import LSE_TOL, TOL, compare, device_inputs

pytestmark = pytest.mark.gpu

FROZEN_STD = {"q": 1.0, "k": 1.0, "v": 1.0, "tq": 1.0, "tk": 0.0, "tv": 0.0}


@pytest.fixture(scope="module")
def A():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_forward_mode_attn_amd as A

    A.load_library()
    return A


def check(w, res, label):
    tol = TOL[w.dtype]
    extra = f" tlse {res['tlse']:.3e}" if "tlse" in res else ""
    print(f"  {label}: O {res['O']:.3e} tO {res['tO']:.3e} lse {res['lse']:.3e}{extra}", flush=True)
    assert res["O"] <= tol and res["tO"] <= tol, res
    assert res["lse"] <= LSE_TOL[w.dtype], res["lse"]
    if "tlse" in res:
        assert res["tlse"] <= tol, res["tlse"]


SHAPES = [
    # (B, H, Lq, Lk, d, dtype)
    (1, 1, 1, 1, 128, "bf16"),
    (2, 2, 257, 273, 128, "bf16"),
    (1, 3, 130, 200, 64, "bf16"),
    (1, 1, 300, 65, 128, "bf16"),
    (1, 2, 129, 7, 128, "fp32"),
    (2, 1, 200, 96, 64, "fp32"),
]


@pytest.mark.parametrize("B,H,Lq,Lk,d,dtype", SHAPES)
def test_frozen_context_matches_oracle_and_full_path(A, B, H, Lq, Lk, d, dtype):
    w = custom_workload(B, H, Lq, Lk, d, dtype, seed_id=4000 + Lq * 7 + Lk, std=FROZEN_STD)
    print(f"case frozen B{B} H{H} Lq{Lq} Lk{Lk} d{d} {dtype}", flush=True)
    x = device_inputs(w)
    o, to, lse = A.fwd(x["q"], x["k"], x["v"], x["tq"], None, None, scale=w.scale)
    o2, to2, lse2 = A.fwd(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], scale=w.scale)
    torch.cuda.synchronize()
    check(w, compare(w, o, to, lse), "frozen")
    assert torch.equal(o, o2) and torch.equal(to, to2) and torch.equal(lse, lse2)


def test_frozen_split_and_merge(A):
    w = custom_workload(1, 2, 200, 300, 128, "bf16", seed_id=4100, std=FROZEN_STD)
    print("case frozen split n3", flush=True)
    x = device_inputs(w)
    o, to, lse, tlse = A.fwd_split(x["q"], x["k"], x["v"], x["tq"], None, None, 3, scale=w.scale)
    torch.cuda.synchronize()
    check(w, compare(w, o, to, lse, tlse=tlse), "frozen, 3 shards")


def test_frozen_text_cross_config(A):
    """The text cross-attention workload (tK = tV = 0) on the frozen path."""
    w = WORKLOADS["text_cross_bf16"]
    print(f"case frozen {w.name}", flush=True)
    x = device_inputs(w)
    o, to, lse = A.fwd(x["q"], x["k"], x["v"], x["tq"], None, None, scale=w.scale)
    o2, to2, lse2 = A.fwd(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], scale=w.scale)
    torch.cuda.synchronize()
    rows = lambda b, h: sample_rows(w, b, h, n_random=64)  # noqa: E731
    check(w, compare(w, o, to, lse, rows_fn=rows), "text cross, frozen, sampled rows")
    assert torch.equal(o, o2) and torch.equal(to, to2) and torch.equal(lse, lse2)


def test_one_null_tangent_is_rejected(A):
    w = custom_workload(1, 1, 64, 64, 64, "bf16", seed_id=4200)
    x = device_inputs(w)
    with pytest.raises(ValueError):
        A.fwd(x["q"], x["k"], x["v"], x["tq"], None, x["tv"])
    o = torch.empty_like(x["q"])
    lse = torch.empty((1, 1, 64), dtype=torch.float32, device=o.device)
    st = A.attn_jvp_fwd(x["q"], x["k"], x["v"], x["tq"], x["tk"], None, o, o.clone(), lse, 1, 1, 64, 64, 64,
                        0.125, A.ATTN_JVP_BF16)
    assert st == A.ATTN_JVP_EINVAL
