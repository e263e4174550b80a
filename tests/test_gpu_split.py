"""GPU parity of the key-sharded path: attn_jvp_fwd_part (with the tangent of
lse, tlse) and the exact merge attn_jvp_merge, through the C ABI, against the
fp64 oracle over all keys.

A split result must equal the unsplit attention-JVP up to rounding: the merge
is exact algebra (the oracle's merge_shards, pinned on the CPU against the
full-key definition), so the tolerance is the spec one on O and tO, the
lse bound of the unsplit tests, and the O/tO bound on tlse (normalised max
error).  Shards are cut on 64-key tile boundaries where the length allows, and
include single-key and ragged shards.
"""
import numpy as np
import pytest
import torch

from workloads import WORKLOADS, custom_workload, sample_rows

from _parity import LSE_TOL, TOL, compare, device_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def A():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_forward_mode_attn_amd as A

    A.load_library()
    return A


def check(w, res, label):
    tol = TOL[w.dtype]
    print(f"  {label}: O {res['O']:.3e} tO {res['tO']:.3e} lse {res['lse']:.3e} tlse {res['tlse']:.3e}",
          flush=True)
    assert res["O"] <= tol, res["O"]
    assert res["tO"] <= tol, res["tO"]
    assert res["lse"] <= LSE_TOL[w.dtype], res["lse"]
    assert res["tlse"] <= tol, res["tlse"]


FULL = [
    # (B, H, Lq, Lk, d, dtype)
    (1, 2, 128, 128, 64, "fp32"),
    (2, 1, 65, 63, 64, "bf16"),
    (1, 2, 257, 273, 128, "bf16"),
    (1, 1, 130, 7, 128, "fp32"),
]


@pytest.mark.parametrize("B,H,Lq,Lk,d,dtype", FULL)
def test_part_over_all_keys_is_fwd_plus_tlse(A, B, H, Lq, Lk, d, dtype):
    w = custom_workload(B, H, Lq, Lk, d, dtype, seed_id=3000 + Lq * 7 + Lk)
    print(f"case part-full B{B} H{H} Lq{Lq} Lk{Lk} d{d} {dtype}", flush=True)
    x = device_inputs(w)
    args = (x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"])
    o, to, lse, tlse = A.fwd_part(*args, 0, Lk, scale=w.scale)
    o2, to2, lse2 = A.fwd(*args, scale=w.scale)
    torch.cuda.synchronize()
    # the same kernel with the same key range: identical bits
    assert torch.equal(o, o2) and torch.equal(to, to2) and torch.equal(lse, lse2)
    check(w, compare(w, o, to, lse, tlse=tlse), "part over all keys")


SPLITS = [
    # (B, H, Lq, Lk, d, dtype, n_split)
    (1, 2, 130, 200, 64, "bf16", 3),
    (2, 1, 65, 300, 128, "fp32", 2),
    (1, 1, 17, 5000, 128, "bf16", 4),
    (1, 2, 129, 65, 128, "bf16", 2),     # shards of 64 and 1 keys
    (1, 1, 64, 7, 64, "fp32", 7),        # single-key shards
    (1, 1, 200, 1024, 128, "bf16", 16),  # the most parts one merge takes
    (2, 4, 512, 512, 128, "bf16", 4),
]


@pytest.mark.parametrize("B,H,Lq,Lk,d,dtype,n", SPLITS)
def test_split_and_merge_matches_oracle(A, B, H, Lq, Lk, d, dtype, n):
    w = custom_workload(B, H, Lq, Lk, d, dtype, seed_id=3100 + Lq * 7 + Lk + n)
    print(f"case split B{B} H{H} Lq{Lq} Lk{Lk} d{d} {dtype} n{n} shards {A.shard_bounds(Lk, n)}", flush=True)
    x = device_inputs(w)
    o, to, lse, tlse = A.fwd_split(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], n, scale=w.scale)
    torch.cuda.synchronize()
    check(w, compare(w, o, to, lse, tlse=tlse), f"{n} shards merged")


def test_merge_of_one_part_is_the_part(A):
    w = custom_workload(1, 2, 200, 150, 128, "bf16", seed_id=3200)
    print("case merge n=1", flush=True)
    x = device_inputs(w)
    part = A.fwd_part(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], 0, 150, scale=w.scale)
    o, to, lse, tlse = A.merge([part])
    torch.cuda.synchronize()
    for got, ref in zip((o, to, lse, tlse), part):
        assert torch.equal(got, ref)


def test_merge_is_independent_of_part_order(A):
    w = custom_workload(1, 1, 100, 400, 64, "fp32", seed_id=3300)
    print("case merge order", flush=True)
    x = device_inputs(w)
    args = (x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"])
    parts = [A.fwd_part(*args, a, b, scale=w.scale) for a, b in A.shard_bounds(400, 3)]
    m1 = A.merge(parts)
    m2 = A.merge(parts[::-1])
    torch.cuda.synchronize()
    for a, b in zip(m1, m2):
        assert float((a - b).abs().max()) <= 1e-6 * max(1.0, float(b.abs().max()))


def test_split_on_text_cross_config(A):
    """The text cross-attention workload (Lk = 512) as 2 shards of 256 keys."""
    w = WORKLOADS["text_cross_bf16"]
    print(f"case split {w.name} n2", flush=True)
    x = device_inputs(w)
    o, to, lse, tlse = A.fwd_split(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], 2, scale=w.scale)
    torch.cuda.synchronize()
    rows = lambda b, h: sample_rows(w, b, h, n_random=64)  # noqa: E731
    check(w, compare(w, o, to, lse, rows_fn=rows, tlse=tlse), "text cross, 2 shards, sampled rows")
