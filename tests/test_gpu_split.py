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


@pytest.mark.parametrize("d,frozen", [(128, False), (64, False), (128, True)])
def test_float32_outputs_of_a_bf16_pass(A, d, frozen):
    """dtype 2: the bf16 pass writes O and tO in float32.  O rounded to bf16 is
    the bf16 pass's O bit for bit (the same fp32 value, rounded to nearest
    even); tO rounded to bf16 is within one bf16 ulp of the bf16 pass's tO (the
    compiler may contract the epilogue's multiply-add differently in the two
    store paths); both match the oracle."""
    w = custom_workload(1, 2, 200, 300, d, "bf16", seed_id=3700 + d + frozen)
    print(f"case f32 outputs d{d} frozen={frozen}", flush=True)
    x = device_inputs(w)
    tk, tv = (None, None) if frozen else (x["tk"], x["tv"])
    o32, to32, lse32 = A.fwd(x["q"], x["k"], x["v"], x["tq"], tk, tv, scale=w.scale, f32_out=True)
    o, to, lse = A.fwd(x["q"], x["k"], x["v"], x["tq"], tk, tv, scale=w.scale)
    torch.cuda.synchronize()
    assert o32.dtype == torch.float32 and to32.dtype == torch.float32
    assert torch.equal(o32.to(torch.bfloat16), o) and torch.equal(lse32, lse)
    if frozen:
        w = custom_workload(1, 2, 200, 300, d, "bf16", seed_id=3700 + d + frozen,
                            std={"q": 1.0, "k": 1.0, "v": 1.0, "tq": 1.0, "tk": 0.0, "tv": 0.0})
    res32 = compare(w, o32, to32, lse32)
    res = compare(w, o, to, lse)
    print(f"  f32 out: O {res32['O']:.3e} tO {res32['tO']:.3e}; bf16 out: O {res['O']:.3e} tO {res['tO']:.3e}",
          flush=True)
    assert res32["O"] <= TOL["bf16"] and res32["tO"] <= TOL["bf16"] and res32["lse"] <= LSE_TOL["bf16"]
    t16 = to32.to(torch.bfloat16).float()
    ulp = torch.abs(to.float()) * 2.0 ** -7 + 1e-30
    assert bool((torch.abs(t16 - to.float()) <= ulp).all())


@pytest.mark.parametrize("n_split", [2, 4, 7])
def test_float32_partials_merge_no_worse_than_unsplit(A, n_split):
    """Key shards kept in float32 and rounded to bf16 once, by the merge.  The
    merged result carries the unsplit pass's kind of error: each shard rounds
    its own P to bf16 against its own exponent base, a different set of
    roundings of the same size, so the error equals the unsplit one only
    statistically (measured: equal at 4 and 7 shards, 9% above at 2).  bf16
    partials add a second rounding of O and tO on top (measured 15-35% more
    on tO).  Gate: the tolerance, within 15% of unsplit, and no worse than
    bf16 partials."""
    w = custom_workload(1, 3, 600, 2500, 128, "bf16", seed_id=3800 + n_split)
    print(f"case f32 partials {n_split} shards", flush=True)
    x = device_inputs(w)
    args = (x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"])
    o, to, lse = A.fwd(*args, scale=w.scale)
    om, tom, lsem, tlsem = A.fwd_split(*args, n_split, scale=w.scale, f32_partials=True)
    ob, tob, lseb, tlseb = A.fwd_split(*args, n_split, scale=w.scale)
    torch.cuda.synchronize()
    assert om.dtype == torch.bfloat16
    r0 = compare(w, o, to, lse)
    rm = compare(w, om, tom, lsem, tlse=tlsem)
    rb = compare(w, ob, tob, lseb, tlse=tlseb)
    print(f"  unsplit O {r0['O']:.3e} tO {r0['tO']:.3e} | f32 partials O {rm['O']:.3e} tO {rm['tO']:.3e} | "
          f"bf16 partials O {rb['O']:.3e} tO {rb['tO']:.3e}", flush=True)
    check(w, rm, "f32 partials")
    assert rm["O"] <= r0["O"] * 1.15 and rm["tO"] <= r0["tO"] * 1.15
    assert rm["O"] <= rb["O"] and rm["tO"] <= rb["tO"]


def test_float32_partials_on_text_cross_config(A):
    w = WORKLOADS["text_cross_bf16"]
    print(f"case {w.name} 4 shards, f32 partials (sampled rows)", flush=True)
    x = device_inputs(w)
    o, to, lse, tlse = A.fwd_split(x["q"], x["k"], x["v"], x["tq"], None, None, 4, scale=w.scale,
                                   f32_partials=True)
    torch.cuda.synchronize()
    check(w, compare(w, o, to, lse, rows_fn=lambda b, h: sample_rows(w, b, h), tlse=tlse), "text cross f32 parts")


def test_split_on_video_self_config(A):
    """The key-shard path at full size in the configuration `bench.py --split 4`
    times (4 shards of the 32760 keys, then the merge), with bf16 and with
    float32 partials, on sampled rows of every head (both edges of the first
    query tile, rows of the ragged tail tile, seeded random rows)."""
    w = WORKLOADS["video_self_bf16"]
    x = device_inputs(w)
    for f32_partials in (False, True):
        kind = "f32" if f32_partials else "bf16"
        print(f"case {w.name} 4 shards, {kind} partials (sampled rows)", flush=True)
        o, to, lse, tlse = A.fwd_split(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], 4, scale=w.scale,
                                       f32_partials=f32_partials)
        torch.cuda.synchronize()
        check(w, compare(w, o, to, lse, rows_fn=lambda b, h: sample_rows(w, b, h, n_random=24), tlse=tlse),
              f"video self {kind} parts")
        del o, to, lse, tlse


def test_cp_shard_config_unsplit_and_split(A):
    """One GPU's share of the video layer under head and query sharding (5
    heads, 4095 queries, 32760 keys; 160 workgroups): the single pass and the
    4-shard path on sampled rows of every head."""
    w = WORKLOADS["video_self_cp_shard_bf16"]
    x = device_inputs(w)
    print(f"case {w.name} single pass over all keys (sampled rows)", flush=True)
    o, to, lse, tlse = A.fwd_part(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], 0, w.Lk, scale=w.scale)
    torch.cuda.synchronize()
    check(w, compare(w, o, to, lse, rows_fn=lambda b, h: sample_rows(w, b, h, n_random=48), tlse=tlse), "cp shard")
    print(f"case {w.name} 4 shards (sampled rows)", flush=True)
    o, to, lse, tlse = A.fwd_split(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], 4, scale=w.scale)
    torch.cuda.synchronize()
    check(w, compare(w, o, to, lse, rows_fn=lambda b, h: sample_rows(w, b, h, n_random=48), tlse=tlse),
          "cp shard 4 parts")
