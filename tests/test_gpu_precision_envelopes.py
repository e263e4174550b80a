"""GPU: the regimes at the edge of the precision of the bf16 path and of the
float32 key-shard path.

A seeded random sweep over all entry points (4400 cases, logit standard
deviations up to ~130) met every tolerance except in three regimes, all with
softmax rows that are effectively one-hot (scaled logits of standard deviation
65-130, |lse| in the hundreds).  Representative cases:

* bf16 rows whose weight sits on a few keys with tangent logits of tens: P and
  P*tS meet V as bf16 values; normalising O and tO by the fp32 sum of p left a
  mismatch of about 2^-9 |scale*tS| |V| (tO 2.1e-2 here).  The kernel now
  normalises by the sum of the bf16 weights the products consume, so the
  centring cancels for a dominant key; this case is checked at 2e-2;
* float32 key shards: each shard's lse is a float32, so the merge weights
  carry a relative error of about 2^-24 |lse|; with |lse| near 1000 the merged
  O and tO are off by 1-2e-5 (the unsplit pass stays far inside 1e-5): an
  expected failure with its measured error;
* one key: p = 2^y with y the rounding residual of the exponent, so p is 1
  only to within about 2^-24 |scale*S|; with a frozen context the exact tO is
  zero, so a relative error is undefined, and the computed one is a residual of
  that size (plus, in float32, a few roundings of |scale*tS| |v|): checked
  against that absolute bound.
"""
import numpy as np
import pytest
import torch

from workloads import custom_workload

from _parity import TOL, compare, device_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def A():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_forward_mode_attn_amd as A

    A.load_library()
    return A


def test_bf16_nearly_one_hot_rows_with_large_tangent_logits(A):
    # logit std ~66, |lse| ~450, |scale*tS| up to ~24 (key rows scaled up to 27x)
    std = {"q": 2.0, "k": 2.0, "v": 1.0, "tq": 0.1, "tk": 0.1, "tv": 0.1}
    w = custom_workload(1, 1, 71, 2654, 64, "bf16", seed_id=81843, std=std, key_ramp=0.01)
    print("case bf16 one-hot rows B1 H1 Lq71 Lk2654 d64 ramp0.01", flush=True)
    x = device_inputs(w)
    o, to, lse = A.fwd(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], scale=w.scale)
    torch.cuda.synchronize()
    res = compare(w, o, to, lse)
    print(f"  O {res['O']:.3e} tO {res['tO']:.3e} lse {res['lse']:.3e}", flush=True)
    assert res["O"] <= TOL["bf16"] and res["tO"] <= TOL["bf16"] and res["lse"] <= 1e-4


def test_float32_shards_at_large_lse(A):
    # logit std ~130, |lse| up to ~970, 8 key shards merged in fp32
    std = {"q": 3.0, "k": 3.0, "v": 1.0, "tq": 1.0, "tk": 1.0, "tv": 1.0}
    w = custom_workload(1, 1, 260, 2352, 64, "fp32", seed_id=80457, std=std, key_ramp=0.01)
    print("case fp32 8 shards B1 H1 Lq260 Lk2352 d64 ramp0.01", flush=True)
    x = device_inputs(w)
    o, to, lse = A.fwd(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], scale=w.scale)
    torch.cuda.synchronize()
    whole = compare(w, o, to, lse)
    o, to, lse, _ = A.fwd_split(x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"], 8, scale=w.scale)
    torch.cuda.synchronize()
    res = compare(w, o, to, lse)
    print(f"  unsplit O {whole['O']:.3e} tO {whole['tO']:.3e}; 8 shards O {res['O']:.3e} tO {res['tO']:.3e}",
          flush=True)
    assert whole["O"] <= TOL["fp32"] and whole["tO"] <= TOL["fp32"]
    assert res["O"] <= 1e-4 and res["tO"] <= 1e-4
    if res["O"] > TOL["fp32"] or res["tO"] > TOL["fp32"]:
        pytest.xfail(f"float32 shard lse at |lse| ~ 1000: O {res['O']:.2e}, tO {res['tO']:.2e} > 1e-5")


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("bf16", 128), ("fp32", 64)])
def test_single_key_frozen_context_residual(A, dtype, d):
    """One key and tK = tV = 0: the exact tO is zero.  The computed one is a
    rounding residual of two kinds.  p = 2^y is not exactly 1: y is the rounding
    residual of the exponent (the running maximum is kept in float32), about
    2^-24 |scale*S*log2 e|, and in bf16 the weights that meet V are bf16(p) while
    l sums p.  In float32, the products P*tS, P*V and (a/l)*(P*V) and the quotient
    a/l are each rounded once, a few units of 2^-24 |scale*tS| |v|.  Together:
    |tO| <= 2^-21 (1 + |scale*S|) |scale*tS| |v| per element."""
    std = {"q": 3.0, "k": 3.0, "v": 1.0, "tq": 5.0, "tk": 0.0, "tv": 0.0}
    w = custom_workload(2, 1, 384, 1, d, dtype, seed_id=81333 + d, std=std)
    print(f"case single key frozen B2 H1 Lq384 Lk1 d{d} {dtype}", flush=True)
    x = device_inputs(w)
    o, to, lse = A.fwd(x["q"], x["k"], x["v"], x["tq"], None, None, scale=w.scale)
    torch.cuda.synchronize()
    q, k, v, tq = (x[t].float().cpu().double() for t in ("q", "k", "v", "tq"))
    s = w.scale * (q @ k.transpose(-1, -2))[..., 0]          # [B, H, Lq]
    ts = w.scale * (tq @ k.transpose(-1, -2))[..., 0]
    bound = 2.0 ** -21 * ((1 + s.abs()) * ts.abs())[..., None] * v.abs()[..., 0:1, :] + 1e-30
    got = to.float().cpu().double().abs()
    print(f"  max |tO| {got.max().item():.3e}, max bound {bound.max().item():.3e}", flush=True)
    assert bool((got <= bound).all())
    assert torch.allclose(o.float().cpu().double(), v.expand_as(o.float()).double(), rtol=2.0 ** -7, atol=0)
