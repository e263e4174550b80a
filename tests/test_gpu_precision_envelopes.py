"""GPU: the regimes at the edge of the precision of the bf16 path and of the
float32 key-shard path.

Seeded random sweeps over all entry points (about 16000 cases, logit standard
deviations up to ~130) met every tolerance except in the regimes below, all
with softmax rows that are effectively one-hot (scaled logits of standard
deviation 65-130, |lse| in the hundreds).  Representative cases:

* bf16 rows whose weight sits on a few keys with tangent logits of tens: P and
  P*tS meet V as bf16 values; normalising O and tO by the fp32 sum of p left a
  mismatch of about 2^-9 |scale*tS| |V| (tO 2.1e-2 here).  The kernel now
  normalises by the sum of the bf16 weights the products consume, so the
  centring cancels for a dominant key; this case is checked at 2e-2;
* bf16 rows with tangent logits in the hundreds (tangent std 5 on keys whose
  norms grow 30-fold): the bf16 rounding of P*tS, about 2^-9 |scale*tS| |V|,
  exceeded the tolerance against the much smaller tO (2.1e-2).  The kernel now
  centres the tangent logits on a per-row value before that rounding (d = 128);
  this case is checked at 2e-2;
* float32 key shards: each shard's lse is a float32, so the merge weights
  carry a relative error of about 2^-24 |lse|; with |lse| near 1000 the merged
  O and tO are off by 1-2e-5 (the unsplit pass stays far inside 1e-5): an
  expected failure with its measured error;
* fp32 rows carried by one key: the exact tO is small next to |scale*tS| |v|
  and the computed one carries a few units of 2^-24 |scale*tS| |v| of
  rounding: checked as an absolute error;
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


def test_bf16_tangent_logits_in_the_hundreds(A):
    """Peaky rows (logit std ~9, key norms rising 30-fold along the keys) with
    tangent logits in the hundreds: P*tS meets V as bf16, so each product
    carries about 2^-9 |scale*tS - c| |V| of rounding, while tO (the spread of
    tS around its mean, times V) is far smaller.  Without centring (c = 0) the
    worst head was off by 2.1e-2 of the tensor's largest tO; with tS centred on
    the weighted mean of the tile that set each row's exponent base it is
    within the tolerance, unsplit and in key shards alike."""
    std = {"q": 3.0, "k": 3.0, "v": 1.0, "tq": 5.0, "tk": 0.0, "tv": 0.0}
    w = custom_workload(1, 3, 25, 2999, 128, "bf16", seed_id=101735, std=std, key_ramp=0.01)
    print("case bf16 tangent logits in the hundreds B1 H3 Lq25 Lk2999 d128 frozen ramp0.01", flush=True)
    x = device_inputs(w)
    o, to, lse = A.fwd(x["q"], x["k"], x["v"], x["tq"], None, None, scale=w.scale)
    torch.cuda.synchronize()
    whole = compare(w, o, to, lse)
    o, to, lse, _ = A.fwd_split(x["q"], x["k"], x["v"], x["tq"], None, None, 2, scale=w.scale)
    torch.cuda.synchronize()
    split = compare(w, o, to, lse)
    print(f"  unsplit O {whole['O']:.3e} tO {whole['tO']:.3e}; 2 shards O {split['O']:.3e} tO {split['tO']:.3e}",
          flush=True)
    for r in (whole, split):
        assert r["O"] <= TOL["bf16"] and r["tO"] <= TOL["bf16"] and r["lse"] <= 1e-4


def test_fp32_rows_carried_by_one_key(A):
    """fp32, a frozen context and rows whose softmax puts 0.9999 of its weight on
    one key: the exact tO is small (here ~4e-3) next to |scale*tS| |v| (~30),
    and the computed one carries the rounding residual of the centring, a few
    units of 2^-24 |scale*tS| |v|.  Checked as an absolute error."""
    std = {"q": 3.0, "k": 3.0, "v": 1.0, "tq": 1.0, "tk": 0.0, "tv": 0.0}
    w = custom_workload(1, 1, 64, 209, 128, "fp32", seed_id=110957, std=std, key_ramp=0.01)
    print("case fp32 rows carried by one key B1 H1 Lq64 Lk209 d128 frozen ramp0.01", flush=True)
    x = device_inputs(w)
    o, to, lse = A.fwd(x["q"], x["k"], x["v"], x["tq"], None, None, scale=w.scale)
    torch.cuda.synchronize()
    res = compare(w, o, to, lse)
    q, k, v, tq = (x[t].double().cpu() for t in ("q", "k", "v", "tq"))
    ts_v = (w.scale * (tq @ k.transpose(-1, -2))).abs().max().item() * v.abs().max().item()
    from _parity import oracle_head

    _, tO, _, _ = oracle_head(w, 0, 0, with_tlse=True)
    abs_err = float(np.max(np.abs(to[0, 0].double().cpu().numpy() - tO)))
    print(f"  O {res['O']:.3e} tO {res['tO']:.3e} (relative); |tO| error {abs_err:.3e} against "
          f"2^-24 |tS| |v| = {2.0 ** -24 * ts_v:.3e}", flush=True)
    assert res["O"] <= TOL["fp32"] and res["lse"] <= 1e-5
    assert abs_err <= 16 * 2.0 ** -24 * ts_v


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
