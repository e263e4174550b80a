"""GPU: the fp32 path at large logits.

The fp32 kernel accumulates the logits S = q.k in fp64 and forms the exponent
S * scale * log2(e) - m in fp64 before a single rounding to fp32, so the
weights carry a relative error of a few 2^-24 whatever the size of the
logits.  (An fp32 sum of S would carry an absolute error of about
2^-24 sqrt(d) |S|, which every weight inherits through exp(scale * S): beyond
scaled logits of standard deviation ~8 that alone exceeds the 1e-5
tolerance.)  These cases push |scale * S| into the hundreds: logits of
standard deviation 40 and 100, keys whose logits rise along the sequence so
that the exponent base moves tile after tile, the frozen-context path and
key shards merged in fp32.  Each must meet the fp32 tolerance.
"""
import pytest
import torch

from workloads import custom_workload

from _parity import LSE_TOL, TOL, compare, device_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def A():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_forward_mode_attn_amd as A

    A.load_library()
    return A


CASES = [
    # (B, H, Lq, Lk, d, operand std, tangent std, key ramp, frozen, shards, what)
    (1, 2, 300, 4000, 128, 2.83, 1.0, 0.0, False, 1, "logit std 8"),
    (1, 2, 300, 9000, 64, 2.0, 10.0, 0.0, False, 1, "logit std 4 over 9000 keys, large tangents"),
    (1, 2, 256, 2000, 128, 6.3, 1.0, 0.0, False, 1, "logit std 40"),
    (1, 1, 200, 1500, 64, 10.0, 1.0, 0.0, False, 1, "logit std 100"),
    (1, 1, 256, 2437, 128, 2.0, 1.0, 0.05, False, 1, "rising logits, last keys scaled 120x"),
    (1, 1, 128, 6000, 64, 1.0, 1.0, 0.04, False, 1, "rising logits, last keys scaled 240x"),
    (2, 1, 130, 3001, 128, 2.0, 1.0, 0.05, True, 1, "rising logits, frozen context"),
    (1, 2, 190, 5003, 128, 6.3, 1.0, 0.0, False, 4, "logit std 40 over 4 key shards"),
    (1, 1, 96, 4100, 64, 1.0, 1.0, 0.05, False, 3, "rising logits over 3 key shards"),
]


@pytest.mark.parametrize("B,H,Lq,Lk,d,sq,st,ramp,frozen,shards,what", CASES)
def test_fp32_large_logits(A, B, H, Lq, Lk, d, sq, st, ramp, frozen, shards, what):
    std = {"q": sq, "k": sq, "v": 1.0, "tq": st, "tk": 0.0 if frozen else st, "tv": 0.0 if frozen else st}
    w = custom_workload(B, H, Lq, Lk, d, "fp32", seed_id=6300 + Lk + d, std=std, key_ramp=ramp)
    print(f"case fp32 {what}: B{B} H{H} Lq{Lq} Lk{Lk} d{d} sq{sq} st{st} ramp{ramp} frozen={frozen} "
          f"shards={shards}", flush=True)
    x = device_inputs(w)
    tk, tv = (None, None) if frozen else (x["tk"], x["tv"])
    if shards == 1:
        o, to, lse = A.fwd(x["q"], x["k"], x["v"], x["tq"], tk, tv, scale=w.scale)
    else:
        o, to, lse, _ = A.fwd_split(x["q"], x["k"], x["v"], x["tq"], tk, tv, shards, scale=w.scale)
    torch.cuda.synchronize()
    res = compare(w, o, to, lse)
    print(f"  O {res['O']:.3e} tO {res['tO']:.3e} lse {res['lse']:.3e}", flush=True)
    assert res["O"] <= TOL["fp32"] and res["tO"] <= TOL["fp32"] and res["lse"] <= LSE_TOL["fp32"]
