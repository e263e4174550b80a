"""GPU: where the fp32 path meets its 1e-5 tolerance, and where it does not.

The fp32 kernel accumulates the logits S = q.k of a (query, key) pair in fp32
on the matrix cores: the partial sums have the size of |S| and each addition
rounds at 2^-24 of it, so S carries an absolute error of about
2^-24 sqrt(d) |S|.  Every probability inherits it through exp(scale * S): the
relative error of P, and with it of O and tO, grows in proportion to the
magnitude of the scaled logits, whatever their spread.  Inside the envelope
stated in include/attn_jvp.h (scaled logits of standard deviation up to
about 8, |scale * S| up to about 40) the path meets 1e-5; the cases marked
xfail below lie beyond it, and their reasons give the error measured on
MI355X.  Widening the envelope needs S accumulated in wider precision (fp64
matrix products, or exact integer products of split operands), which the
kernel's register budget does not hold next to its fp32 operands.
"""
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


def run_case(A, w, frozen=False):
    x = device_inputs(w)
    tk, tv = (None, None) if frozen else (x["tk"], x["tv"])
    o, to, lse = A.fwd(x["q"], x["k"], x["v"], x["tq"], tk, tv, scale=w.scale)
    torch.cuda.synchronize()
    res = compare(w, o, to, lse)
    print(f"  O {res['O']:.3e} tO {res['tO']:.3e} lse {res['lse']:.3e}", flush=True)
    return res


INSIDE = [
    # (B, H, Lq, Lk, d, operand std, tangent std): scaled logit std = operand std^2
    (1, 2, 300, 4000, 128, 2.83, 1.0),   # logit std 8, the envelope's edge
    (1, 2, 300, 9000, 64, 2.0, 10.0),    # logit std 4 over 9000 keys
]


@pytest.mark.parametrize("B,H,Lq,Lk,d,sq,st", INSIDE)
def test_inside_the_envelope(A, B, H, Lq, Lk, d, sq, st):
    std = {"q": sq, "k": sq, "v": 1.0, "tq": st, "tk": st, "tv": st}
    w = custom_workload(B, H, Lq, Lk, d, "fp32", seed_id=6100 + Lk + d, std=std)
    print(f"case fp32 inside envelope B{B} H{H} Lq{Lq} Lk{Lk} d{d} sq{sq} st{st}", flush=True)
    res = run_case(A, w)
    assert res["O"] <= TOL["fp32"] and res["tO"] <= TOL["fp32"]


OUTSIDE = [
    # (B, H, Lq, Lk, d, operand std, key ramp, reason)
    (1, 2, 256, 2000, 128, 6.3, 0.0,
     "scaled logits of std 40: fp32 logits lose about 2^-24 sqrt(d) |scale S|"),
    (1, 1, 256, 2437, 128, 2.0, 0.05,
     "rising logits (last keys scaled 120x): |scale S| in the hundreds"),
    (1, 1, 128, 6000, 64, 1.0, 0.04,
     "rising logits (last keys scaled 240x): |scale S| in the hundreds"),
]


@pytest.mark.parametrize("B,H,Lq,Lk,d,sq,ramp,reason", OUTSIDE)
def test_outside_the_envelope(A, B, H, Lq, Lk, d, sq, ramp, reason):
    std = {"q": sq, "k": sq, "v": 1.0, "tq": 1.0, "tk": 1.0, "tv": 1.0}
    w = custom_workload(B, H, Lq, Lk, d, "fp32", seed_id=6200 + Lk + d, std=std, key_ramp=ramp)
    print(f"case fp32 outside envelope B{B} H{H} Lq{Lq} Lk{Lk} d{d} sq{sq} ramp{ramp}: {reason}", flush=True)
    res = run_case(A, w)
    # still far inside the bf16 tolerance: the loss is gradual, not a failure mode
    assert res["O"] <= 1e-3 and res["tO"] <= 1e-3
    if res["O"] > TOL["fp32"] or res["tO"] > TOL["fp32"]:
        pytest.xfail(f"{reason}; measured O {res['O']:.2e}, tO {res['tO']:.2e} against the 1e-5 tolerance")
