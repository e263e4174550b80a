"""Pins for the fp64 oracle of the query/key normalisation and rotary
embedding (``oracle.norm_rope_jvp``), each from a source other than the
oracle itself.

The pages define a JVP as the Jacobian applied to a tangent (notes on
"Consistent Distribution Matching for Data-Free Diffusion Distillation",
prerequisites, "JVP") and name torch.func.jvp as the stock forward-mode tool
(ai.info summary of the rCM paper, "Methodology in Plain English").  Here the
tangent is pinned by torch.func.jvp through torch's own rms_norm followed by a
rotation written with complex numbers, and by central finite differences; the
primal by the same torch composition, a hand-worked example and invariants of
normalisation and rotation.  The last test plants plausible mistakes and
checks that the pins reject each.
"""
import json
import os

import numpy as np
import torch

from oracle import norm_rope_jvp

HERE = os.path.dirname(os.path.abspath(__file__))


def rel(a, b):
    a, b = np.asarray(a), np.asarray(b)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def case(seed, L=5, d=8, lead=(2, 3), eps=1e-6):
    rng = np.random.default_rng(seed)
    x = rng.normal(0, 1.5, (*lead, L, d))
    tx = rng.normal(0, 0.7, (*lead, L, d))
    g = 1.0 + rng.normal(0, 0.3, d)
    theta = rng.uniform(-np.pi, np.pi, (L, d // 2))
    return x, tx, g, np.cos(theta), np.sin(theta), theta, eps


# ---- pins, each a function of a candidate implementation (the oracle or a mutant) -----

def torch_layer(x, g, theta, eps):
    """rms_norm from torch, then each adjacent pair (2i, 2i+1) read as the
    complex number z = n_2i + i n_2i+1 and multiplied by exp(i theta)."""
    n = torch.nn.functional.rms_norm(x, (x.shape[-1],), weight=g, eps=eps)
    z = torch.view_as_complex(n.reshape(*n.shape[:-1], -1, 2).contiguous())
    rot = torch.polar(torch.ones_like(theta), theta)
    return torch.view_as_real(z * rot).reshape(n.shape)


def pin_torch_func_jvp(f):
    x, tx, g, c, s, theta, eps = case(1)
    y, ty = f(x, tx, g, c, s, eps)
    T = lambda a: torch.tensor(a, dtype=torch.float64)  # noqa: E731
    yt, tyt = torch.func.jvp(lambda xx: torch_layer(xx, T(g), T(theta), eps), (T(x),), (T(tx),))
    return rel(y, yt.numpy()) < 1e-13 and rel(ty, tyt.numpy()) < 1e-13


def pin_central_difference(f):
    x, tx, g, c, s, _, eps = case(2)
    _, ty = f(x, tx, g, c, s, eps)
    h = 1e-6
    yp, _ = f(x + h * tx, None, g, c, s, eps)
    ym, _ = f(x - h * tx, None, g, c, s, eps)
    return rel(ty, (yp - ym) / (2 * h)) < 1e-8


def pin_hand_example(f):
    doc = json.load(open(os.path.join(HERE, "golden", "norm_rope_hand_example.json")))
    i = doc["inputs"]
    y, ty = f(np.array(i["x"]), np.array(i["tx"]), np.array(i["gamma"]), np.array(i["cos"]), np.array(i["sin"]),
              i["eps"])
    return rel(y, doc["expected"]["y"]) < 1e-15 and rel(ty, doc["expected"]["ty"]) < 1e-15


def pin_pair_norms(f):
    """A rotation keeps each pair's length: |y_2i, y_2i+1| = |n_2i, n_2i+1|, the
    same for the tangent (n, tn from the identity rotation)."""
    x, tx, g, c, s, _, eps = case(3)
    y, ty = f(x, tx, g, c, s, eps)
    n, tn = f(x, tx, g, None, None, eps)
    pn = lambda z: np.hypot(z[..., 0::2], z[..., 1::2])  # noqa: E731
    return rel(pn(y), pn(n)) < 1e-14 and rel(pn(ty), pn(tn)) < 1e-14


def pin_unit_rms(f):
    """Gain 1, eps 0: every output row has root-mean-square exactly 1."""
    x, tx, _, c, s, _, _ = case(4)
    y, _ = f(x, tx, None, c, s, 0.0)
    return float(np.max(np.abs(np.sqrt(np.mean(y * y, axis=-1)) - 1.0))) < 1e-14


def pin_scale_invariance(f):
    """eps 0: the layer ignores a positive scale of its input, so its
    derivative along the input itself is zero."""
    x, tx, g, c, s, _, _ = case(5)
    y, ty = f(x, x, g, c, s, 0.0)
    y3, _ = f(3.7 * x, None, g, c, s, 0.0)
    return rel(y3, y) < 1e-14 and float(np.max(np.abs(ty))) < 1e-13 * float(np.max(np.abs(y)))


def pin_identity_rotation(f):
    """cos = 1, sin = 0: y is g * x / sqrt(mean(x^2) + eps) written out per row."""
    x, tx, g, _, _, _, eps = case(6, L=3, d=4, lead=(2,))
    one, zero = np.ones((3, 2)), np.zeros((3, 2))
    y, _ = f(x, tx, g, one, zero, eps)
    want = np.empty_like(x)
    for b in range(2):
        for t in range(3):
            ms = sum(v * v for v in x[b, t]) / 4.0
            want[b, t] = g * x[b, t] / np.sqrt(ms + eps)
    return rel(y, want) < 1e-14


def pin_there_and_back(f):
    """Gain 1, eps 0: rotating by -theta the output of a rotation by theta
    (the second normalisation is a no-op on unit-RMS rows) gives the first
    normalisation back."""
    x, tx, _, c, s, _, _ = case(7)
    y, _ = f(x, tx, None, c, s, 0.0)
    back, _ = f(y, None, None, c, -s, 0.0)
    n, _ = f(x, None, None, None, None, 0.0)
    return rel(back, n) < 1e-14


def pin_linearity(f):
    x, tx, g, c, s, _, eps = case(8)
    tx2 = np.random.default_rng(9).normal(0, 1, x.shape)
    _, t1 = f(x, tx, g, c, s, eps)
    _, t2 = f(x, tx2, g, c, s, eps)
    _, t12 = f(x, 2.0 * tx - 0.5 * tx2, g, c, s, eps)
    return rel(t12, 2.0 * t1 - 0.5 * t2) < 1e-13


def pin_pairing(f):
    """A row with a single nonzero element at index 2i + e lands on the pair
    (2i, 2i+1) only, as (c, s) * v for e = 0 and (-s, c) * v for e = 1."""
    d, i = 8, 2
    ang = 0.3
    c, s = np.full((1, d // 2), np.cos(ang)), np.full((1, d // 2), np.sin(ang))
    for e in (0, 1):
        x = np.zeros((1, d))
        x[0, 2 * i + e] = 2.0
        y, _ = f(x, None, None, c, s, 0.0)
        v = 2.0 / np.sqrt(4.0 / d)
        want = np.zeros((1, d))
        want[0, 2 * i], want[0, 2 * i + 1] = (np.cos(ang) * v, np.sin(ang) * v) if e == 0 else \
            (-np.sin(ang) * v, np.cos(ang) * v)
        if rel(y, want) > 1e-14:
            return False
    return True


PINS = [pin_torch_func_jvp, pin_central_difference, pin_hand_example, pin_pair_norms, pin_unit_rms,
        pin_scale_invariance, pin_identity_rotation, pin_there_and_back, pin_linearity, pin_pairing]


def test_torch_func_jvp():
    assert pin_torch_func_jvp(norm_rope_jvp)


def test_central_difference():
    assert pin_central_difference(norm_rope_jvp)


def test_hand_worked_example():
    assert pin_hand_example(norm_rope_jvp)


def test_invariants():
    for p in (pin_pair_norms, pin_unit_rms, pin_scale_invariance, pin_identity_rotation, pin_there_and_back,
              pin_linearity, pin_pairing):
        assert p(norm_rope_jvp), p.__name__


def test_no_tangent_and_no_tables():
    x, tx, g, c, s, _, eps = case(10)
    y, ty = norm_rope_jvp(x, None, g, c, s, eps)
    assert ty is None
    y2, _ = norm_rope_jvp(x, tx, g, c, s, eps)
    assert np.array_equal(y, y2)


# ---- planted mistakes: each must fail at least one pin ------------------------------------

def _mutant(kind):
    def f(x, tx, gamma, cos, sin, eps):
        x = np.asarray(x, dtype=np.float64)
        d = x.shape[-1]
        g = np.ones(d) if gamma is None else np.asarray(gamma, dtype=np.float64)
        m = np.sum(x * x, -1, keepdims=True) / (d if kind != "sum_not_mean" else 1)
        r = 1.0 / (np.sqrt(m) + eps) if kind == "eps_outside" else 1.0 / np.sqrt(m + eps)
        n = g * x * r

        def rot(z):
            if cos is None:
                return z
            c, s = np.asarray(cos), np.asarray(sin)
            out = np.empty_like(z)
            if kind == "half_pairs":
                a, b = z[..., : d // 2], z[..., d // 2:]
                out[..., : d // 2], out[..., d // 2:] = c * a - s * b, s * a + c * b
                return out
            e, o = z[..., 0::2], z[..., 1::2]
            sg = -1.0 if kind == "sign" else 1.0
            out[..., 0::2] = c * e - sg * s * o
            out[..., 1::2] = sg * s * e + c * o
            return out

        if tx is None:
            return rot(n), None
        tx = np.asarray(tx, dtype=np.float64)
        xt = np.mean(x * tx, -1, keepdims=True)
        if kind == "no_r3_term":
            tn = g * tx * r
        elif kind == "r2_term":
            tn = g * (tx * r - x * r ** 2 * xt)
        elif kind == "no_gain_in_tangent":
            tn = tx * r - x * r ** 3 * xt
        else:
            tn = g * (tx * r - x * r ** 3 * xt)
        if kind == "tangent_not_rotated":
            return rot(n), tn
        return rot(n), rot(tn)
    return f


def test_planted_mistakes_are_rejected():
    for kind in ("sum_not_mean", "eps_outside", "half_pairs", "sign", "no_r3_term", "r2_term",
                 "no_gain_in_tangent", "tangent_not_rotated"):
        f = _mutant(kind)
        failed = [p.__name__ for p in PINS if not p(f)]
        assert failed, f"mistake {kind} passes every pin"
    # the mutant builder itself, with no mistake, passes every pin
    assert all(p(_mutant("none")) for p in PINS)
