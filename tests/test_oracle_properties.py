"""Property pins of the attention oracle (CPU), over arbitrary small inputs.

The fixed pins (tests/test_oracle_pins.py) check the oracle on chosen cases;
these draw shapes, softmax scales and values with hypothesis (derandomized,
so every run draws the same cases) and check what must hold for any input:

* the tangent is the complex-step derivative of the plain forward map
  softmax(scale Q K^T) V evaluated in complex arithmetic (Squire and Trapp's
  complex-step method), and the lse tangent that of the log-sum-exp;
* the tangent map is linear;
* a tangent that adds one vector to every key leaves the output unchanged
  (the softmax is invariant to a per-row constant), and tangent (0, 0, V) gives
  O back;
* key shards of any split, each computed on its own and merged, give the
  result over all keys.
"""
import numpy as np
from hypothesis import given, settings, strategies as st

from oracle import attention_jvp_head, merge_shards

SETTINGS = dict(max_examples=60, deadline=None, derandomize=True)


@st.composite
def problems(draw):
    Lq = draw(st.integers(1, 4))
    Lk = draw(st.integers(1, 6))
    d = draw(st.integers(1, 5))
    seed = draw(st.integers(0, 2**31 - 1))
    spread = draw(st.sampled_from([0.1, 1.0, 3.0]))
    scale = draw(st.floats(0.05, 2.0))
    rng = np.random.default_rng(seed)
    q, tq = (spread * rng.standard_normal((Lq, d)) for _ in range(2))
    k, v, tk, tv = (spread * rng.standard_normal((Lk, d)) for _ in range(4))
    return q, k, v, tq, tk, tv, scale


def forward_complex(q, k, v, scale):
    """softmax(scale q k^T) v and the row log-sum-exp in complex arithmetic; the
    row shift uses the real part only (a real constant per row changes nothing)."""
    s = scale * (q @ k.T)
    m = s.real.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    return (e / z) @ v, (m + np.log(z))[:, 0]


@given(problems())
@settings(**SETTINGS)
def test_tangent_is_the_complex_step_derivative(pr):
    q, k, v, tq, tk, tv, scale = pr
    h = 1e-30
    O_c, lse_c = forward_complex(q + 1j * h * tq, k + 1j * h * tk, v + 1j * h * tv, scale)
    O, tO, lse, mu = attention_jvp_head(q, k, v, tq, tk, tv, scale, with_tlse=True)
    assert np.allclose(O, O_c.real, rtol=1e-12, atol=1e-12)
    assert np.allclose(lse, lse_c.real, rtol=1e-12, atol=1e-12)
    assert np.allclose(tO, O_c.imag / h, rtol=1e-9, atol=1e-9 * max(1.0, np.abs(tO).max()))
    assert np.allclose(mu, lse_c.imag / h, rtol=1e-9, atol=1e-9 * max(1.0, np.abs(mu).max()))


@given(problems(), st.floats(-2.0, 2.0), st.floats(-2.0, 2.0), st.integers(0, 2**31 - 1))
@settings(**SETTINGS)
def test_tangent_map_is_linear(pr, a, b, seed):
    q, k, v, tq, tk, tv, scale = pr
    rng = np.random.default_rng(seed)
    t2 = [rng.standard_normal(x.shape) for x in (tq, tk, tv)]
    _, t_1, _ = attention_jvp_head(q, k, v, tq, tk, tv, scale)
    _, t_2, _ = attention_jvp_head(q, k, v, *t2, scale)
    mix = [a * x + b * y for x, y in zip((tq, tk, tv), t2)]
    _, t_mix, _ = attention_jvp_head(q, k, v, *mix, scale)
    assert np.allclose(t_mix, a * t_1 + b * t_2, rtol=1e-9, atol=1e-9 * max(1.0, np.abs(t_mix).max()))


@given(problems(), st.integers(0, 2**31 - 1))
@settings(**SETTINGS)
def test_shift_of_every_key_and_the_value_tangent(pr, seed):
    q, k, v, tq, tk, tv, scale = pr
    w = np.random.default_rng(seed).standard_normal((1, k.shape[1]))
    zero_q, zero_k = np.zeros_like(q), np.zeros_like(k)
    _, t_shift, _ = attention_jvp_head(q, k, v, zero_q, np.repeat(w, k.shape[0], axis=0), zero_k, scale)
    assert np.allclose(t_shift, 0.0, atol=1e-12)
    O, t_v, _ = attention_jvp_head(q, k, v, zero_q, zero_k, v, scale)
    assert np.allclose(t_v, O, rtol=1e-12, atol=1e-12)


@given(problems(), st.integers(0, 2**31 - 1))
@settings(**SETTINGS)
def test_any_key_split_merges_to_the_whole(pr, seed):
    q, k, v, tq, tk, tv, scale = pr
    Lk = k.shape[0]
    rng = np.random.default_rng(seed)
    cuts = sorted(set(rng.integers(1, Lk, size=rng.integers(0, Lk)).tolist())) if Lk > 1 else []
    bounds = list(zip([0] + cuts, cuts + [Lk]))
    parts = [attention_jvp_head(q, k[a:b], v[a:b], tq, tk[a:b], tv[a:b], scale, with_tlse=True) for a, b in bounds]
    O, tO, lse, mu = merge_shards(parts)
    O_f, tO_f, lse_f, mu_f = attention_jvp_head(q, k, v, tq, tk, tv, scale, with_tlse=True)
    for got, want in ((O, O_f), (tO, tO_f), (lse, lse_f), (mu, mu_f)):
        assert np.allclose(got, want, rtol=1e-11, atol=1e-11 * max(1.0, np.abs(want).max()))


def _variant(mistake):
    """The oracle's steps 1-6 with one planted mistake (test code only)."""
    def f(q, k, v, tq, tk, tv, scale, with_tlse=False):
        S = scale * q @ k.T
        m = S.max(axis=1, keepdims=True)
        E = np.exp(S - m)
        Z = E.sum(axis=1, keepdims=True)
        P = E / Z
        tS = (tq @ k.T + q @ tk.T) * (1.0 if mistake == "unscaled tS" else scale)
        if mistake == "tK dropped":
            tS = scale * (tq @ k.T)
        mu = (P * tS).sum(axis=1) * (0.0 if mistake == "mu dropped" else 1.0)
        tO = P @ (v if mistake == "V for tV" else tv) + (P * (tS - mu[:, None])) @ v
        lse = (m + np.log(Z))[:, 0] / (np.log(2.0) if mistake == "lse in base 2" else 1.0)
        return (P @ v, tO, lse, mu) if with_tlse else (P @ v, tO, lse)
    return f


def _complex_step_holds(fn, pr):
    q, k, v, tq, tk, tv, scale = pr
    h = 1e-30
    O_c, lse_c = forward_complex(q + 1j * h * tq, k + 1j * h * tk, v + 1j * h * tv, scale)
    O, tO, lse, mu = fn(q, k, v, tq, tk, tv, scale, with_tlse=True)
    return (np.allclose(O, O_c.real, rtol=1e-12, atol=1e-12) and np.allclose(lse, lse_c.real, rtol=1e-12, atol=1e-12)
            and np.allclose(tO, O_c.imag / h, rtol=1e-9, atol=1e-9 * max(1.0, np.abs(tO).max()))
            and np.allclose(mu, lse_c.imag / h, rtol=1e-9, atol=1e-9 * max(1.0, np.abs(mu).max())))


def test_complex_step_pin_rejects_planted_mistakes():
    rng = np.random.default_rng(4242)
    cases = []
    for _ in range(10):
        Lq, Lk, d = (int(x) for x in rng.integers(1, 6, size=3))
        q, tq = (rng.standard_normal((Lq, d)) for _ in range(2))
        k, v, tk, tv = (rng.standard_normal((Lk, d)) for _ in range(4))
        cases.append((q, k, v, tq, tk, tv, float(rng.uniform(0.1, 1.5))))
    assert all(_complex_step_holds(_variant(None), pr) for pr in cases)
    for mistake in ("unscaled tS", "tK dropped", "mu dropped", "V for tV", "lse in base 2"):
        assert not all(_complex_step_holds(_variant(mistake), pr) for pr in cases), mistake


# ---- the layers in front of attention ------------------------------------------


@st.composite
def projections(draw):
    B, L, D = draw(st.integers(1, 2)), draw(st.integers(1, 4)), draw(st.integers(1, 6))
    n_out, H, d = draw(st.integers(1, 3)), draw(st.integers(1, 2)), draw(st.integers(1, 3))
    seed = draw(st.integers(0, 2**31 - 1))
    rng = np.random.default_rng(seed)
    x, tx = (rng.standard_normal((B, L, D)) for _ in range(2))
    w = rng.standard_normal((n_out * H * d, D))
    bias = rng.standard_normal(n_out * H * d) if draw(st.booleans()) else None
    return x, tx, w, bias, n_out, H, d


@given(projections())
@settings(**SETTINGS)
def test_projection_tangent_is_the_complex_step_derivative(pr):
    """Y = x W^T + b written out per output element in complex arithmetic, then
    laid out [n, b, h, t, j] with feature f = (n H + h) d + j."""
    from oracle import projection_jvp

    x, tx, w, bias, n_out, H, d = pr
    hstep = 1e-30
    xc = x + 1j * hstep * tx
    B, L, D = x.shape
    Yc = np.zeros((n_out, B, H, L, d), dtype=complex)
    for n in range(n_out):
        for h in range(H):
            for j in range(d):
                f = (n * H + h) * d + j
                Yc[n, :, h, :, j] = (xc * w[f]).sum(axis=-1) + (0.0 if bias is None else bias[f])
    Y, TY = projection_jvp(x, tx, w, bias, n_out, H, d)
    assert np.allclose(Y, Yc.real, rtol=1e-12, atol=1e-12)
    assert np.allclose(TY, Yc.imag / hstep, rtol=1e-12, atol=1e-12)


@st.composite
def norm_rope_cases(draw):
    L, half = draw(st.integers(1, 4)), draw(st.integers(1, 4))
    seed = draw(st.integers(0, 2**31 - 1))
    rng = np.random.default_rng(seed)
    x, tx = (draw(st.sampled_from([0.1, 1.0, 5.0])) * rng.standard_normal((2, L, 2 * half)) for _ in range(2))
    gamma = 1.0 + 0.3 * rng.standard_normal(2 * half) if draw(st.booleans()) else None
    if draw(st.booleans()):
        ang = rng.uniform(-np.pi, np.pi, size=(L, half))
        cos, sin = np.cos(ang), np.sin(ang)
    else:
        cos = sin = None
    eps = draw(st.sampled_from([0.0, 1e-6, 0.5]))
    return x, tx, gamma, cos, sin, eps


@given(norm_rope_cases())
@settings(**SETTINGS)
def test_norm_rope_tangent_is_the_complex_step_derivative(pr):
    """The RMS normalisation (x^2, not |x|^2, so the map is analytic) and the
    rotation of each pair (2i, 2i+1), written in complex arithmetic."""
    from oracle import norm_rope_jvp

    x, tx, gamma, cos, sin, eps = pr
    hstep = 1e-30
    xc = x + 1j * hstep * tx
    n = xc / np.sqrt(np.mean(xc * xc, axis=-1, keepdims=True) + eps)
    if gamma is not None:
        n = n * gamma
    if cos is not None:
        even, odd = n[..., 0::2].copy(), n[..., 1::2].copy()
        n = n.copy()
        n[..., 0::2] = cos * even - sin * odd
        n[..., 1::2] = sin * even + cos * odd
    y, ty = norm_rope_jvp(x, tx, gamma, cos, sin, eps)
    assert np.allclose(y, n.real, rtol=1e-12, atol=1e-12)
    assert np.allclose(ty, n.imag / hstep, rtol=1e-9, atol=1e-9 * max(1.0, np.abs(ty).max()))
