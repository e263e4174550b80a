"""Pins for the fp64 oracle, each from a source other than the oracle itself.

The pages define the JVP as the Jacobian applied to a tangent (notes on
"Consistent Distribution Matching for Data-Free Diffusion Distillation",
prerequisites, "JVP") and name torch.func.jvp as the stock forward-mode tool
(ai.info summary of the rCM paper, "Methodology in Plain English").  So tO is
pinned by: torch.func.jvp, central finite differences, complex-step
differentiation, and a brute-force Jacobian; O and lse by torch's
scaled_dot_product_attention and scipy's logsumexp; plus closed forms and
invariants of the tangent map.  The last tests plant plausible mistakes in the
oracle's outputs and check that the pins reject every one of them.

The tangent of lse (mu, step 5, returned with ``with_tlse``) is pinned by the
complex-step and finite-difference derivatives of lse; the merge of key-shard
results (``merge_shards``) by the full-key definition, which the pins above
fix.
"""
import numpy as np
import pytest
import scipy.special
import torch

from oracle import attention_jvp, attention_jvp_head, merge_shards


def case(seed, Lq, Lk, d, sig=1.0):
    rng = np.random.default_rng(seed)
    q, tq = rng.normal(0, sig, (Lq, d)), rng.normal(0, 1, (Lq, d))
    k, tk = rng.normal(0, sig, (Lk, d)), rng.normal(0, 1, (Lk, d))
    v, tv = rng.normal(0, 1, (Lk, d)), rng.normal(0, 1, (Lk, d))
    return q, k, v, tq, tk, tv


def plain_forward(q, k, v, scale):
    """Attention forward written with scipy's softmax, real or complex inputs."""
    S = scale * (q @ k.T)
    if np.iscomplexobj(S):
        m = S.real.max(axis=1, keepdims=True)
        E = np.exp(S - m)
        Z = E.sum(axis=1, keepdims=True)
        return (E / Z) @ v, m[:, 0] + np.log(Z[:, 0])
    return scipy.special.softmax(S, axis=1) @ v, scipy.special.logsumexp(S, axis=1)


def complex_step(q, k, v, tq, tk, tv, scale, h=1e-30):
    """Directional derivative of (O, lse) by the complex-step method."""
    O, lse = plain_forward(q + 1j * h * tq, k + 1j * h * tk, v + 1j * h * tv, scale)
    return O.imag / h, lse.imag / h


def rel(a, b):
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


SHAPES = [(7, 5, 4), (1, 1, 3), (3, 9, 8), (16, 33, 16)]


@pytest.mark.parametrize("Lq,Lk,d", SHAPES)
def test_torch_func_jvp(Lq, Lk, d):
    q, k, v, tq, tk, tv = case(1, Lq, Lk, d)
    s = d ** -0.5
    O, tO, lse = attention_jvp_head(q, k, v, tq, tk, tv, s)
    T = lambda x: torch.tensor(x, dtype=torch.float64)  # noqa: E731

    def f(qq, kk, vv):
        return torch.softmax(s * qq @ kk.T, dim=-1) @ vv

    o_ref, t_ref = torch.func.jvp(f, (T(q), T(k), T(v)), (T(tq), T(tk), T(tv)))
    assert rel(O, o_ref.numpy()) < 1e-13
    assert rel(tO, t_ref.numpy()) < 1e-12


@pytest.mark.parametrize("Lq,Lk,d", SHAPES)
def test_central_finite_difference(Lq, Lk, d):
    q, k, v, tq, tk, tv = case(2, Lq, Lk, d)
    s = d ** -0.5
    _, tO, lse = attention_jvp_head(q, k, v, tq, tk, tv, s)
    eps = 1e-5
    Op, lp = plain_forward(q + eps * tq, k + eps * tk, v + eps * tv, s)
    Om, lm = plain_forward(q - eps * tq, k - eps * tk, v - eps * tv, s)
    assert rel(tO, (Op - Om) / (2 * eps)) < 1e-7
    # mu (the tangent of lse) is not an output, but the forward lse must be right
    assert rel(lse, plain_forward(q, k, v, s)[1]) < 1e-14


@pytest.mark.parametrize("Lq,Lk,d", SHAPES)
def test_complex_step(Lq, Lk, d):
    q, k, v, tq, tk, tv = case(3, Lq, Lk, d)
    s = d ** -0.5
    _, tO, _ = attention_jvp_head(q, k, v, tq, tk, tv, s)
    t_cs, _ = complex_step(q, k, v, tq, tk, tv, s)
    assert rel(tO, t_cs) < 1e-13


def test_brute_force_jacobian():
    Lq, Lk, d = 5, 6, 3
    q, k, v, tq, tk, tv = case(4, Lq, Lk, d)
    s = 0.7
    x0 = np.concatenate([q.ravel(), k.ravel(), v.ravel()])
    t = np.concatenate([tq.ravel(), tk.ravel(), tv.ravel()])
    nq, nk = q.size, k.size

    def f(x):
        return plain_forward(x[:nq].reshape(Lq, d), x[nq:nq + nk].reshape(Lk, d),
                             x[nq + nk:].reshape(Lk, d), s)[0].ravel()

    h = 1e-30
    J = np.empty((Lq * d, x0.size))
    for j in range(x0.size):
        e = np.zeros(x0.size, dtype=complex)
        e[j] = 1j * h
        J[:, j] = f(x0 + e).imag / h
    _, tO, _ = attention_jvp_head(q, k, v, tq, tk, tv, s)
    assert rel(tO.ravel(), J @ t) < 1e-13


def test_against_sdpa_and_logsumexp():
    q, k, v, tq, tk, tv = case(5, 20, 37, 16)
    s = 16 ** -0.5
    O, _, lse = attention_jvp_head(q, k, v, tq, tk, tv, s)
    T = lambda x: torch.tensor(x, dtype=torch.float64)[None, None]  # noqa: E731
    o_ref = torch.nn.functional.scaled_dot_product_attention(T(q), T(k), T(v), scale=s)[0, 0].numpy()
    assert rel(O, o_ref) < 1e-13
    assert rel(lse, scipy.special.logsumexp(s * q @ k.T, axis=1)) < 1e-14


# ---- invariants of the tangent map ------------------------------------------------

def test_tangent_along_v_reproduces_output():
    q, k, v, _, _, _ = case(6, 9, 11, 8)
    z = np.zeros_like
    O, tO, _ = attention_jvp_head(q, k, v, z(q), z(k), v, 0.4)
    assert rel(tO, O) < 1e-14


def test_tangent_q_equals_tangent_k():
    # S is bilinear: moving q along q changes S exactly as moving k along k.
    q, k, v, _, _, tv = case(7, 9, 11, 8)
    z = np.zeros_like
    _, t1, _ = attention_jvp_head(q, k, v, q, z(k), z(v), 0.4)
    _, t2, _ = attention_jvp_head(q, k, v, z(q), k, z(v), 0.4)
    assert rel(t1, t2) < 1e-13


def test_linear_in_tangent():
    q, k, v, tq, tk, tv = case(8, 9, 11, 8)
    _, _, _, uq, uk, uv = case(9, 9, 11, 8)
    a, b = 1.7, -0.3
    _, t1, _ = attention_jvp_head(q, k, v, tq, tk, tv, 0.4)
    _, t2, _ = attention_jvp_head(q, k, v, uq, uk, uv, 0.4)
    _, t3, _ = attention_jvp_head(q, k, v, a * tq + b * uq, a * tk + b * uk, a * tv + b * uv, 0.4)
    assert rel(t3, a * t1 + b * t2) < 1e-13


def test_value_tangent_only_is_p_tv():
    q, k, v, _, _, tv = case(10, 9, 11, 8)
    z = np.zeros_like
    _, tO, _ = attention_jvp_head(q, k, v, z(q), z(k), tv, 0.4)
    P = scipy.special.softmax(0.4 * q @ k.T, axis=1)
    assert rel(tO, P @ tv) < 1e-14


def test_constant_key_shift_has_no_effect():
    # tK = 1 w^T shifts every logit of a row by the same amount: softmax ignores it.
    q, k, v, _, _, _ = case(11, 9, 11, 8)
    w = np.random.default_rng(0).normal(size=8)
    z = np.zeros_like
    _, tO, _ = attention_jvp_head(q, k, v, z(q), np.tile(w, (11, 1)), z(v), 0.4)
    assert np.max(np.abs(tO)) < 1e-13


def test_constant_value_tangent_passes_through():
    q, k, v, _, _, _ = case(12, 9, 11, 8)
    u = np.random.default_rng(1).normal(size=8)
    z = np.zeros_like
    _, tO, _ = attention_jvp_head(q, k, v, z(q), z(k), np.tile(u, (11, 1)), 0.4)
    assert rel(tO, np.tile(u, (9, 1))) < 1e-14


def test_single_key():
    q, k, v, tq, tk, tv = case(13, 6, 1, 8)
    O, tO, lse = attention_jvp_head(q, k, v, tq, tk, tv, 0.4)
    assert rel(O, np.tile(v, (6, 1))) < 1e-15
    assert rel(tO, np.tile(tv, (6, 1))) < 1e-15
    assert rel(lse, 0.4 * (q @ k.T)[:, 0]) < 1e-15


def test_uniform_attention_closed_form():
    # q = 0: every row attends uniformly; S = 0 so tS_j = s * tq . k_j and
    # tO = mean_j tv_j + (1/Lk) sum_j (tS_j - mean tS) v_j, lse = ln Lk.
    _, k, v, tq, tk, tv = case(14, 4, 10, 8)
    s = 0.35
    q = np.zeros((4, 8))
    O, tO, lse = attention_jvp_head(q, k, v, tq, tk, tv, s)
    tS = s * tq @ k.T
    want = tv.mean(0)[None, :] + ((tS - tS.mean(1, keepdims=True)) @ v) / 10
    assert rel(O, np.tile(v.mean(0), (4, 1))) < 1e-15
    assert rel(tO, want) < 1e-14
    assert rel(lse, np.full(4, np.log(10.0))) < 1e-15


def test_hand_worked_two_key_example():
    """S = [0, ln 3] gives P = [1/4, 3/4] exactly (d = 1, scale = 1, q = 1).

    tS_j = tq k_j + q tk_j = [0.5*0 + 1*0.2, 0.5*ln3 + 1*(-0.4)];
    mu = (1/4) tS_0 + (3/4) tS_1;  tO = sum_j P_j tv_j + sum_j P_j (tS_j - mu) v_j.
    """
    import json
    import os

    with open(os.path.join(os.path.dirname(__file__), "golden", "two_key_hand_example.json")) as f:
        g = json.load(f)
    a = {key: np.array(g["inputs"][key], dtype=np.float64) for key in ("q", "k", "v", "tq", "tk", "tv")}
    O, tO, lse = attention_jvp_head(a["q"], a["k"], a["v"], a["tq"], a["tk"], a["tv"], g["scale"])
    assert rel(O, np.array(g["expected"]["O"])) < 1e-15
    assert rel(tO, np.array(g["expected"]["tO"])) < 1e-14
    assert rel(lse, np.array(g["expected"]["lse"])) < 1e-15


def test_batched_matches_per_head_and_rows():
    rng = np.random.default_rng(15)
    B, H, Lq, Lk, d = 2, 3, 10, 7, 4
    q, tq = rng.normal(size=(B, H, Lq, d)), rng.normal(size=(B, H, Lq, d))
    k, tk, v, tv = (rng.normal(size=(B, H, Lk, d)) for _ in range(4))
    O, tO, lse = attention_jvp(q, k, v, tq, tk, tv, 0.5)
    rows = np.array([0, 3, 9])
    Os, tOs, ls = attention_jvp(q, k, v, tq, tk, tv, 0.5, rows=rows)
    for b in range(B):
        for h in range(H):
            o1, t1, l1 = attention_jvp_head(q[b, h], k[b, h], v[b, h], tq[b, h], tk[b, h], tv[b, h], 0.5)
            assert np.array_equal(O[b, h], o1) and np.array_equal(tO[b, h], t1)
            assert np.array_equal(lse[b, h], l1)
    assert np.array_equal(Os, O[:, :, rows]) and np.array_equal(tOs, tO[:, :, rows])
    assert np.array_equal(ls, lse[:, :, rows])


def test_peaky_softmax_is_finite():
    # logit std ~ 64: the row max must be subtracted, else exp overflows.
    q, k, v, tq, tk, tv = case(16, 8, 50, 16, sig=8.0)
    O, tO, lse = attention_jvp_head(q, k, v, tq, tk, tv, 16 ** -0.5)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(tO)) and np.all(np.isfinite(lse))
    t_cs, _ = complex_step(q, k, v, tq, tk, tv, 16 ** -0.5)
    assert rel(tO, t_cs) < 1e-11


# ---- planted mistakes: each must be rejected by a pin --------------------------------

def _mutants(q, k, v, tq, tk, tv, s):
    O, tO, lse = attention_jvp_head(q, k, v, tq, tk, tv, s)
    P = scipy.special.softmax(s * q @ k.T, axis=1)
    tS = s * (tq @ k.T + q @ tk.T)
    mu = (P * tS).sum(1, keepdims=True)
    z = np.zeros_like
    return {
        "dropped mu term": (tO + mu * O, lse),
        "wrong sign of mu": (tO + 2 * mu * O, lse),
        "dropped Q tK^T": (attention_jvp_head(q, k, v, tq, z(tk), tv, s)[1], lse),
        "dropped tQ K^T": (attention_jvp_head(q, k, v, z(tq), tk, tv, s)[1], lse),
        "unscaled tS": (attention_jvp_head(q, k, v, tq / s, tk / s, tv, s)[1], lse),
        "V in place of tV": (tO - P @ tv + P @ v, lse),
        "dropped P tV": (tO - P @ tv, lse),
        "lse in base 2": (tO, lse / np.log(2.0)),
        "unscaled lse": (tO, lse / s),
    }


def test_pins_reject_planted_mistakes():
    q, k, v, tq, tk, tv = case(17, 6, 9, 5)
    s = 5 ** -0.5
    t_cs, _ = complex_step(q, k, v, tq, tk, tv, s)
    lse_ref = scipy.special.logsumexp(s * q @ k.T, axis=1)
    _, tO, lse = attention_jvp_head(q, k, v, tq, tk, tv, s)
    assert rel(tO, t_cs) < 1e-13 and rel(lse, lse_ref) < 1e-14
    for name, (t_bad, l_bad) in _mutants(q, k, v, tq, tk, tv, s).items():
        caught = rel(t_bad, t_cs) > 1e-3 or rel(l_bad, lse_ref) > 1e-3
        assert caught, name


@pytest.mark.parametrize("Lq,Lk,d", SHAPES)
def test_tlse_is_the_tangent_of_lse(Lq, Lk, d):
    q, k, v, tq, tk, tv = case(21, Lq, Lk, d)
    s = d ** -0.5
    _, _, _, mu = attention_jvp_head(q, k, v, tq, tk, tv, s, with_tlse=True)
    _, l_cs = complex_step(q, k, v, tq, tk, tv, s)
    assert rel(mu, l_cs) < 1e-13
    eps = 1e-5
    lp = plain_forward(q + eps * tq, k + eps * tk, v, s)[1]
    lm = plain_forward(q - eps * tq, k - eps * tk, v, s)[1]
    assert rel(mu, (lp - lm) / (2 * eps)) < 1e-7


def test_tlse_vanishes_without_logit_tangents():
    q, k, v, tq, tk, tv = case(22, 5, 7, 4)
    z = np.zeros_like
    _, _, _, mu = attention_jvp_head(q, k, v, z(tq), z(tk), tv, 0.5, with_tlse=True)
    assert np.all(mu == 0.0)


SPLITS = [(9, [4, 5]), (33, [1, 32]), (33, [10, 11, 12]), (64, [16, 16, 16, 16]), (7, [1, 1, 5])]


@pytest.mark.parametrize("Lk,sizes", SPLITS)
def test_merge_of_key_shards_is_the_full_result(Lk, sizes):
    Lq, d = 6, 8
    q, k, v, tq, tk, tv = case(23, Lq, Lk, d, sig=1.5)
    s = d ** -0.5
    full = attention_jvp_head(q, k, v, tq, tk, tv, s, with_tlse=True)
    cuts = np.concatenate([[0], np.cumsum(sizes)])
    parts = [attention_jvp_head(q, k[a:b], v[a:b], tq, tk[a:b], tv[a:b], s, with_tlse=True)
             for a, b in zip(cuts[:-1], cuts[1:])]
    merged = merge_shards(parts)
    for got, ref in zip(merged, full):
        assert rel(got, ref) < 1e-12


def test_merge_pins_reject_planted_mistakes():
    Lq, Lk, d = 6, 12, 8
    q, k, v, tq, tk, tv = case(24, Lq, Lk, d, sig=1.5)
    s = d ** -0.5
    O, tO, lse, mu = attention_jvp_head(q, k, v, tq, tk, tv, s, with_tlse=True)
    parts = [attention_jvp_head(q, k[a:b], v[a:b], tq, tk[a:b], tv[a:b], s, with_tlse=True)
             for a, b in ((0, 5), (5, 12))]
    lse_s = np.stack([p[2] for p in parts])
    mu_s = np.stack([p[3] for p in parts])
    w = np.exp(lse_s - lse)
    mutants = {
        "no re-centring of the tangent": sum(w[i][:, None] * p[1] for i, p in enumerate(parts)),
        "equal shard weights": sum(0.5 * (p[1] + (mu_s[i] - mu)[:, None] * p[0]) for i, p in enumerate(parts)),
        "shift with the wrong sign": sum(w[i][:, None] * (p[1] - (mu_s[i] - mu)[:, None] * p[0])
                                         for i, p in enumerate(parts)),
    }
    assert rel(merge_shards(parts)[1], tO) < 1e-12
    for name, bad in mutants.items():
        assert rel(bad, tO) > 1e-3, name
