"""Pins for the fp64 projection oracle (``oracle.projection_jvp``), each from a
source other than the oracle itself.

The pages define a JVP as the Jacobian applied to a tangent (notes on
"Consistent Distribution Matching for Data-Free Diffusion Distillation",
prerequisites, "JVP") and name torch.func.jvp as the stock forward-mode tool
(ai.info summary of the rCM paper, "Methodology in Plain English").  The
projection's tangent is pinned by central finite differences of the primal map
and by torch.func.jvp through a torch linear layer followed by softmax
attention in torch operations; the primal map and the head layout by explicit
loops and by a permutation weight that sends named input features to named
output slots.
The last test plants plausible mistakes and checks that the pins reject each.
"""
import numpy as np
import pytest
import torch

from oracle import attention_jvp_head, projection_jvp


def rel(a, b):
    a, b = np.asarray(a), np.asarray(b)
    return float(np.max(np.abs(a - b)) / max(np.max(np.abs(b)), 1e-300))


def case(seed, B, L, D, n_out, H, d, bias=True):
    rng = np.random.default_rng(seed)
    F = n_out * H * d
    x, tx = rng.normal(0, 1, (B, L, D)), rng.normal(0, 1, (B, L, D))
    w = rng.normal(0, D ** -0.5, (F, D))
    b = rng.normal(0, 0.5, (F,)) if bias else None
    return x, tx, w, b


# ---- pins, each a function of a candidate projection (the oracle or a mutant) ----------

def loops(x, tx, w, b, n_out, H, d):
    """Brute force: every output element as an explicit sum over the hidden dim."""
    B, L, D = x.shape
    Y = np.zeros((n_out, B, H, L, d))
    TY = np.zeros((n_out, B, H, L, d))
    for n in range(n_out):
        for bb in range(B):
            for h in range(H):
                for t in range(L):
                    for j in range(d):
                        f = (n * H + h) * d + j
                        acc = 0.0 if b is None else float(b[f])
                        tacc = 0.0
                        for k in range(D):
                            acc += float(x[bb, t, k]) * float(w[f, k])
                            tacc += float(tx[bb, t, k]) * float(w[f, k])
                        Y[n, bb, h, t, j] = acc
                        TY[n, bb, h, t, j] = tacc
    return Y, TY


def pin_loops(proj):
    x, tx, w, b = case(1, 2, 3, 5, 2, 2, 3)
    Y, TY = proj(x, tx, w, b, 2, 2, 3)
    Yl, TYl = loops(x, tx, w, b, 2, 2, 3)
    return rel(Y, Yl) < 1e-13 and rel(TY, TYl) < 1e-13


def pin_central_difference(proj):
    x, tx, w, b = case(2, 2, 4, 6, 3, 2, 4)
    _, TY = proj(x, tx, w, b, 3, 2, 4)
    e = 1e-3
    Yp, _ = proj(x + e * tx, None, w, b, 3, 2, 4)
    Ym, _ = proj(x - e * tx, None, w, b, 3, 2, 4)
    return rel(TY, (Yp - Ym) / (2 * e)) < 1e-10


def pin_permutation(proj):
    """W = a permutation matrix: output feature f is input feature pi(f), plus b[f],
    at [n, b, h, t, j] with f = (n*H + h)*d + j."""
    n_out, H, d, B, L = 3, 2, 2, 2, 3
    F = n_out * H * d
    pi = np.random.default_rng(3).permutation(F)
    w = np.zeros((F, F))
    w[np.arange(F), pi] = 1.0
    x = np.random.default_rng(4).normal(0, 1, (B, L, F))
    b = np.arange(F, dtype=np.float64) * 100.0
    Y, _ = proj(x, None, w, b, n_out, H, d)
    for n in range(n_out):
        for h in range(H):
            for j in range(d):
                f = (n * H + h) * d + j
                if not np.array_equal(Y[n, :, h, :, j], x[:, :, pi[f]] + b[f]):
                    return False
    return True


def pin_bias_has_no_tangent(proj):
    x, tx, w, b = case(5, 1, 3, 4, 1, 2, 2)
    Y1, TY1 = proj(x, tx, w, b, 1, 2, 2)
    Y0, TY0 = proj(x, tx, w, None, 1, 2, 2)
    return np.array_equal(TY1, TY0) and rel(Y1 - Y0, b.reshape(1, 1, 2, 1, 2).repeat(3, axis=3)) < 1e-14


PINS = [pin_loops, pin_central_difference, pin_permutation, pin_bias_has_no_tangent]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_passes_pin(pin):
    assert pin(projection_jvp)


def test_linear_in_tangent():
    x, tx, w, b = case(6, 2, 3, 5, 3, 1, 2)
    tx2 = np.random.default_rng(7).normal(0, 1, tx.shape)
    _, T1 = projection_jvp(x, tx, w, b, 3, 1, 2)
    _, T2 = projection_jvp(x, tx2, w, b, 3, 1, 2)
    _, T12 = projection_jvp(x, 2.0 * tx - 3.0 * tx2, w, b, 3, 1, 2)
    assert rel(T12, 2.0 * T1 - 3.0 * T2) < 1e-13


def test_rows_select_tokens():
    x, tx, w, b = case(8, 2, 9, 6, 2, 2, 2)
    rows = np.array([0, 4, 8])
    Y, TY = projection_jvp(x, tx, w, b, 2, 2, 2)
    Yr, TYr = projection_jvp(x, tx, w, b, 2, 2, 2, rows=rows)
    assert np.array_equal(Yr, Y[:, :, :, rows]) and np.array_equal(TYr, TY[:, :, :, rows])


def test_no_tangent_gives_none():
    x, _, w, b = case(9, 1, 2, 3, 1, 1, 2)
    assert projection_jvp(x, None, w, b, 1, 1, 2)[1] is None


def test_chain_rule_through_attention_matches_torch_func_jvp():
    """Projection tangents fed to the attention oracle equal torch.func.jvp of
    the composed map x -> attention(split(x W^T + b)) in float64, written with
    torch's linear layer, matmul and softmax."""
    B, L, D, H, d = 1, 7, 12, 2, 4
    x, tx, w, b = case(10, B, L, D, 3, H, d)
    s = d ** -0.5
    Y, TY = projection_jvp(x, tx, w, b, 3, H, d)

    def composed(xt):
        z = torch.nn.functional.linear(xt, torch.from_numpy(w), torch.from_numpy(b))
        z = z.reshape(B, L, 3, H, d).permute(2, 0, 3, 1, 4)
        att = torch.softmax(s * (z[0] @ z[1].transpose(-1, -2)), dim=-1)
        return att @ z[2]

    O_t, tO_t = torch.func.jvp(composed, (torch.from_numpy(x),), (torch.from_numpy(tx),))
    for h in range(H):
        O, tO, _ = attention_jvp_head(Y[0, 0, h], Y[1, 0, h], Y[2, 0, h], TY[0, 0, h], TY[1, 0, h],
                                      TY[2, 0, h], s)
        assert rel(O, O_t[0, h].numpy()) < 1e-12
        assert rel(tO, tO_t[0, h].numpy()) < 1e-12


# ---- planted mistakes: each must be rejected by a pin ---------------------------------------

def _mutants():
    def transposed_weight(x, tx, w, b, n_out, H, d):
        # uses W rather than W^T (only defined for square W, else falls back to a wrong slice)
        D = x.shape[-1]
        wt = w.T if w.shape[0] == w.shape[1] else np.roll(w, 1, axis=1)
        return projection_jvp(x, tx, wt[: n_out * H * d, :D], b, n_out, H, d)

    def bias_in_tangent(x, tx, w, b, n_out, H, d):
        Y, TY = projection_jvp(x, tx, w, b, n_out, H, d)
        if TY is not None and b is not None:
            TY = TY + np.asarray(b).reshape(n_out, 1, H, 1, d)
        return Y, TY

    def heads_and_projections_swapped(x, tx, w, b, n_out, H, d):
        # features read as [head, projection, dim] instead of [projection, head, dim]
        Y, TY = projection_jvp(x, tx, w, b, n_out, H, d)

        def sw(z):
            if z is None:
                return None
            B, L = z.shape[1], z.shape[3]
            flat = z.transpose(1, 3, 0, 2, 4).reshape(B, L, n_out * H * d)
            return flat.reshape(B, L, H, n_out, d).transpose(3, 0, 2, 1, 4)

        return sw(Y), sw(TY)

    def halved_tangent(x, tx, w, b, n_out, H, d):
        Y, TY = projection_jvp(x, tx, w, b, n_out, H, d)
        return Y, None if TY is None else 0.5 * TY

    def dropped_bias(x, tx, w, b, n_out, H, d):
        return projection_jvp(x, tx, w, None, n_out, H, d)

    def tokens_reversed(x, tx, w, b, n_out, H, d):
        Y, TY = projection_jvp(x, tx, w, b, n_out, H, d)
        return Y[:, :, :, ::-1], None if TY is None else TY[:, :, :, ::-1]

    return [transposed_weight, bias_in_tangent, heads_and_projections_swapped,
            halved_tangent, dropped_bias, tokens_reversed]


@pytest.mark.parametrize("mutant", _mutants(), ids=lambda m: m.__name__)
def test_pins_reject_planted_mistake(mutant):
    assert not all(pin(mutant) for pin in PINS), mutant.__name__
