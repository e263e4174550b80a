"""The algebra the bf16 and fp32 kernels run, modelled in fp64 and checked
against the oracle (CPU, no GPU).

The rCM pages describe a JVP carried through the block-wise tiling of the
FlashAttention-2 forward (ai.info summary of "Large Scale Diffusion
Distillation via Score-Regularized Continuous-Time Consistency", "Methodology
in Plain English"; papernotes.org notes on the same paper, "Key designs" item
1) without printing the recurrence.  The kernels use this one, per query row,
over tiles of 64 keys:

  * logits in the log2 domain, y = S * scale * log2(e) - m, with an exponent
    base m that moves only when a tile's maximum exceeds it by more than 32
    (p = 2^y <= 2^32); moving it by delta scales l, a and both accumulators by
    2^-delta;
  * l += sum p,  a += sum p * tS,  acc_o += p V,  acc_t += p tV + (p * tS) V;
  * epilogue O = acc_o / l, tO = (acc_t - (a / l) acc_o) / l,
    lse = (m + log2 l) ln 2, tlse = a / l.

In exact arithmetic this is the definition the oracle writes out, so in fp64
the two agree to rounding; a slip in the recurrence (a missing rescale of one
accumulator, the centring term, the log base) shows up far above it.  The
model is test code: it shares nothing with the kernels or with the oracle.
"""
import numpy as np
import pytest

from oracle import attention_jvp_head

BC = 64
SLACK = 32.0
LOG2E = 1.0 / np.log(2.0)


def tiled(q, k, v, tq, tk, tv, scale, bc=BC, slack=SLACK, fixed_base=False):
    """fp64 model of the kernels' online recurrence (see the module docstring)."""
    Lq, d = q.shape
    Lk = k.shape[0]
    c2 = scale * LOG2E
    m = np.full(Lq, -np.inf)
    l = np.zeros(Lq)
    a = np.zeros(Lq)
    acc_o = np.zeros((Lq, v.shape[1]))
    acc_t = np.zeros((Lq, v.shape[1]))
    pmax = 0.0
    for j0 in range(0, Lk, bc):
        j1 = min(j0 + bc, Lk)  # ragged last tile: keys past Lk do not exist
        S = q @ k[j0:j1].T
        tS = scale * (tq @ k[j0:j1].T + q @ tk[j0:j1].T)
        ymax = (S * c2).max(axis=1)
        # the first tile sets the base; later tiles move it only past the slack
        move = (~np.isfinite(m)) | (ymax - m > (np.inf if fixed_base else slack))
        new_m = np.where(move, ymax, m)
        alpha = np.where(np.isfinite(m), np.exp2(m - new_m), 0.0)
        l, a = l * alpha, a * alpha
        acc_o *= alpha[:, None]
        acc_t *= alpha[:, None]
        m = new_m
        p = np.exp2(S * c2 - m[:, None])
        pmax = max(pmax, float(p.max()))
        pt = p * tS
        l += p.sum(axis=1)
        a += pt.sum(axis=1)
        acc_o += p @ v[j0:j1]
        acc_t += p @ tv[j0:j1] + pt @ v[j0:j1]
    O = acc_o / l[:, None]
    mu = a / l
    tO = (acc_t - mu[:, None] * acc_o) / l[:, None]
    lse = (m + np.log2(l)) * np.log(2.0)
    return O, tO, lse, mu, pmax


def case(seed, Lq, Lk, d, sig=1.0):
    rng = np.random.default_rng(seed)
    return (rng.normal(0, sig, (Lq, d)), rng.normal(0, sig, (Lk, d)), rng.normal(0, 1, (Lk, d)),
            rng.normal(0, 1, (Lq, d)), rng.normal(0, 1, (Lk, d)), rng.normal(0, 1, (Lk, d)))


def rel(x, y):
    return float(np.max(np.abs(x - y)) / max(np.max(np.abs(y)), 1e-300))


@pytest.mark.parametrize("Lq,Lk,d,sig", [
    (5, 1, 8, 1.0),        # one key, one partial tile
    (9, 63, 16, 1.0),      # one ragged tile
    (9, 64, 16, 1.0),      # exactly one tile
    (7, 65, 16, 1.0),      # a full tile and a one-key tail
    (12, 300, 32, 1.0),    # several tiles and a ragged tail
    (6, 517, 64, np.sqrt(8.0)),  # peaky logits (std ~ 8): the base moves mid-row
    (4, 700, 64, 4.0),     # very peaky logits (std ~ 16)
])
def test_tiled_recurrence_equals_the_definition(Lq, Lk, d, sig):
    q, k, v, tq, tk, tv = case(Lq * 1000 + Lk, Lq, Lk, d, sig)
    scale = d ** -0.5
    O, tO, lse, mu, pmax = tiled(q, k, v, tq, tk, tv, scale)
    R = attention_jvp_head(q, k, v, tq, tk, tv, scale, with_tlse=True)
    assert rel(O, R[0]) < 1e-12 and rel(tO, R[1]) < 1e-12
    assert np.max(np.abs(lse - R[2])) < 1e-11 and rel(mu, R[3]) < 1e-11
    assert pmax <= 2.0 ** SLACK  # the lazy base keeps every weight within 2^32 of it


def test_the_base_does_move_on_peaky_rows():
    """On logits of std ~ 16 the slack is exceeded after the first tile, so the
    rescale path is exercised (the test above then checks its algebra)."""
    q, k, v, tq, tk, tv = case(7, 4, 700, 64, 4.0)
    scale = 64 ** -0.5
    c2 = scale * LOG2E
    first = (q @ k[:BC].T * c2).max(axis=1)
    later = (q @ k[BC:].T * c2).max(axis=1)
    assert np.any(later - first > SLACK)


def test_recurrence_slips_are_caught():
    """Plausible slips in the recurrence each miss the definition by far more
    than rounding: the centring term dropped, acc_t not rescaled when the base
    moves, lse in base 2.  (Logits of std ~ 16, so that the base moves.)"""
    q, k, v, tq, tk, tv = case(7, 4, 700, 64, 4.0)
    scale = 64 ** -0.5
    R = attention_jvp_head(q, k, v, tq, tk, tv, scale, with_tlse=True)
    O, tO, lse, mu, _ = tiled(q, k, v, tq, tk, tv, scale)
    acc_o = O  # (acc_o / l)
    no_centre = tO + mu[:, None] * acc_o
    assert rel(no_centre, R[1]) > 1e-2
    assert np.max(np.abs(lse / np.log(2.0) - R[2])) > 1e-2

    def tiled_without_acc_t_rescale():
        Lq, d = q.shape
        c2 = scale * LOG2E
        m = np.full(Lq, -np.inf)
        l = np.zeros(Lq)
        a = np.zeros(Lq)
        acc_o = np.zeros((Lq, d))
        acc_t = np.zeros((Lq, d))
        for j0 in range(0, k.shape[0], BC):
            j1 = min(j0 + BC, k.shape[0])
            S = q @ k[j0:j1].T
            tS = scale * (tq @ k[j0:j1].T + q @ tk[j0:j1].T)
            ymax = (S * c2).max(axis=1)
            move = (~np.isfinite(m)) | (ymax - m > SLACK)
            new_m = np.where(move, ymax, m)
            alpha = np.where(np.isfinite(m), np.exp2(m - new_m), 0.0)
            l, a = l * alpha, a * alpha
            acc_o *= alpha[:, None]  # acc_t left unscaled: the slip
            m = new_m
            p = np.exp2(S * c2 - m[:, None])
            l += p.sum(axis=1)
            a += (p * tS).sum(axis=1)
            acc_o += p @ v[j0:j1]
            acc_t += p @ tv[j0:j1] + (p * tS) @ v[j0:j1]
        return (acc_t - (a / l)[:, None] * acc_o) / l[:, None]

    assert rel(tiled_without_acc_t_rescale(), R[1]) > 1e-2


def test_fixed_base_needs_the_slack():
    """Without moving the base after the first tile, peaky rows overflow the
    weights' headroom: the bound that the lazy rule keeps is a real constraint."""
    q, k, v, tq, tk, tv = case(7, 4, 700, 64, 4.0)
    *_, pmax = tiled(q, k, v, tq, tk, tv, 64 ** -0.5, fixed_base=True)
    assert pmax > 2.0 ** SLACK
