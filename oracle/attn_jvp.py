"""Plain fp64 CPU oracle: softmax attention and its forward-mode derivative.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check of the entry
point and the ``cpu_baseline`` leg of the benchmark use it.  It shares no code,
constant or helper with the HIP library; the two meet only through the seeded
inputs of ``workloads/``.

What is computed
----------------
The rCM pages describe a FlashAttention-2 kernel that returns, besides the
attention output, its Jacobian-vector product, for self- and cross-attention
(papernotes.org reading notes on "Large Scale Diffusion Distillation via
Score-Regularized Continuous-Time Consistency", section "Key designs", item 1;
ai.info summary of the same paper, "Key Contributions" item 1).  The notes on
"Consistent Distribution Matching for Data-Free Diffusion Distillation"
(prerequisites, "JVP") define a JVP as the Jacobian of f applied to a tangent
vector, obtained in one forward pass without forming the Jacobian.  The pages
never print the attention formulas, so this module writes out the plain
definition for f(Q, K, V) = softmax(scale * Q K^T) V along (tQ, tK, tV), per
(batch, head), in float64, with no tiling, fusion or reordering:

  1. S   = scale * Q K^T
  2. P   = row-softmax(S)     (row max subtracted first, for range only)
  3. O   = P V;   lse = log of the row sum of exp(S)   (natural log)
  4. tS  = scale * (tQ K^T + Q tK^T)      (scale is a constant: no tangent)
  5. mu  = row sum of P * tS              (the tangent of lse)
  6. tO  = P tV + (P * (tS - mu)) V

Step 6 is the product rule through O = P V plus the derivative of the
row softmax, dP = P * (dS - rowsum(P * dS)).

Readings where the pages are silent: scale carries no tangent; lse is the
natural log of the row sum over the scaled logits; there is no mask, dropout or
bias (every query attends to all Lk keys); tensors are [..., L, d].

Key shards (``merge_shards``): the pages call the fused kernel compatible
with context parallelism, the tangents of Q, K and V distributed like Q, K and
V (ai.info summary, "Methodology in Plain English").  Over disjoint key shards
s, each with its own softmax P_s, O_s, tO_s, lse_s and mu_s (steps 1-6 on its
keys), the softmax over all keys is w_s P_s with w_s = exp(lse_s - lse),
lse = log sum_s exp(lse_s).  Substituting into steps 3, 5 and 6:
  O = sum_s w_s O_s,   mu = sum_s w_s mu_s,
  tO = sum_s w_s (tO_s + (mu_s - mu) O_s).

Pins (tests/test_oracle_pins.py): torch.func.jvp in float64, central finite
differences, complex-step differentiation, a brute-force Jacobian, closed forms
(uniform attention, Lk = 1), invariants of the tangent map, scipy's logsumexp
and torch's scaled_dot_product_attention for O.
"""
from __future__ import annotations

import numpy as np


def attention_jvp_head(q, k, v, tq, tk, tv, scale, rows=None, with_tlse=False):
    """One head.  q, tq: [Lq, d]; k, v, tk, tv: [Lk, d].

    ``rows`` restricts the computation to those query rows (every output row
    depends only on its own q, tq rows and on all of k, v, tk, tv).
    Returns (O [R, d], tO [R, d], lse [R]) in float64, and mu [R] (the tangent
    of lse, step 5) as a fourth value when ``with_tlse``.
    """
    f64 = np.float64
    q = np.asarray(q, dtype=f64)
    tq = np.asarray(tq, dtype=f64)
    k = np.asarray(k, dtype=f64)
    v = np.asarray(v, dtype=f64)
    tk = np.asarray(tk, dtype=f64)
    tv = np.asarray(tv, dtype=f64)
    if rows is not None:
        q = q[rows]
        tq = tq[rows]
    s = f64(scale)

    S = s * (q @ k.T)                                   # step 1
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    Z = E.sum(axis=1, keepdims=True)
    P = E / Z                                           # step 2
    O = P @ v                                           # step 3
    lse = m[:, 0] + np.log(Z[:, 0])
    tS = s * (tq @ k.T + q @ tk.T)                      # step 4
    mu = (P * tS).sum(axis=1, keepdims=True)            # step 5
    tO = P @ tv + (P * (tS - mu)) @ v                   # step 6
    if with_tlse:
        return O, tO, lse, mu[:, 0]
    return O, tO, lse


def merge_shards(parts):
    """Combine per-shard results [(O_s, tO_s, lse_s, mu_s), ...] of disjoint
    key shards (any leading shape, float64) into the result over all keys:
    the formulas in the module docstring.  Returns (O, tO, lse, mu)."""
    lse_s = np.stack([np.asarray(p[2], dtype=np.float64) for p in parts])
    mu_s = np.stack([np.asarray(p[3], dtype=np.float64) for p in parts])
    top = lse_s.max(axis=0)
    lse = top + np.log(np.exp(lse_s - top).sum(axis=0))
    w = np.exp(lse_s - lse)
    mu = (w * mu_s).sum(axis=0)
    O = sum(w[i][..., None] * np.asarray(p[0], dtype=np.float64) for i, p in enumerate(parts))
    tO = sum(
        w[i][..., None] * (np.asarray(p[1], dtype=np.float64) + (mu_s[i] - mu)[..., None] * np.asarray(p[0], dtype=np.float64))
        for i, p in enumerate(parts)
    )
    return O, tO, lse, mu


def attention_jvp(q, k, v, tq, tk, tv, scale, rows=None, with_tlse=False):
    """Batched over leading dims: q, tq [..., Lq, d]; k, v, tk, tv [..., Lk, d].

    ``rows`` (optional) is either one index array used for every head, or a
    callable ``rows(index_tuple) -> index array`` giving each head its rows.
    """
    q = np.asarray(q)
    lead = q.shape[:-2]
    outs_o, outs_t, outs_l, outs_m = [], [], [], []
    for idx in np.ndindex(*lead):
        r = rows(idx) if callable(rows) else rows
        res = attention_jvp_head(q[idx], k[idx], v[idx], tq[idx], tk[idx], tv[idx], scale, r, with_tlse=True)
        outs_o.append(res[0])
        outs_t.append(res[1])
        outs_l.append(res[2])
        outs_m.append(res[3])
    R = outs_o[0].shape[0]
    d = outs_o[0].shape[1]
    if callable(rows):
        return (outs_o, outs_t, outs_l, outs_m) if with_tlse else (outs_o, outs_t, outs_l)
    res = (
        np.stack(outs_o).reshape(*lead, R, d),
        np.stack(outs_t).reshape(*lead, R, d),
        np.stack(outs_l).reshape(*lead, R),
    )
    if with_tlse:
        return res + (np.stack(outs_m).reshape(*lead, R),)
    return res
