"""Plain fp64 CPU oracle: the projection of hidden states into attention heads
and its forward-mode derivative.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check of the entry
point and the ``cpu_baseline`` leg of the benchmark use it.  It shares no code,
constant or helper with the HIP library; the two meet only through the seeded
inputs of ``workloads/``.

What is computed
----------------
The rCM pages make every layer of the distilled networks take and return
tangents, so that the JVP composes layer by layer under sharding, and hand the
tangents of Q, K and V to the attention kernel distributed like Q, K and V
(ai.info summary of "Large Scale Diffusion Distillation via Score-Regularized
Continuous-Time Consistency", "Methodology in Plain English"; same summary,
"Key Contributions" item 1).  The pages name no architecture; the layer that
emits Q, K, V and their tangents from a hidden state is read as a linear map
with bias.  With hidden states X [B, L, D], their tangent TX, a weight
W [F, D] and a bias b [F] (F = n_out * H * d output features), in float64:

  1. Y  = X W^T + b
  2. TY = TX W^T        (the JVP of an affine map is its linear part applied
                         to the tangent; the constant b has no tangent)
  3. output feature f = (n * H + h) * d + j of token t of batch b is element
     [n, b, h, t, j] of the result: projection n (Q, K, V for n_out = 3),
     head h, in the [B, H, L, d] layout the attention oracle and kernel take.

Pins (tests/test_oracle_proj_pins.py): central finite differences of the
primal map, a brute-force loop over the sum, a permutation weight that routes
named input features to named output slots, the bias's absence from the
tangent, linearity in the tangent, and the chain rule through the attention
oracle (finite differences of the composed primal map).
"""
from __future__ import annotations

import numpy as np


def projection_jvp(x, tx, w, bias, n_out, H, d, rows=None):
    """x, tx: [B, L, D] (tx may be None: no tangent); w: [F, D] with
    F = n_out*H*d; bias: [F] or None.  ``rows`` restricts the result to those
    token indices (of every batch).  Returns (Y, TY) in float64, each
    [n_out, B, H, R, d]; TY is None when tx is None."""
    f64 = np.float64
    x = np.asarray(x, dtype=f64)
    w = np.asarray(w, dtype=f64)
    if rows is not None:
        x = x[:, rows]
    B, R, _ = x.shape
    F = n_out * H * d
    if w.shape[0] != F:
        raise ValueError("w must have n_out*H*d rows")

    def heads(z):  # step 3: [B, R, F] -> [n_out, B, H, R, d]
        return z.reshape(B, R, n_out, H, d).transpose(2, 0, 3, 1, 4)

    Y = x @ w.T                                               # step 1
    if bias is not None:
        Y = Y + np.asarray(bias, dtype=f64)
    TY = None
    if tx is not None:
        tx = np.asarray(tx, dtype=f64)
        if rows is not None:
            tx = tx[:, rows]
        TY = heads(tx @ w.T)                                  # step 2
    return heads(Y), TY
