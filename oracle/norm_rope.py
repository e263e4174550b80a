"""Plain fp64 CPU oracle: RMS normalisation and rotary position embedding of
queries or keys, with their forward-mode derivative.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the test suite, the smoke check of the entry
point and the ``cpu_baseline`` leg of the benchmark use it.  It shares no code,
constant or helper with the HIP library; the two meet only through the seeded
inputs of ``workloads/``.

What is computed
----------------
The rCM pages refactor every layer of the distilled networks to take and
return tangents, and hand the tangents of Q and K to the attention kernel laid
out like Q and K (ai.info summary of "Large Scale Diffusion Distillation via
Score-Regularized Continuous-Time Consistency", "Methodology in Plain English"
and "Key Contributions" item 1).  They do not describe what lies between the
projection and the attention product.  The reading taken here is the one the
projection oracle leaves open: queries and keys are RMS-normalised over the
head dimension with a gain, then rotated pairwise by a rotary position
embedding whose angles depend on the token's position.  Gain, epsilon and
angles are constants (no tangent).  Pairs are adjacent elements (2i, 2i + 1);
the angles come as tables cos[t, i], sin[t, i] (any position scheme can be
written into them).  For one row x in R^d (token t of one head), its tangent
tx, gain g in R^d and eps >= 0, in float64:

  1. m  = mean_j x_j^2,   r = (m + eps)^(-1/2)
  2. n  = g * x * r
  3. y_{2i} = c_i n_{2i} - s_i n_{2i+1},   y_{2i+1} = s_i n_{2i} + c_i n_{2i+1}
     with c_i = cos[t, i], s_i = sin[t, i]
  4. tn = g * (tx * r - x * r^3 * mean_j(x_j tx_j))
     (step 2 differentiated along tx: dm = 2 mean(x dx), dr = -r^3 mean(x dx))
  5. ty = the rotation of step 3 applied to tn (the rotation is linear and its
     angles are constants)

Without tables (cos = sin = None) the rotation is the identity; without a
gain, g = 1.

Pins (tests/test_oracle_norm_rope_pins.py): torch.func.jvp through torch's
rms_norm and a rotation written with complex numbers, central finite
differences, a hand-worked example (tests/golden/norm_rope_hand_example.json),
pair-norm preservation, unit RMS, scale invariance, the identity rotation,
rotation there and back, linearity in the tangent, the pairing and sign
convention, and planted mistakes.
"""
from __future__ import annotations

import numpy as np


def norm_rope_jvp(x, tx, gamma, cos, sin, eps):
    """x: [..., L, d] (each row a token of one head); tx: same shape or None;
    gamma: [d] or None; cos, sin: [L, d/2] or both None; eps >= 0.

    Returns (y, ty) in float64; ty is None when tx is None."""
    f64 = np.float64
    x = np.asarray(x, dtype=f64)
    d = x.shape[-1]
    g = np.ones(d, dtype=f64) if gamma is None else np.asarray(gamma, dtype=f64)

    m = np.mean(x * x, axis=-1, keepdims=True)                  # step 1
    r = 1.0 / np.sqrt(m + eps)
    n = g * x * r                                               # step 2

    def rotate(z):                                              # steps 3 and 5
        if cos is None:
            return z
        c = np.asarray(cos, dtype=f64)
        s = np.asarray(sin, dtype=f64)
        even, odd = z[..., 0::2], z[..., 1::2]
        out = np.empty_like(z)
        out[..., 0::2] = c * even - s * odd
        out[..., 1::2] = s * even + c * odd
        return out

    y = rotate(n)
    if tx is None:
        return y, None
    tx = np.asarray(tx, dtype=f64)
    xt = np.mean(x * tx, axis=-1, keepdims=True)
    tn = g * (tx * r - x * r ** 3 * xt)                         # step 4
    return y, rotate(tn)
