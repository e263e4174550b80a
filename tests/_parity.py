"""Helpers for the GPU parity tests: seeded device inputs, oracle rows, error norms.

The oracle always recomputes from the seeded generator (workloads/), never from
anything the device produced.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

from oracle import attention_jvp_head
from workloads import TENSORS, head_array
from workloads.device import device_inputs  # noqa: F401  (re-exported for the tests)

# Spec tolerances on O and tO: normalised max error max|x - ref| / max|ref|.
TOL = {"fp32": 1e-5, "bf16": 2e-2}
# lse: |x - ref| <= LSE_TOL * max(1, |ref|).  The kernel sums up to Lk fp32
# terms per row; 1e-4 bounds that rounding with margin for Lk = 32760.
LSE_TOL = {"fp32": 1e-5, "bf16": 1e-4}


def norm_err(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 1.0
    return float(np.max(np.abs(x - ref))) / max(den, 1e-300) if ref.size else 0.0


def lse_err(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    return float(np.max(np.abs(x - ref) / np.maximum(1.0, np.abs(ref)))) if ref.size else 0.0


def oracle_head(w, b, h, rows=None, with_tlse=False):
    a = {t: head_array(w, t, b, h) for t in TENSORS}
    return attention_jvp_head(a["q"], a["k"], a["v"], a["tq"], a["tk"], a["tv"], w.scale, rows=rows,
                              with_tlse=with_tlse)


def compare(w, o, to, lse, rows_fn=None, threads=8, tlse=None):
    """Errors of device outputs against the oracle, over all heads.

    rows_fn(b, h) -> row indices to check (None: all rows).  Returns a dict with
    the global normalised errors and per-head errors of tO; with ``tlse`` (the
    device's tangent of lse) also its normalised error "tlse".
    """
    import torch

    heads = [(b, h) for b in range(w.B) for h in range(w.H)]

    def one(bh):
        b, h = bh
        rows = rows_fn(b, h) if rows_fn else None
        O, tO, L, M = oracle_head(w, b, h, rows, with_tlse=True)
        return bh, rows, O, tO, L, M

    dO = dT = dM = 0.0
    maxO = maxT = maxM = 0.0
    lse_e = 0.0
    per_head = {}
    with ThreadPoolExecutor(threads) as ex:
        for (b, h), rows, O, tO, L, M in ex.map(one, heads):
            idx = torch.as_tensor(rows, device=o.device) if rows is not None else None
            go = (o[b, h] if idx is None else o[b, h].index_select(0, idx)).float().cpu().numpy()
            gt = (to[b, h] if idx is None else to[b, h].index_select(0, idx)).float().cpu().numpy()
            gl = (lse[b, h] if idx is None else lse[b, h].index_select(0, idx)).cpu().numpy()
            dO = max(dO, float(np.max(np.abs(go - O))))
            dT = max(dT, float(np.max(np.abs(gt - tO))))
            maxO = max(maxO, float(np.max(np.abs(O))))
            maxT = max(maxT, float(np.max(np.abs(tO))))
            lse_e = max(lse_e, lse_err(gl, L))
            per_head[(b, h)] = (norm_err(go, O), norm_err(gt, tO))
            if tlse is not None:
                gm = (tlse[b, h] if idx is None else tlse[b, h].index_select(0, idx)).cpu().numpy()
                dM = max(dM, float(np.max(np.abs(gm - M))))
                maxM = max(maxM, float(np.max(np.abs(M))))
    res = {
        "O": dO / max(maxO, 1e-300),
        "tO": dT / max(maxT, 1e-300),
        "lse": lse_e,
        "per_head": per_head,
    }
    if tlse is not None:
        res["tlse"] = dM / max(maxM, 1e-300)
    return res
