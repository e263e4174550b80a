"""Seeded per-(tensor, batch, head) input generation and bf16 rounding.

Every head of every tensor has its own PCG64 stream, seeded by
``SeedSequence([0xA77E, seed_id, tensor_index, b, h])``, so any single head
(or any set of sampled rows) can be regenerated without producing the whole
tensor.  Draws are float32 standard normals scaled by the tensor's standard
deviation; bf16 workloads are then rounded to bf16 with round-to-nearest-even,
and both the device and the oracle see exactly those rounded values.
"""
from __future__ import annotations

import numpy as np

from .configs import TENSORS, Workload

_SEED_ROOT = 0xA77E


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([_SEED_ROOT, *key])))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round-to-nearest, ties to even); returns uint16 bits.

    Inputs are finite by construction, so no NaN handling is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def tq_head_scale(w: Workload, h: int) -> float:
    """Per-head tangent scale 10**U(-2, 2) (1.0 unless the workload asks for it)."""
    if not w.per_head_tq_scale:
        return 1.0
    u = _rng(w.seed_id, 99).uniform(-2.0, 2.0, size=w.H)
    return float(10.0 ** u[h])


def _raw_head(w: Workload, tensor: str, b: int, h: int) -> np.ndarray:
    ti = TENSORS.index(tensor)
    L = w.Lq if tensor in ("q", "tq") else w.Lk
    std = float(w.std.get(tensor, 1.0))
    if tensor == "tq":
        std *= tq_head_scale(w, h)
    if std == 0.0:
        return np.zeros((L, w.d), dtype=np.float32)
    x = _rng(w.seed_id, ti, b, h).standard_normal((L, w.d), dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if tensor == "k" and w.key_ramp:
        x *= (np.float32(1.0) + np.float32(w.key_ramp) * np.arange(L, dtype=np.float32))[:, None]
    return x


def head_array(w: Workload, tensor: str, b: int, h: int) -> np.ndarray:
    """float32 [L, d] values of one head, exactly as the device receives them."""
    x = _raw_head(w, tensor, b, h)
    if w.dtype == "bf16":
        return bf16_bits_to_f32(f32_to_bf16_bits(x))
    return x


def head_upload(w: Workload, tensor: str, b: int, h: int) -> np.ndarray:
    """The bytes to upload for one head: uint16 bf16 bits, or float32."""
    x = _raw_head(w, tensor, b, h)
    if w.dtype == "bf16":
        return f32_to_bf16_bits(x)
    return x


def sample_rows(w: Workload, b: int, h: int, n_random: int = 224) -> np.ndarray:
    """Query rows checked on the large workloads: both edges of the first
    128-row tile, the last rows (inside the ragged tail tile when Lq is not a
    multiple of 128), plus ``n_random`` seeded random rows; sorted, unique."""
    Lq = w.Lq
    fixed = set(range(0, min(8, Lq)))
    fixed |= set(r for r in range(120, 136) if r < Lq)
    fixed |= set(range(max(0, Lq - 8), Lq))
    rest = np.array(sorted(set(range(Lq)) - fixed), dtype=np.int64)
    n = min(n_random, rest.size)
    pick = _rng(w.seed_id, 77, b, h).choice(rest, size=n, replace=False) if n else rest[:0]
    return np.array(sorted(fixed | set(int(r) for r in pick)), dtype=np.int64)
