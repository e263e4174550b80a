"""Seeded inputs of the query/key normalisation and rotary embedding that sit
between the projection and attention: one tensor of rows X [B, H, L, d] (the
queries or the keys of a layer) with its tangent TX, a gain g [d], epsilon,
and the rotation tables cos, sin [L, d/2].

The shapes are the queries (or keys) of the attention workloads of
``configs.py``.  Values: X, TX ~ N(0, 1); g ~ 1 + N(0, 0.1^2).  Rotation
angles follow positions 0 .. L-1 at frequencies base^(-2i/d) (base 10000), the
common rotary recipe: angle[t, i] = t * base^(-2i/d), evaluated in float64 and
stored as float32 cos and sin tables, which both the device and the oracle
read.  Each tensor (and each (batch, head) of X and TX) has its own PCG64
stream, ``SeedSequence([0xA77E, seed_id, 200 + tensor_index, b, h])``; float32
draws are rounded to bf16 (round to nearest even) for bf16 workloads.

This module holds shapes, seeds, rounding and the caller's position tables,
none of the layer's arithmetic.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .inputs import _SEED_ROOT, bf16_bits_to_f32, f32_to_bf16_bits

NORM_ROPE_TENSORS = ("x", "tx", "gamma")


@dataclass(frozen=True)
class NormRopeWorkload:
    name: str
    seed_id: int
    B: int
    H: int
    L: int
    d: int
    dtype: str = "bf16"
    tangent: bool = True
    rope: bool = True      # False: normalisation only (no tables)
    gain: bool = True      # False: no gain (g = 1)
    eps: float = 1e-6
    base: float = 10000.0
    description: str = ""

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    @property
    def rows(self) -> int:
        return self.B * self.H * self.L

    @property
    def algorithmic_bytes(self) -> float:
        """Read X (and TX), write Y (and TY) once, the tables and the gain once."""
        n = 2 if self.tangent else 1
        e = self.elem_bytes
        tables = (2 * self.L * (self.d // 2) * 4) if self.rope else 0
        return float(2 * n * self.rows * self.d * e + tables + (self.d * e if self.gain else 0))

    def shape(self) -> tuple:
        return (self.B, self.H, self.L, self.d)


NORM_ROPE_WORKLOADS = {
    w.name: w
    for w in (
        NormRopeWorkload("q_video_bf16", 21, B=1, H=40, L=32760, d=128,
                         description="queries (or keys) of the video self-attention and their tangent"),
        NormRopeWorkload("q_image_bf16", 22, B=2, H=16, L=4096, d=128,
                         description="queries (or keys) of the image self-attention and their tangent"),
        NormRopeWorkload("k_text_frozen_bf16", 23, B=2, H=16, L=512, d=128, tangent=False, rope=False,
                         description="keys of a frozen text context: normalisation only, no tangent"),
    )
}


def custom_norm_rope(B, H, L, d, dtype="bf16", tangent=True, rope=True, gain=True, eps=1e-6, seed_id=3000,
                     name="custom_norm_rope") -> NormRopeWorkload:
    return NormRopeWorkload(name, seed_id, B=B, H=H, L=L, d=d, dtype=dtype, tangent=tangent, rope=rope, gain=gain,
                            eps=eps)


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([_SEED_ROOT, *key])))


def _raw(w: NormRopeWorkload, tensor: str, b: int = 0, h: int = 0) -> np.ndarray:
    ti = NORM_ROPE_TENSORS.index(tensor)
    if tensor == "gamma":
        g = _rng(w.seed_id, 200 + ti).standard_normal(w.d, dtype=np.float32)
        return np.float32(1.0) + np.float32(0.1) * g
    return _rng(w.seed_id, 200 + ti, b, h).standard_normal((w.L, w.d), dtype=np.float32)


def norm_rope_array(w: NormRopeWorkload, tensor: str, b: int = 0, h: int = 0) -> np.ndarray:
    """float32 values of x / tx (one head, [L, d]) or gamma ([d]) exactly as the
    device receives them."""
    x = _raw(w, tensor, b, h)
    return bf16_bits_to_f32(f32_to_bf16_bits(x)) if w.dtype == "bf16" else x


def norm_rope_upload(w: NormRopeWorkload, tensor: str, b: int = 0, h: int = 0) -> np.ndarray:
    """The bytes to upload: uint16 bf16 bits or float32."""
    x = _raw(w, tensor, b, h)
    return f32_to_bf16_bits(x) if w.dtype == "bf16" else x


def rope_tables(w: NormRopeWorkload):
    """(cos, sin) float32 [L, d/2] for positions 0 .. L-1, or (None, None)."""
    if not w.rope:
        return None, None
    t = np.arange(w.L, dtype=np.float64)[:, None]
    inv = w.base ** (-2.0 * np.arange(w.d // 2, dtype=np.float64) / w.d)
    ang = t * inv[None, :]
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)
