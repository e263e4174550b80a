"""Seeded inputs of the projection that feeds attention: hidden states X, their
tangent TX, and the weight W and bias b of a linear layer with n_out*H*d
output features (n_out = 3 for a fused Q/K/V projection).

The rCM pages refactor every layer of the distilled networks to take and return
tangents, and hand the tangents of Q, K and V to the attention kernel laid out
like Q, K and V themselves (ai.info summary of "Large Scale Diffusion
Distillation via Score-Regularized Continuous-Time Consistency", "Methodology in
Plain English" and "Key Contributions" item 1).  The shapes below are the
projections in front of the attention workloads of ``configs.py``: hidden width
D = H*d, the token counts and head layouts of those workloads.  No weight or
dataset is used: every value is drawn from a seeded generator.

Values: X, TX ~ N(0, 1); W ~ N(0, 1/D) (so the projected features are of unit
size); b ~ N(0, 0.1^2).  Each tensor (and each batch of X and TX) has its own
PCG64 stream, ``SeedSequence([0xA77E, seed_id, 100 + tensor_index, b])``;
float32 draws are rounded to bf16 with round-to-nearest-even, and the device
and the oracle both see exactly those rounded values.

This module holds shapes, seeds and rounding only, none of the method's
arithmetic.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .inputs import _SEED_ROOT, bf16_bits_to_f32, f32_to_bf16_bits

PROJ_TENSORS = ("x", "tx", "w", "bias")


@dataclass(frozen=True)
class ProjWorkload:
    name: str
    seed_id: int
    B: int
    L: int
    D: int
    n_out: int
    H: int
    d: int
    tangent: bool = True  # False: a frozen input (no TX, no TY)
    bias: bool = True
    description: str = ""

    @property
    def F(self) -> int:
        """Output features: n_out projections of H heads of d."""
        return self.n_out * self.H * self.d

    @property
    def flops(self) -> float:
        """2*B*L*D*F per product; two products (X W^T, TX W^T) with a tangent."""
        return 2.0 * (2 if self.tangent else 1) * self.B * self.L * self.D * self.F

    @property
    def algorithmic_bytes(self) -> float:
        """Read X (and TX), W and b once; write Y (and TY) once; bf16."""
        n = 2 if self.tangent else 1
        reads = n * self.B * self.L * self.D + self.F * self.D + (self.F if self.bias else 0)
        writes = n * self.B * self.L * self.F
        return 2.0 * (reads + writes)

    def shape(self, tensor: str) -> tuple:
        return {
            "x": (self.B, self.L, self.D),
            "tx": (self.B, self.L, self.D),
            "w": (self.F, self.D),
            "bias": (self.F,),
        }[tensor]

    @property
    def out_shape(self) -> tuple:
        return (self.n_out, self.B, self.H, self.L, self.d)


PROJ_WORKLOADS = {
    w.name: w
    for w in (
        ProjWorkload(
            "qkv_video_bf16", 14, B=1, L=32760, D=5120, n_out=3, H=40, d=128,
            description="Q/K/V projection and its tangent in front of the video self-attention "
            "(32760 tokens, 40 heads of 128)",
        ),
        ProjWorkload(
            "qkv_image_bf16", 12, B=2, L=4096, D=2048, n_out=3, H=16, d=128,
            description="Q/K/V projection and its tangent in front of the image self-attention",
        ),
        ProjWorkload(
            "kv_text_frozen_bf16", 13, B=2, L=512, D=2048, n_out=2, H=16, d=128, tangent=False,
            description="K/V projection of a frozen text context (no tangent), in front of the "
            "text cross-attention",
        ),
    )
}


def custom_proj(B, L, D, n_out, H, d, tangent=True, bias=True, seed_id=2000, name="custom_proj") -> ProjWorkload:
    return ProjWorkload(name, seed_id, B=B, L=L, D=D, n_out=n_out, H=H, d=d, tangent=tangent, bias=bias)


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([_SEED_ROOT, *key])))


def _raw(w: ProjWorkload, tensor: str, b: int = 0) -> np.ndarray:
    ti = 100 + PROJ_TENSORS.index(tensor)
    if tensor in ("x", "tx"):
        return _rng(w.seed_id, ti, b).standard_normal((w.L, w.D), dtype=np.float32)
    if tensor == "w":
        x = _rng(w.seed_id, ti, 0).standard_normal((w.F, w.D), dtype=np.float32)
        x *= np.float32(1.0 / np.sqrt(w.D))
        return x
    x = _rng(w.seed_id, ti, 0).standard_normal((w.F,), dtype=np.float32)
    x *= np.float32(0.1)
    return x


def proj_upload(w: ProjWorkload, tensor: str, b: int = 0) -> np.ndarray:
    """uint16 bf16 bits of one tensor (of batch ``b`` for x and tx)."""
    return f32_to_bf16_bits(_raw(w, tensor, b))


def proj_array(w: ProjWorkload, tensor: str, b: int = 0) -> np.ndarray:
    """float32 values of one tensor exactly as the device receives them."""
    return bf16_bits_to_f32(proj_upload(w, tensor, b))


def proj_host_inputs(w: ProjWorkload) -> dict:
    """All inputs as float32 arrays: x, tx [B, L, D] (tx None without tangent),
    w [F, D], bias [F] (None without bias)."""
    out = {
        "x": np.stack([proj_array(w, "x", b) for b in range(w.B)]),
        "tx": np.stack([proj_array(w, "tx", b) for b in range(w.B)]) if w.tangent else None,
        "w": proj_array(w, "w"),
        "bias": proj_array(w, "bias") if w.bias else None,
    }
    return out
