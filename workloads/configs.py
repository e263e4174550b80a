"""The attention-JVP workloads: shapes, dtypes and value distributions.

The shapes stand in for the attention layers of the models that the rCM pages
distil (ai.info summary of "Large Scale Diffusion Distillation via
Score-Regularized Continuous-Time Consistency", Main Findings: Cosmos-Predict2
text-to-image at 1360x768 and Wan2.1 480p video at 832x480x81).  No dataset,
prompt or weight is used: every tensor is drawn from a seeded generator.

  * 32760 = 21 x 30 x 52 latent video tokens, 4096 ~ 1360*768/16^2 image tokens,
    512 text tokens for cross-attention.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

TENSORS = ("q", "k", "v", "tq", "tk", "tv")


@dataclass(frozen=True)
class Workload:
    name: str
    seed_id: int
    B: int
    H: int
    Lq: int
    Lk: int
    d: int
    dtype: str  # "fp32" or "bf16": inputs, O and tO; lse is always fp32
    std: dict = field(default_factory=dict)  # per-tensor standard deviation
    # When set, tq of head h is additionally scaled by 10**U(-2, 2) drawn per head.
    per_head_tq_scale: bool = False
    # Key row j is additionally scaled by 1 + key_ramp * j (0: no ramp): logits
    # that grow along the keys, so the row max keeps rising tile after tile.
    key_ramp: float = 0.0
    description: str = ""

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def flops(self) -> float:
        """Nominal work: the six dense products, 2*Lq*Lk*d flops each."""
        return 12.0 * self.B * self.H * self.Lq * self.Lk * self.d

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    @property
    def algorithmic_bytes(self) -> float:
        """Bytes a single pass must move: read Q,tQ,K,tK,V,tV once, write O,tO,lse."""
        e = self.elem_bytes
        B, H = self.B, self.H
        reads = (2 * B * H * self.Lq * self.d + 4 * B * H * self.Lk * self.d) * e
        writes = 2 * B * H * self.Lq * self.d * e + 4 * B * H * self.Lq
        return float(reads + writes)

    def shape(self, tensor: str) -> tuple:
        L = self.Lq if tensor in ("q", "tq") else self.Lk
        return (self.B, self.H, L, self.d)


def _std(q=1.0, k=1.0, v=1.0, tq=1.0, tk=1.0, tv=1.0) -> dict:
    return {"q": q, "k": k, "v": v, "tq": tq, "tk": tk, "tv": tv}


_SQRT8 = math.sqrt(8.0)  # std(scale * q.k) = sigma_q * sigma_k when scale = d**-0.5

WORKLOADS = {
    w.name: w
    for w in (
        Workload(
            "tiny_self_fp32", 1, B=1, H=2, Lq=128, Lk=128, d=64, dtype="fp32", std=_std(),
            description="tiny self-attention JVP, fp32 in/out/compute",
        ),
        Workload(
            "image_self_bf16", 2, B=2, H=16, Lq=4096, Lk=4096, d=128, dtype="bf16",
            std=_std(tq=0.5, tk=0.5, tv=0.5),
            description="image-token self-attention JVP (64x64 latent patches)",
        ),
        Workload(
            "image_self_fp32", 6, B=2, H=16, Lq=4096, Lk=4096, d=128, dtype="fp32",
            std=_std(tq=0.5, tk=0.5, tv=0.5),
            description="the image-token self-attention JVP in fp32 in/out/compute",
        ),
        Workload(
            "text_cross_bf16", 3, B=2, H=16, Lq=4096, Lk=512, d=128, dtype="bf16",
            std=_std(tk=0.0, tv=0.0),
            description="image queries x text keys, frozen text context (tK = tV = 0)",
        ),
        Workload(
            "video_self_bf16", 4, B=1, H=40, Lq=32760, Lk=32760, d=128, dtype="bf16", std=_std(),
            description="video-token self-attention JVP (21x30x52 latent tokens), one GPU's layer",
        ),
        Workload(
            "video_self_d64_bf16", 7, B=1, H=80, Lq=32760, Lk=32760, d=64, dtype="bf16", std=_std(),
            description="the video self-attention layer's width split into 80 heads of 64",
        ),
        Workload(
            "video_self_cp_shard_bf16", 8, B=1, H=5, Lq=4095, Lk=32760, d=128, dtype="bf16", std=_std(),
            description="one GPU's share of the video self-attention layer sharded 8 ways over heads and 8 "
            "over queries (5 heads, 4095 queries, all 32760 keys): 160 workgroups, fewer than the CUs",
        ),
        Workload(
            "video_cross_stress_bf16", 5, B=1, H=40, Lq=32760, Lk=512, d=128, dtype="bf16",
            std=_std(q=_SQRT8, k=_SQRT8), per_head_tq_scale=True,
            description="video cross-attention with peaky softmax (logit std ~ 8) and "
            "per-head tangent scales log-uniform in [1e-2, 1e2]",
        ),
    )
}


def custom_workload(B, H, Lq, Lk, d, dtype, seed_id=1000, std=None, name="custom", key_ramp=0.0) -> Workload:
    """An ad-hoc shape (ragged tails, edge cases) with the default N(0,1) inputs."""
    return Workload(name, seed_id, B=B, H=H, Lq=Lq, Lk=Lk, d=d, dtype=dtype, std=std or _std(),
                    key_ramp=key_ramp)
