"""Upload seeded workload inputs to a device (torch used only for memory)."""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

from .configs import TENSORS
from .inputs import head_upload


def device_inputs(w, device="cuda", threads=8):
    """Allocate the six inputs of workload ``w`` on ``device``; fill head by head."""
    import torch

    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    out = {t: torch.empty(w.shape(t), dtype=tdt, device=device) for t in TENSORS}
    jobs = [(t, b, h) for t in TENSORS for b in range(w.B) for h in range(w.H)]

    def gen(job):
        t, b, h = job
        return job, head_upload(w, t, b, h)

    with ThreadPoolExecutor(threads) as ex:
        for (t, b, h), arr in ex.map(gen, jobs):
            src = torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16) if w.dtype == "bf16" \
                else torch.from_numpy(arr)
            out[t][b, h].copy_(src)
    return out


def device_proj_inputs(w, device="cuda"):
    """The projection inputs of ``w`` on ``device`` as bf16 tensors: x, tx
    [B, L, D] (tx None without tangent), w [F, D], bias [F] (None without bias)."""
    import torch

    from .proj import proj_upload

    def up(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(device)

    out = {"x": torch.empty(w.shape("x"), dtype=torch.bfloat16, device=device)}
    for b in range(w.B):
        out["x"][b].copy_(up(proj_upload(w, "x", b)))
    out["tx"] = None
    if w.tangent:
        out["tx"] = torch.empty(w.shape("tx"), dtype=torch.bfloat16, device=device)
        for b in range(w.B):
            out["tx"][b].copy_(up(proj_upload(w, "tx", b)))
    out["w"] = up(proj_upload(w, "w"))
    out["bias"] = up(proj_upload(w, "bias")) if w.bias else None
    return out


def device_norm_rope_inputs(w, device="cuda", threads=8):
    """The inputs of norm/rope workload ``w`` on ``device``: x, tx [B, H, L, d]
    (tx None without tangent), gamma [d] (None without gain), cos, sin [L, d/2]
    float32 (None without rotation)."""
    import torch

    from .norm_rope import norm_rope_upload, rope_tables

    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def up(arr):
        return (torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16) if w.dtype == "bf16"
                else torch.from_numpy(arr))

    names = ("x", "tx") if w.tangent else ("x",)
    out = {t: torch.empty(w.shape(), dtype=tdt, device=device) for t in names}
    jobs = [(t, b, h) for t in names for b in range(w.B) for h in range(w.H)]
    with ThreadPoolExecutor(threads) as ex:
        for (t, b, h), arr in ex.map(lambda j: (j, norm_rope_upload(w, *j)), jobs):
            out[t][b, h].copy_(up(arr))
    out.setdefault("tx", None)
    out["gamma"] = up(norm_rope_upload(w, "gamma")).to(device) if w.gain else None
    c, s = rope_tables(w)
    out["cos"] = torch.from_numpy(c).to(device) if c is not None else None
    out["sin"] = torch.from_numpy(s).to(device) if s is not None else None
    return out
