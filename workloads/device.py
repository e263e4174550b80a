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
