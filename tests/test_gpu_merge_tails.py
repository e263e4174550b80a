"""GPU: the merge kernel at every row count up to 70, against the fp64 merge.

attn_jvp_merge handles 8 elements of a row per thread and 2048/d (bf16) or
1024/d (float32) rows per workgroup; these cases cover every row count up to
two workgroups and a tail, 2, 5 and 16 parts, d 64 and 128, and the three
precision modes (float32 parts to float32, bf16 to bf16, float32 parts to
bf16).  The partial results are seeded synthetic values (lse spread over a
range of ±6 so that the weights differ by orders of magnitude); the reference
is the oracle's fp64 merge of exactly the values the device reads.
"""
import numpy as np
import pytest
import torch

from oracle import merge_shards

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def A():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_forward_mode_attn_amd as A

    A.load_library()
    return A


MODES = {
    # name: (part dtype, result dtype)
    "fp32": (torch.float32, torch.float32),
    "bf16": (torch.bfloat16, torch.bfloat16),
    "f32parts_bf16": (torch.float32, torch.bfloat16),
}


@pytest.mark.parametrize("mode", sorted(MODES))
@pytest.mark.parametrize("d", [64, 128])
def test_merge_every_row_count(A, mode, d):
    pdt, odt = MODES[mode]
    bad = []
    for n in (2, 5, 16):
        for rows in range(1, 71):
            rng = np.random.default_rng([9000, d, n, rows, sorted(MODES).index(mode)])
            print(f"case merge {mode} d{d} n{n} rows{rows}", flush=True)
            parts_dev, parts_ref = [], []
            for _ in range(n):
                o = torch.from_numpy(rng.standard_normal((rows, d)).astype(np.float32)).to(pdt)
                to = torch.from_numpy(rng.standard_normal((rows, d)).astype(np.float32)).to(pdt)
                lse = torch.from_numpy(rng.uniform(-6.0, 6.0, rows).astype(np.float32))
                tlse = torch.from_numpy(rng.standard_normal(rows).astype(np.float32))
                parts_dev.append(tuple(t.cuda() for t in (o, to, lse, tlse)))
                parts_ref.append(tuple(t.double().numpy() for t in (o.float(), to.float(), lse, tlse)))
            got = A.merge(parts_dev, out_dtype=odt)
            torch.cuda.synchronize()
            ref = merge_shards(parts_ref)
            for name, g, r in zip(("O", "tO", "lse", "tlse"), got, ref):
                g = g.float().cpu().numpy().astype(np.float64)
                scale = max(np.abs(r).max(), 1.0)
                if name in ("O", "tO") and odt == torch.bfloat16:
                    ok = np.all(np.abs(g - r) <= 2.0 ** -8 * np.abs(r) + 1e-5 * scale)
                else:
                    ok = np.abs(g - r).max() <= 1e-5 * scale
                if not ok:
                    print(f"  {name}: max error {np.abs(g - r).max():.3e}", flush=True)
                    bad.append((n, rows, name))
    assert not bad, bad[:10]
