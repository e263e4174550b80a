"""GPU: the projection's tile edges, against the fp64 oracle.

Grids of at most 128 workgroups of the 256-feature tiling run 128-feature
tiles (without a tangent with 128-wide hidden steps when D % 128 == 0, else
the 256-feature tiles).  This sweep covers hidden sizes of one to three steps
of either width (and widths that select the fallback), feature counts that
leave partial 128- and 256-feature tiles, and token counts at the 128-token
tile edge, with and without the tangent and the bias, every output checked.
"""
import numpy as np
import pytest
import torch

from oracle import projection_jvp
from workloads import custom_proj, proj_host_inputs
from workloads.device import device_proj_inputs

pytestmark = pytest.mark.gpu

REL = 2.0 ** -8
ABS = 2e-4


@pytest.fixture(scope="module")
def A():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_forward_mode_attn_amd as A

    A.load_library()
    return A


HEADS = [  # (n_out, H, d): F = n_out * H * d features
    (1, 1, 64),    # 64: one partial 128-feature tile
    (1, 1, 128),   # 128
    (3, 1, 64),    # 192: a full and a partial narrow tile
    (3, 1, 128),   # 384
    (1, 5, 64),    # 320
    (2, 5, 64),    # 640: a partial wide tile as well
]


@pytest.mark.parametrize("tangent", [True, False])
@pytest.mark.parametrize("D", [64, 128, 192, 256, 384])
def test_projection_tile_edges(A, tangent, D):
    bad = []
    for i, (n_out, H, d) in enumerate(HEADS):
        for L in (1, 127, 129):
            bias = (i + L) % 2 == 0
            w = custom_proj(1, L, D, n_out, H, d, tangent=tangent, bias=bias, seed_id=8300 + 7 * D + 3 * i + L)
            print(f"case proj edge L{L} D{D} n_out{n_out} H{H} d{d} tangent={tangent} bias={bias}", flush=True)
            h = proj_host_inputs(w)
            x = device_proj_inputs(w)
            y, ty = A.proj(x["x"], x["tx"], x["w"], x["bias"], n_out=n_out, heads=H)
            torch.cuda.synchronize()
            Y, TY = projection_jvp(h["x"], h["tx"], h["w"], h["bias"], n_out, H, d)
            for got, ref in ((y, Y), (ty, TY)):
                if ref is None:
                    continue
                err = np.abs(got.float().cpu().numpy() - ref)
                if not np.all(err <= REL * np.abs(ref) + ABS * np.abs(ref).max()):
                    print(f"  max error {err.max():.3e}", flush=True)
                    bad.append((L, n_out, H, d))
    assert not bad, bad
