"""GPU parity of the projection into attention heads and its tangent
(``attn_jvp_proj``), through the C ABI, against the fp64 oracle
``oracle.projection_jvp`` on the same seeded bf16 inputs.

Tolerance, from the arithmetic: every output is one fp32 accumulation of D
bf16 products (exact in fp32) rounded once to bf16 with round-to-nearest-even,
so |y - ref| <= 2^-8 |ref| (half an ulp of an 8-bit significand) plus the fp32
accumulation error, bounded here by 2e-4 * max|ref| (D <= 5120 terms of
relative rounding 2^-24 each, with margin).  Any index, layout or operand
mistake breaks this by orders of magnitude.
"""
import numpy as np
import pytest
import torch

from oracle import attention_jvp_head, projection_jvp
from workloads import PROJ_WORKLOADS, custom_proj, proj_host_inputs
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


def check(got, ref, label):
    got = got.float().cpu().numpy().astype(np.float64)
    err = np.abs(got - ref)
    bound = REL * np.abs(ref) + ABS * np.abs(ref).max()
    worst = float((err / bound).max())
    print(f"  {label}: max err {err.max():.3e} (max |ref| {np.abs(ref).max():.3e}), worst err/bound {worst:.3f}",
          flush=True)
    assert worst <= 1.0, label


def run_case(A, w, rows=None):
    h = proj_host_inputs(w)
    x = device_proj_inputs(w)
    y, ty = A.proj(x["x"], x["tx"], x["w"], x["bias"], n_out=w.n_out, heads=w.H)
    torch.cuda.synchronize()
    Y, TY = projection_jvp(h["x"], h["tx"], h["w"], h["bias"], w.n_out, w.H, w.d, rows=rows)
    sel = (lambda t: t) if rows is None else (lambda t: t[:, :, :, torch.as_tensor(rows, device=t.device)])
    check(sel(y), Y, "Y")
    if w.tangent:
        check(sel(ty), TY, "TY")
    else:
        assert ty is None
    return x, y, ty


SHAPES = [
    # (B, L, D, n_out, H, d, tangent, bias)
    (2, 200, 192, 3, 2, 128, True, True),     # ragged token tile, three steps, 3 feature tiles
    (1, 129, 64, 3, 3, 64, True, True),       # one step; last feature tile holds 64 features
    (2, 77, 128, 2, 2, 128, False, True),     # frozen input: no tangent
    (3, 1, 256, 1, 1, 128, True, False),      # a single token; 128 features; no bias
    (1, 128, 512, 3, 4, 64, True, True),      # exact tiles, d = 64 heads
    (1, 300, 320, 2, 3, 64, False, False),    # frozen, no bias, ragged everything
]


# Grids of at most 128 workgroups of the 256-feature tiling run 128-feature
# tiles (without a tangent with a 128-wide hidden step when D % 128 == 0).
def wide_grid(B, L, n_out, H, d):
    return -(-n_out * H * d // 256) * -(-L // 128) * B


TILE_SHAPES = [
    # (B, L, D, n_out, H, d, tangent, bias): narrow tiles
    (1, 100, 128, 3, 1, 64, False, True),     # frozen, one 128-wide step, partial feature tile (192)
    (2, 257, 256, 2, 2, 64, False, True),     # frozen, two steps, ragged tokens
    (1, 130, 384, 3, 2, 128, False, False),   # frozen, three steps, no bias
    (1, 90, 64, 3, 1, 64, True, True),        # tangent, one 64-wide step, partial feature tile
    (2, 200, 192, 1, 3, 128, True, False),    # tangent, three steps
    (1, 5376, 128, 3, 2, 128, False, True),   # frozen at the switch: 42 token x 3 feature tiles = 126
    (1, 5376, 64, 3, 2, 128, True, True),     # tangent at the switch
    # wide tiles
    (1, 5504, 128, 3, 2, 128, False, True),   # frozen just past the switch: 129 workgroups
    (1, 5504, 64, 3, 2, 128, True, True),     # tangent just past the switch
    (1, 4096, 256, 2, 8, 128, False, True),   # frozen, 256 workgroups
    (1, 200, 192, 2, 2, 64, False, True),     # frozen narrow grid, D % 128 != 0: wide tiles
]


@pytest.mark.parametrize("B,L,D,n_out,H,d,tangent,bias", TILE_SHAPES)
def test_tile_shapes_match_oracle(A, B, L, D, n_out, H, d, tangent, bias):
    narrow = wide_grid(B, L, n_out, H, d) <= 128 and (tangent or D % 128 == 0)
    w = custom_proj(B, L, D, n_out, H, d, tangent=tangent, bias=bias, seed_id=2300 + L + D + n_out)
    print(f"case proj {'narrow' if narrow else 'wide'} tiles B{B} L{L} D{D} n_out{n_out} H{H} d{d} "
          f"tangent={tangent} bias={bias}", flush=True)
    run_case(A, w)


@pytest.mark.parametrize("tangent", [False, True])
def test_narrow_tiles_equal_wide_tiles_bitwise(A, tangent):
    """Both tilings sum each output's hidden chunks of 16 in the same order, so a
    batch element projected alone (a narrow grid) and inside a batch large enough
    for the wide tiles must agree bit for bit."""
    L, D, n_out, H, d = 300, 256, 3, 2, 64
    B = 1
    while wide_grid(B, L, n_out, H, d) <= 128:
        B += 1
    assert wide_grid(1, L, n_out, H, d) <= 128
    w = custom_proj(B, L, D, n_out, H, d, tangent=tangent, seed_id=2400 + int(tangent))
    print(f"case proj narrow vs wide bitwise B{B} L{L} D{D} tangent={tangent}", flush=True)
    x = device_proj_inputs(w)
    y, ty = A.proj(x["x"], x["tx"], x["w"], x["bias"], n_out=n_out, heads=H)
    x1 = x["x"][:1].contiguous()
    tx1 = x["tx"][:1].contiguous() if tangent else None
    y1, ty1 = A.proj(x1, tx1, x["w"], x["bias"], n_out=n_out, heads=H)
    torch.cuda.synchronize()
    assert torch.equal(y[:, :1], y1)
    if tangent:
        assert torch.equal(ty[:, :1], ty1)


@pytest.mark.parametrize("B,L,D,n_out,H,d,tangent,bias", SHAPES)
def test_projection_matches_oracle(A, B, L, D, n_out, H, d, tangent, bias):
    w = custom_proj(B, L, D, n_out, H, d, tangent=tangent, bias=bias, seed_id=2100 + L + D)
    print(f"case proj B{B} L{L} D{D} n_out{n_out} H{H} d{d} tangent={tangent} bias={bias}", flush=True)
    run_case(A, w)


def test_outputs_stay_inside_their_buffers(A):
    """Outputs written through offset views of guarded buffers: the guard bands
    before and after keep their sentinel values, and every output element is
    written (no sentinel left inside)."""
    w = custom_proj(2, 150, 128, 3, 2, 64, seed_id=2201)
    print("case proj guard bands", flush=True)
    x = device_proj_inputs(w)
    n = int(np.prod(w.out_shape))
    guard = 4096
    sentinel = torch.tensor(-12345.0, dtype=torch.bfloat16)
    bufs = [torch.full((n + 2 * guard,), sentinel.item(), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    outs = tuple(b[guard:guard + n].view(w.out_shape) for b in bufs)
    A.proj(x["x"], x["tx"], x["w"], x["bias"], n_out=w.n_out, heads=w.H, out=outs)
    torch.cuda.synchronize()
    for b in bufs:
        assert bool((b[:guard] == sentinel).all()) and bool((b[guard + n:] == sentinel).all())
        assert not bool((b[guard:guard + n] == sentinel).any())


def test_wrong_output_buffers_are_rejected(A):
    w = custom_proj(1, 40, 64, 3, 2, 64, seed_id=2202)
    print("case proj wrong output buffers", flush=True)
    x = device_proj_inputs(w)
    y = torch.empty(w.out_shape, dtype=torch.bfloat16, device="cuda")
    short = torch.empty((3, 1, 2, 39, 64), dtype=torch.bfloat16, device="cuda")
    for out in ((short, y), (y, short), (y, y.float()), (y, None)):
        with pytest.raises(ValueError):
            A.proj(x["x"], x["tx"], x["w"], x["bias"], n_out=3, heads=2, out=out)
    with pytest.raises(ValueError):
        A.proj(x["x"], None, x["w"], x["bias"], n_out=3, heads=2, out=(y, y))


def test_bitwise_deterministic(A):
    w = custom_proj(1, 260, 256, 3, 2, 128, seed_id=2202)
    print("case proj determinism", flush=True)
    x = device_proj_inputs(w)
    y1, t1 = A.proj(x["x"], x["tx"], x["w"], x["bias"], n_out=3, heads=2)
    y2, t2 = A.proj(x["x"], x["tx"], x["w"], x["bias"], n_out=3, heads=2)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2) and torch.equal(t1, t2)


def test_tangent_path_primal_equals_frozen_path(A):
    """The primal output does not depend on whether the tangent is computed."""
    w = custom_proj(1, 140, 192, 2, 2, 128, seed_id=2203)
    print("case proj primal with and without tangent", flush=True)
    x = device_proj_inputs(w)
    y1, _ = A.proj(x["x"], x["tx"], x["w"], x["bias"], n_out=2, heads=2)
    y2, t2 = A.proj(x["x"], None, x["w"], x["bias"], n_out=2, heads=2)
    torch.cuda.synchronize()
    assert t2 is None and torch.equal(y1, y2)


@pytest.mark.parametrize("name", ["qkv_image_bf16", "kv_text_frozen_bf16"])
def test_full_size_projection(A, name):
    w = PROJ_WORKLOADS[name]
    print(f"case proj {name} (sampled tokens)", flush=True)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([np.arange(8), np.arange(120, 136), np.arange(w.L - 8, w.L),
                                     rng.choice(w.L, 96, replace=False)]))
    run_case(A, w, rows=rows)


def test_video_projection_sampled(A):
    """The video Q/K/V projection at full size (32760 tokens, D = 5120,
    15360 features), checked on sampled tokens across all features."""
    w = PROJ_WORKLOADS["qkv_video_bf16"]
    print("case proj qkv_video_bf16 (sampled tokens)", flush=True)
    rng = np.random.default_rng(6)
    rows = np.unique(np.concatenate([np.arange(8), np.arange(120, 136), np.arange(w.L - 8, w.L),
                                     rng.choice(w.L, 40, replace=False)]))
    run_case(A, w, rows=rows)


def test_projection_feeds_attention(A):
    """proj -> fwd on the device equals the fp64 composition of the two oracles
    (the device rounds Q, K, V and their tangents to bf16 in between, which the
    attention tolerance of the bf16 path covers)."""
    w = custom_proj(1, 230, 256, 3, 2, 128, seed_id=2204)
    print("case proj -> attention", flush=True)
    h = proj_host_inputs(w)
    x = device_proj_inputs(w)
    y, ty = A.proj(x["x"], x["tx"], x["w"], x["bias"], n_out=3, heads=2)
    o, to, lse = A.fwd(y[0], y[1], y[2], ty[0], ty[1], ty[2])
    torch.cuda.synchronize()
    Y, TY = projection_jvp(h["x"], h["tx"], h["w"], h["bias"], 3, 2, 128)
    s = 128 ** -0.5
    for hd in range(2):
        O, tO, L = attention_jvp_head(Y[0, 0, hd], Y[1, 0, hd], Y[2, 0, hd], TY[0, 0, hd], TY[1, 0, hd],
                                      TY[2, 0, hd], s)
        eo = np.abs(o[0, hd].float().cpu().numpy() - O).max() / np.abs(O).max()
        et = np.abs(to[0, hd].float().cpu().numpy() - tO).max() / np.abs(tO).max()
        print(f"  head {hd}: O {eo:.3e} tO {et:.3e}", flush=True)
        assert eo <= 2e-2 and et <= 2e-2
