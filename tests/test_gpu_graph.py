"""The C-ABI calls inside a captured HIP graph (torch.cuda.CUDAGraph on ROCm).

Every entry point only enqueues kernels on the caller's stream and allocates
nothing, so it can be captured.  The graph is replayed several times with the
program's own eager work and synchronisations between replays, and every
replay is compared with the eager result: bit-identical (same kernels, same
inputs).
"""
import pytest
import torch

from workloads import custom_workload

from _parity import device_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def A():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_forward_mode_attn_amd as A

    A.load_library()
    return A


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp32", 64)])
def test_fwd_replays_in_a_graph(A, dtype, d):
    w = custom_workload(2, 3, 300, 257, d, dtype, seed_id=7000 + d)
    print(f"case graph fwd {dtype} d{d}", flush=True)
    x = device_inputs(w)
    args = (x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"])
    ref = [t.clone() for t in A.fwd(*args, scale=w.scale)]
    out = (torch.empty_like(x["q"]), torch.empty_like(x["q"]),
           torch.empty((w.B, w.H, w.Lq), dtype=torch.float32, device=x["q"].device))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # warm-up on the capture stream
        A.fwd(*args, scale=w.scale, out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        A.fwd(*args, scale=w.scale, out=out)
    for i in range(4):
        for t in out:
            t.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip(out, ref):
            assert torch.equal(got, want), i


def test_split_and_merge_replay_in_a_graph(A):
    w = custom_workload(1, 2, 200, 700, 128, "bf16", seed_id=7100)
    print("case graph split + merge", flush=True)
    x = device_inputs(w)
    args = (x["q"], x["k"], x["v"], x["tq"], x["tk"], x["tv"])
    bounds = A.shard_bounds(w.Lk, 3)
    ref = [t.clone() for t in A.merge([A.fwd_part(*args, a, b, scale=w.scale) for a, b in bounds])]
    parts = [tuple(torch.empty_like(t) for t in ref) for _ in bounds]
    out = tuple(torch.empty_like(t) for t in ref)

    def body():
        for (a, b), part in zip(bounds, parts):
            A.fwd_part(*args, a, b, scale=w.scale, out=part)
        A.merge(parts, out=out)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        body()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    for i in range(3):
        for t in out:
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip(out, ref):
            assert torch.equal(got, want), i


def test_projection_then_attention_replays_in_a_graph(A):
    """The projection with its tangent followed by the attention JVP on its
    outputs: one captured layer pass, replayed against the eager result."""
    from workloads import custom_proj
    from workloads.device import device_proj_inputs

    w = custom_proj(1, 190, 256, 3, 2, 128, seed_id=7200)
    print("case graph projection + attention", flush=True)
    x = device_proj_inputs(w)
    y, ty = A.proj(x["x"], x["tx"], x["w"], x["bias"], n_out=3, heads=2)
    ref = [y.clone(), ty.clone()] + [t.clone() for t in A.fwd(y[0], y[1], y[2], ty[0], ty[1], ty[2])]
    ys = (torch.empty_like(y), torch.empty_like(ty))
    att = tuple(torch.empty_like(t) for t in ref[2:])

    def body():
        A.proj(x["x"], x["tx"], x["w"], x["bias"], n_out=3, heads=2, out=ys)
        A.fwd(ys[0][0], ys[0][1], ys[0][2], ys[1][0], ys[1][1], ys[1][2], out=att)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        body()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    for i in range(4):
        for t in ys + att:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip(ys + att, ref):
            assert torch.equal(got, want), i


def test_layer_chain_with_norm_and_rotary_replays_in_a_graph(A):
    """Projection with its tangent, then the RMS normalisation and rotary
    embedding of Q and K in place, then the attention JVP: the whole chain in
    one captured graph, every replay bit for bit the eager result."""
    from workloads import custom_proj
    from workloads.device import device_proj_inputs

    B, L, D, H, d = 1, 150, 256, 2, 64
    w = custom_proj(B, L, D, 3, H, d, seed_id=7300)
    print("case graph projection + norm/rotary + attention", flush=True)
    x = device_proj_inputs(w)
    g_q = (1.0 + 0.1 * torch.randn(d, generator=torch.Generator().manual_seed(7301))).to(torch.bfloat16).cuda()
    g_k = (1.0 + 0.1 * torch.randn(d, generator=torch.Generator().manual_seed(7302))).to(torch.bfloat16).cuda()
    pos = torch.arange(L, dtype=torch.float64)[:, None]
    ang = pos * 10000.0 ** (-torch.arange(0, d, 2, dtype=torch.float64) / d)
    cos, sin = ang.cos().float().contiguous().cuda(), ang.sin().float().contiguous().cuda()

    def chain(ys, att):
        A.proj(x["x"], x["tx"], x["w"], x["bias"], n_out=3, heads=H, out=ys)
        A.rmsnorm_rope(ys[0][0], ys[1][0], g_q, cos, sin, inplace=True)
        A.rmsnorm_rope(ys[0][1], ys[1][1], g_k, cos, sin, inplace=True)
        A.fwd(ys[0][0], ys[0][1], ys[0][2], ys[1][0], ys[1][1], ys[1][2], out=att)

    shape = (3, B, H, L, d)
    ref_ys = (torch.empty(shape, dtype=torch.bfloat16, device="cuda"), torch.empty(shape, dtype=torch.bfloat16, device="cuda"))
    ref_att = (torch.empty((B, H, L, d), dtype=torch.bfloat16, device="cuda"),
               torch.empty((B, H, L, d), dtype=torch.bfloat16, device="cuda"),
               torch.empty((B, H, L), dtype=torch.float32, device="cuda"))
    chain(ref_ys, ref_att)
    torch.cuda.synchronize()
    ref = list(ref_ys) + list(ref_att)
    ys = tuple(torch.empty_like(t) for t in ref_ys)
    att = tuple(torch.empty_like(t) for t in ref_att)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        chain(ys, att)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chain(ys, att)
    for i in range(4):
        for t in ys + att:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for got, want in zip(ys + att, ref):
            assert torch.equal(got, want), i
