"""Python binding of libattnjvp.so: fused attention forward + JVP on MI355X.

The functions below carry the C ABI's names and only marshal arguments; every
step of the computation runs in the HIP kernels of the library.  ``fwd`` is a
convenience wrapper that allocates the outputs with torch and raises on error;
``fwd_part``, ``merge`` and ``fwd_split`` do the same for the key-sharded
partial passes and their exact merge, ``proj`` for the projection of
hidden states into attention heads with its tangent, and ``rmsnorm_rope`` for
the RMS normalisation and rotary embedding of queries or keys with theirs.
There is no fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "ATTN_JVP_FP32", "ATTN_JVP_BF16", "ATTN_JVP_BF16_F32OUT", "ATTN_JVP_OK", "ATTN_JVP_EINVAL", "ATTN_JVP_EUNSUPPORTED",
    "ATTN_JVP_EALIGN", "ATTN_JVP_ELAUNCH", "ATTN_JVP_MAX_MERGE_PARTS", "AttnJvpError", "attn_jvp_fwd",
    "attn_jvp_fwd_part", "attn_jvp_merge", "attn_jvp_status_string", "attn_jvp_last_error",
    "attn_jvp_version", "attn_jvp_proj", "attn_jvp_rmsnorm_rope", "fwd", "fwd_part", "merge", "fwd_split",
    "shard_bounds", "proj", "rmsnorm_rope", "library_path", "load_library",
]

ATTN_JVP_FP32, ATTN_JVP_BF16, ATTN_JVP_BF16_F32OUT = 0, 1, 2
ATTN_JVP_OK, ATTN_JVP_EINVAL, ATTN_JVP_EUNSUPPORTED, ATTN_JVP_EALIGN, ATTN_JVP_ELAUNCH = 0, 1, 2, 3, 4
ATTN_JVP_MAX_MERGE_PARTS = 16

_LIB = None


class AttnJvpError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"attn_jvp call failed: {attn_jvp_status_string(status)} ({status}): {detail}")
        self.status = status


def library_path() -> str:
    return os.environ.get("ATTNJVP_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattnjvp.so")


def load_library() -> ctypes.CDLL:
    """Load libattnjvp.so (after torch, so both share torch's HIP runtime)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    import torch  # noqa: F401  -- loads libamdhip64.so.7 first; the library then binds to it

    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built: run `python -m attention_forward_mode_attn_amd.build` "
            "(or __graft_entry__.build())"
        )
    lib = ctypes.CDLL(path)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.attn_jvp_fwd.argtypes = [vp] * 9 + [i64] * 5 + [ctypes.c_float, ctypes.c_int, vp]
    lib.attn_jvp_fwd.restype = ctypes.c_int
    lib.attn_jvp_fwd_part.argtypes = [vp] * 10 + [i64] * 6 + [ctypes.c_float, ctypes.c_int, vp]
    lib.attn_jvp_fwd_part.restype = ctypes.c_int
    lib.attn_jvp_merge.argtypes = [ctypes.c_int] + [ctypes.POINTER(vp)] * 4 + [vp] * 4 + [i64] * 2 + [ctypes.c_int, vp]
    lib.attn_jvp_merge.restype = ctypes.c_int
    lib.attn_jvp_proj.argtypes = [vp] * 6 + [i64] * 6 + [ctypes.c_int, vp]
    lib.attn_jvp_proj.restype = ctypes.c_int
    lib.attn_jvp_rmsnorm_rope.argtypes = [vp] * 7 + [i64] * 4 + [ctypes.c_float, ctypes.c_int, vp]
    lib.attn_jvp_rmsnorm_rope.restype = ctypes.c_int
    lib.attn_jvp_status_string.argtypes = [ctypes.c_int]
    lib.attn_jvp_status_string.restype = ctypes.c_char_p
    lib.attn_jvp_last_error.argtypes = []
    lib.attn_jvp_last_error.restype = ctypes.c_char_p
    lib.attn_jvp_version.argtypes = []
    lib.attn_jvp_version.restype = ctypes.c_int
    _LIB = lib
    return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def attn_jvp_fwd(q, k, v, tq, tk, tv, o, to, lse, B, H, Lq, Lk, d, scale, dtype, stream=None) -> int:
    """Marshal to the C entry point.  Tensors (anything with data_ptr()) or raw
    device addresses as ints; ``stream`` is a hipStream_t as int (None = null
    stream).  Returns the status code."""
    lib = load_library()
    return int(lib.attn_jvp_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(tq), _ptr(tk), _ptr(tv), _ptr(o), _ptr(to), _ptr(lse),
        int(B), int(H), int(Lq), int(Lk), int(d), float(scale), int(dtype), stream,
    ))


def attn_jvp_fwd_part(q, k, v, tq, tk, tv, o, to, lse, tlse, B, H, Lq, Lk, kv_rows, d, scale, dtype,
                      stream=None) -> int:
    """Marshal to the C entry point (arguments as ``attn_jvp_fwd``; ``tlse``
    may be None).  Returns the status code."""
    lib = load_library()
    return int(lib.attn_jvp_fwd_part(
        _ptr(q), _ptr(k), _ptr(v), _ptr(tq), _ptr(tk), _ptr(tv), _ptr(o), _ptr(to), _ptr(lse), _ptr(tlse),
        int(B), int(H), int(Lq), int(Lk), int(kv_rows), int(d), float(scale), int(dtype), stream,
    ))


def attn_jvp_merge(n, o_parts, to_parts, lse_parts, tlse_parts, o, to, lse, tlse, rows, d, dtype,
                   stream=None) -> int:
    """Marshal to the C entry point; the four part lists hold n tensors or
    device addresses each (None entries become NULL).  Returns the status code."""
    lib = load_library()

    def arr(xs):
        if xs is None:
            return None
        return (ctypes.c_void_p * max(len(xs), 1))(*[_ptr(x) for x in xs])

    return int(lib.attn_jvp_merge(
        int(n), arr(o_parts), arr(to_parts), arr(lse_parts), arr(tlse_parts),
        _ptr(o), _ptr(to), _ptr(lse), _ptr(tlse), int(rows), int(d), int(dtype), stream,
    ))


def attn_jvp_proj(x, tx, w, bias, y, ty, B, L, D, n_out, H, d, dtype, stream=None) -> int:
    """Marshal to the C entry point (tx, bias, ty may be None).  Returns the
    status code."""
    lib = load_library()
    return int(lib.attn_jvp_proj(
        _ptr(x), _ptr(tx), _ptr(w), _ptr(bias), _ptr(y), _ptr(ty),
        int(B), int(L), int(D), int(n_out), int(H), int(d), int(dtype), stream,
    ))


def attn_jvp_rmsnorm_rope(x, tx, y, ty, gamma, rope_cos, rope_sin, B, H, L, d, eps, dtype, stream=None) -> int:
    """Marshal to the C entry point (tx, ty, gamma, rope_cos, rope_sin may be
    None).  Returns the status code."""
    lib = load_library()
    return int(lib.attn_jvp_rmsnorm_rope(
        _ptr(x), _ptr(tx), _ptr(y), _ptr(ty), _ptr(gamma), _ptr(rope_cos), _ptr(rope_sin),
        int(B), int(H), int(L), int(d), float(eps), int(dtype), stream,
    ))


def attn_jvp_status_string(status: int) -> str:
    return load_library().attn_jvp_status_string(int(status)).decode()


def attn_jvp_last_error() -> str:
    return load_library().attn_jvp_last_error().decode()


def attn_jvp_version() -> int:
    return int(load_library().attn_jvp_version())


def _out_dtype(q, f32_out):
    """The C dtype code and torch dtype of O and tO: the inputs' own, or float32
    for bfloat16 inputs when ``f32_out`` (ATTN_JVP_BF16_F32OUT)."""
    import torch

    if not f32_out or q.dtype == torch.float32:
        return None, q.dtype
    return ATTN_JVP_BF16_F32OUT, torch.float32


def fwd(q, k, v, tq, tk, tv, scale=None, out=None, stream=None, f32_out=False):
    """O, tO, lse for torch tensors q, tq [B,H,Lq,d] and k, v, tk, tv [B,H,Lk,d]
    (contiguous, same device, all float32 or all bfloat16); tk = tv = None is
    a frozen context (zero key-side tangents, computed without them).  Outputs are
    allocated unless ``out=(o, to, lse)`` is given; with ``f32_out`` bfloat16
    inputs give float32 O and tO.  Runs on ``stream`` (a torch.cuda.Stream) or the
    current stream."""
    import torch

    dtype = _check_inputs(q, k, v, tq, tk, tv)
    code, odt = _out_dtype(q, f32_out)
    dtype = code if code is not None else dtype
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    if scale is None:
        scale = d ** -0.5
    if out is None:
        o = torch.empty(q.shape, dtype=odt, device=q.device)
        to = torch.empty(q.shape, dtype=odt, device=q.device)
        lse = torch.empty((B, H, Lq), dtype=torch.float32, device=q.device)
    else:
        o, to, lse = out
        _check_out(o, q.shape, odt, q.device, "o")
        _check_out(to, q.shape, odt, q.device, "to")
        _check_out(lse, (B, H, Lq), torch.float32, q.device, "lse")
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    with torch.cuda.device(q.device):  # launch on the inputs' device
        status = attn_jvp_fwd(q, k, v, tq, tk, tv, o, to, lse, B, H, Lq, Lk, d, scale, dtype, s.cuda_stream)
    if status != ATTN_JVP_OK:
        raise AttnJvpError(status, attn_jvp_last_error())
    return o, to, lse


def _check_out(x, shape, dtype, device, what):
    """An output buffer passed by the caller: exactly the shape, dtype and
    device the kernel writes, contiguous (the kernels write every element of
    that extent and nothing else)."""
    if x is None or tuple(x.shape) != tuple(shape) or x.dtype != dtype or x.device != device \
            or not x.is_contiguous():
        raise ValueError(f"{what}: expected a contiguous {dtype} tensor of shape {tuple(shape)} on {device}")


def _check_inputs(q, k, v, tq, tk, tv):
    import torch

    dt = q.dtype
    if dt not in (torch.float32, torch.bfloat16):
        raise TypeError("q must be float32 or bfloat16")
    if q.device.type != "cuda":
        raise ValueError("inputs must be GPU tensors")
    if (tk is None) != (tv is None):
        raise ValueError("tk and tv must both be None (frozen context) or both tensors")
    ins = [x for x in (q, k, v, tq, tk, tv) if x is not None]
    for x in ins:
        if x.dtype != dt or x.device != q.device or not x.is_contiguous() or x.dim() != 4:
            raise ValueError("all inputs: same dtype and device, contiguous, 4-D [B,H,L,d]")
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    if tq.shape != q.shape or any(x.shape != (B, H, Lk, d) for x in ins[1:] if x is not tq):
        raise ValueError("shape mismatch: q, tq [B,H,Lq,d]; k, v, tk, tv [B,H,Lk,d]")
    return ATTN_JVP_BF16 if dt == torch.bfloat16 else ATTN_JVP_FP32


def fwd_part(q, k, v, tq, tk, tv, k0, k1, scale=None, out=None, stream=None, f32_out=False):
    """O, tO, lse, tlse of the keys [k0, k1) of k, v, tk, tv (torch tensors as
    in ``fwd``): the partial result of one key shard.  The shard is addressed
    in place (no copy).  ``out=(o, to, lse, tlse)`` reuses buffers; with
    ``f32_out`` bfloat16 inputs give float32 partial O and tO, which ``merge``
    rounds to bfloat16 once."""
    import torch

    dtype = _check_inputs(q, k, v, tq, tk, tv)
    code, odt = _out_dtype(q, f32_out)
    dtype = code if code is not None else dtype
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    if not 0 <= k0 < k1 <= Lk:
        raise ValueError("need 0 <= k0 < k1 <= Lk")
    if scale is None:
        scale = d ** -0.5
    if out is None:
        o = torch.empty(q.shape, dtype=odt, device=q.device)
        to = torch.empty(q.shape, dtype=odt, device=q.device)
        lse = torch.empty((B, H, Lq), dtype=torch.float32, device=q.device)
        tlse = torch.empty((B, H, Lq), dtype=torch.float32, device=q.device)
    else:
        o, to, lse, tlse = out
        _check_out(o, q.shape, odt, q.device, "o")
        _check_out(to, q.shape, odt, q.device, "to")
        _check_out(lse, (B, H, Lq), torch.float32, q.device, "lse")
        _check_out(tlse, (B, H, Lq), torch.float32, q.device, "tlse")
    off = k0 * d * k.element_size()
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    tk_p = None if tk is None else tk.data_ptr() + off
    tv_p = None if tv is None else tv.data_ptr() + off
    with torch.cuda.device(q.device):
        status = attn_jvp_fwd_part(q, k.data_ptr() + off, v.data_ptr() + off, tq, tk_p, tv_p, o, to, lse, tlse,
                                   B, H, Lq, k1 - k0, Lk, d, scale, dtype, s.cuda_stream)
    if status != ATTN_JVP_OK:
        raise AttnJvpError(status, attn_jvp_last_error())
    return o, to, lse, tlse


def merge(parts, out=None, stream=None, out_dtype=None):
    """Exact merge of partial results ``parts`` = [(o, to, lse, tlse), ...]
    over disjoint key shards; returns (o, to, lse, tlse) of the union.  The
    result has the parts' dtype, or bfloat16 for float32 parts with
    ``out_dtype=torch.bfloat16``."""
    import torch

    if not 1 <= len(parts) <= ATTN_JVP_MAX_MERGE_PARTS:
        raise ValueError(f"1 .. {ATTN_JVP_MAX_MERGE_PARTS} parts")
    o0 = parts[0][0]
    if o0.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("o must be float32 or bfloat16")
    if o0.device.type != "cuda":
        raise ValueError("parts must be GPU tensors")
    dtype = ATTN_JVP_BF16 if o0.dtype == torch.bfloat16 else ATTN_JVP_FP32
    odt = o0.dtype if out_dtype is None else out_dtype
    if odt != o0.dtype:
        if not (o0.dtype == torch.float32 and odt == torch.bfloat16):
            raise ValueError("out_dtype: bfloat16 from float32 parts is the one conversion the merge makes")
        dtype = ATTN_JVP_BF16_F32OUT
    d = o0.shape[-1]
    rows = o0.numel() // d
    for o, to, lse, tlse in parts:
        if o.shape != o0.shape or to.shape != o0.shape or o.dtype != o0.dtype or to.dtype != o0.dtype:
            raise ValueError("all parts: o and to of one shape and dtype")
        if lse.numel() != rows or tlse.numel() != rows or lse.dtype != torch.float32 or tlse.dtype != torch.float32:
            raise ValueError("all parts: lse and tlse float32 with one value per row")
        if not all(x.is_contiguous() for x in (o, to, lse, tlse)):
            raise ValueError("all parts contiguous")
        if any(x.device != o0.device for x in (o, to, lse, tlse)):
            raise ValueError("all parts on one device")
    if out is None:
        o = torch.empty(o0.shape, dtype=odt, device=o0.device)
        to = torch.empty(o0.shape, dtype=odt, device=o0.device)
        lse, tlse = torch.empty_like(parts[0][2]), torch.empty_like(parts[0][3])
    else:
        o, to, lse, tlse = out
        _check_out(o, o0.shape, odt, o0.device, "o")
        _check_out(to, o0.shape, odt, o0.device, "to")
        _check_out(lse, parts[0][2].shape, torch.float32, o0.device, "lse")
        _check_out(tlse, parts[0][2].shape, torch.float32, o0.device, "tlse")
    s = stream if stream is not None else torch.cuda.current_stream(o0.device)
    with torch.cuda.device(o0.device):
        status = attn_jvp_merge(len(parts), [p[0] for p in parts], [p[1] for p in parts], [p[2] for p in parts],
                                [p[3] for p in parts], o, to, lse, tlse, rows, d, dtype, s.cuda_stream)
    if status != ATTN_JVP_OK:
        raise AttnJvpError(status, attn_jvp_last_error())
    return o, to, lse, tlse


def shard_bounds(Lk: int, n: int, align: int = 64):
    """Split [0, Lk) into n contiguous non-empty shards, boundaries on multiples
    of ``align`` where the length allows."""
    if not 1 <= n <= Lk:
        raise ValueError("need 1 <= n <= Lk")
    units = -(-Lk // align)
    if units >= n:
        cuts = [min(Lk, (i * units // n) * align) for i in range(n + 1)]
    else:
        cuts = [i * Lk // n for i in range(n + 1)]
    return [(cuts[i], cuts[i + 1]) for i in range(n)]


def fwd_split(q, k, v, tq, tk, tv, n_split, scale=None, stream=None, f32_partials=False):
    """The attention-JVP computed as ``n_split`` key shards and merged:
    returns (o, to, lse, tlse), equal to ``fwd`` (plus tlse) up to rounding.
    With ``f32_partials`` bfloat16 shards are kept in float32 and the result is
    rounded to bfloat16 once, by the merge."""
    parts = [fwd_part(q, k, v, tq, tk, tv, a, b, scale=scale, stream=stream, f32_out=f32_partials)
             for a, b in shard_bounds(k.shape[2], n_split)]
    return merge(parts, stream=stream, out_dtype=q.dtype)


def proj(x, tx, w, bias=None, n_out=3, heads=None, out=None, stream=None):
    """Y = x W^T + bias and TY = tx W^T for bfloat16 torch tensors x, tx
    [B, L, D] (tx None: no tangent), w [n_out*heads*d, D], bias [n_out*heads*d]
    or None; returns (y, ty), each [n_out, B, heads, L, d] (ty None without
    tangent), so that y[0], y[1], y[2] are the q, k, v of ``fwd`` for n_out = 3.
    ``out=(y, ty)`` reuses buffers."""
    import torch

    if heads is None:
        raise ValueError("heads is required")
    if x.dtype != torch.bfloat16:
        raise TypeError("the projection takes bfloat16 tensors")
    if x.device.type != "cuda":
        raise ValueError("inputs must be GPU tensors")
    ins = [t for t in (x, tx, w, bias) if t is not None]
    if any(t.dtype != x.dtype or t.device != x.device or not t.is_contiguous() for t in ins):
        raise ValueError("all inputs: bfloat16, one device, contiguous")
    if x.dim() != 3 or (tx is not None and tx.shape != x.shape):
        raise ValueError("x and tx must be [B, L, D]")
    B, L, D = x.shape
    F = w.shape[0]
    if w.dim() != 2 or w.shape[1] != D or F % (n_out * heads) != 0:
        raise ValueError("w must be [n_out*heads*d, D]")
    d = F // (n_out * heads)
    if bias is not None and bias.shape != (F,):
        raise ValueError("bias must be [n_out*heads*d]")
    shape = (n_out, B, heads, L, d)
    if out is None:
        y = torch.empty(shape, dtype=x.dtype, device=x.device)
        ty = torch.empty(shape, dtype=x.dtype, device=x.device) if tx is not None else None
    else:
        y, ty = out
        _check_out(y, shape, x.dtype, x.device, "y")
        if tx is None:
            if ty is not None:
                raise ValueError("ty must be None without a tangent")
        else:
            _check_out(ty, shape, x.dtype, x.device, "ty")
    s = stream if stream is not None else torch.cuda.current_stream(x.device)
    with torch.cuda.device(x.device):
        status = attn_jvp_proj(x, tx, w, bias, y, ty, B, L, D, n_out, heads, d, ATTN_JVP_BF16, s.cuda_stream)
    if status != ATTN_JVP_OK:
        raise AttnJvpError(status, attn_jvp_last_error())
    return y, ty


def rmsnorm_rope(x, tx=None, gamma=None, rope_cos=None, rope_sin=None, eps=1e-6, out=None, inplace=False,
                 stream=None):
    """RMS normalisation over the head dim with gain ``gamma`` [d] (None: 1),
    then rotation of adjacent pairs by the angles of each row's position
    (``rope_cos``, ``rope_sin`` float32 [L, d/2], both None: no rotation), for
    torch tensors x [B, H, L, d] (float32 or bfloat16) and its tangent tx (or
    None).  Returns (y, ty); ``inplace=True`` writes into x and tx,
    ``out=(y, ty)`` into given buffers."""
    import torch

    if x.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("x must be float32 or bfloat16")
    if x.device.type != "cuda":
        raise ValueError("inputs must be GPU tensors")
    if x.dim() != 4 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [B, H, L, d] tensor")
    B, H, L, d = x.shape
    if tx is not None and (tx.shape != x.shape or tx.dtype != x.dtype or tx.device != x.device
                           or not tx.is_contiguous()):
        raise ValueError("tx must match x")
    if gamma is not None and (gamma.shape != (d,) or gamma.dtype != x.dtype or gamma.device != x.device):
        raise ValueError("gamma must be [d] in x's dtype on x's device")
    if (rope_cos is None) != (rope_sin is None):
        raise ValueError("rope_cos and rope_sin must both be given or both be None")
    for tab in (rope_cos, rope_sin):
        if tab is not None and (tab.shape != (L, d // 2) or tab.dtype != torch.float32 or tab.device != x.device
                                or not tab.is_contiguous()):
            raise ValueError("rope tables must be contiguous float32 [L, d/2] on x's device")
    if inplace:
        if out is not None:
            raise ValueError("out and inplace are exclusive")
        y, ty = x, tx
    elif out is None:
        y = torch.empty_like(x)
        ty = torch.empty_like(x) if tx is not None else None
    else:
        y, ty = out
        _check_out(y, x.shape, x.dtype, x.device, "y")
        if tx is None:
            if ty is not None:
                raise ValueError("ty must be None without a tangent")
        else:
            _check_out(ty, x.shape, x.dtype, x.device, "ty")
    dtype = ATTN_JVP_BF16 if x.dtype == torch.bfloat16 else ATTN_JVP_FP32
    s = stream if stream is not None else torch.cuda.current_stream(x.device)
    with torch.cuda.device(x.device):
        status = attn_jvp_rmsnorm_rope(x, tx, y, ty, gamma, rope_cos, rope_sin, B, H, L, d, eps, dtype,
                                       s.cuda_stream)
    if status != ATTN_JVP_OK:
        raise AttnJvpError(status, attn_jvp_last_error())
    return y, ty
