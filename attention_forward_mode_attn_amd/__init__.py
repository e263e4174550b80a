"""Python binding of libattnjvp.so: fused attention forward + JVP on MI355X.

The functions below carry the C ABI's names and only marshal arguments; every
step of the computation runs in the HIP kernels of the library.  ``fwd`` is a
convenience wrapper that allocates the outputs with torch and raises on error.
There is no fallback: if the library is missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "ATTN_JVP_FP32", "ATTN_JVP_BF16", "ATTN_JVP_OK", "ATTN_JVP_EINVAL", "ATTN_JVP_EUNSUPPORTED",
    "ATTN_JVP_EALIGN", "ATTN_JVP_ELAUNCH", "AttnJvpError", "attn_jvp_fwd", "attn_jvp_status_string",
    "attn_jvp_last_error", "attn_jvp_version", "fwd", "library_path", "load_library",
]

ATTN_JVP_FP32, ATTN_JVP_BF16 = 0, 1
ATTN_JVP_OK, ATTN_JVP_EINVAL, ATTN_JVP_EUNSUPPORTED, ATTN_JVP_EALIGN, ATTN_JVP_ELAUNCH = 0, 1, 2, 3, 4

_LIB = None


class AttnJvpError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"attn_jvp_fwd failed: {attn_jvp_status_string(status)} ({status}): {detail}")
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


def attn_jvp_status_string(status: int) -> str:
    return load_library().attn_jvp_status_string(int(status)).decode()


def attn_jvp_last_error() -> str:
    return load_library().attn_jvp_last_error().decode()


def attn_jvp_version() -> int:
    return int(load_library().attn_jvp_version())


def fwd(q, k, v, tq, tk, tv, scale=None, out=None, stream=None):
    """O, tO, lse for torch tensors q, tq [B,H,Lq,d] and k, v, tk, tv [B,H,Lk,d]
    (contiguous, same device, all float32 or all bfloat16).  Outputs are
    allocated unless ``out=(o, to, lse)`` is given.  Runs on ``stream`` (a
    torch.cuda.Stream) or the current stream."""
    import torch

    ins = (q, k, v, tq, tk, tv)
    dt = q.dtype
    if dt not in (torch.float32, torch.bfloat16):
        raise TypeError("q must be float32 or bfloat16")
    for x in ins:
        if x.dtype != dt or x.device != q.device or not x.is_contiguous() or x.dim() != 4:
            raise ValueError("all inputs: same dtype and device, contiguous, 4-D [B,H,L,d]")
    B, H, Lq, d = q.shape
    Lk = k.shape[2]
    if tq.shape != q.shape or any(x.shape != (B, H, Lk, d) for x in (k, v, tk, tv)):
        raise ValueError("shape mismatch: q, tq [B,H,Lq,d]; k, v, tk, tv [B,H,Lk,d]")
    if scale is None:
        scale = d ** -0.5
    if out is None:
        o = torch.empty_like(q)
        to = torch.empty_like(q)
        lse = torch.empty((B, H, Lq), dtype=torch.float32, device=q.device)
    else:
        o, to, lse = out
    s = stream if stream is not None else torch.cuda.current_stream(q.device)
    status = attn_jvp_fwd(q, k, v, tq, tk, tv, o, to, lse, B, H, Lq, Lk, d, scale,
                          ATTN_JVP_BF16 if dt == torch.bfloat16 else ATTN_JVP_FP32, s.cuda_stream)
    if status != ATTN_JVP_OK:
        raise AttnJvpError(status, attn_jvp_last_error())
    return o, to, lse
