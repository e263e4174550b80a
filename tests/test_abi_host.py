"""Host-side tests of the C ABI: symbols, status strings and argument checks.

None of these launches a kernel: every call here fails a host check (or is a
zero-size no-op) before any HIP call, as the header promises.
"""
import ctypes
import os
import re

import pytest

import attention_forward_mode_attn_amd as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn_jvp.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(A.library_path()):
        pytest.fail("libattnjvp.so not built: run __graft_entry__.build()")
    return A.load_library()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(attn_jvp_\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert names == ["attn_jvp_fwd", "attn_jvp_fwd_part", "attn_jvp_last_error", "attn_jvp_merge",
                     "attn_jvp_proj", "attn_jvp_rmsnorm_rope", "attn_jvp_status_string", "attn_jvp_version"]
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert A.attn_jvp_version() == 10400
    assert A.attn_jvp_status_string(0) == "ok"
    assert A.attn_jvp_status_string(A.ATTN_JVP_EUNSUPPORTED).startswith("unsupported")
    assert A.attn_jvp_status_string(99) == "unknown status"


FAKE = 0x10000  # 16-byte aligned; never dereferenced because every call below fails first


def call(B=1, H=1, Lq=8, Lk=8, d=64, scale=0.125, dtype=0, ptrs=None, lse=None):
    p = ptrs if ptrs is not None else [FAKE] * 8
    return A.attn_jvp_fwd(*p[:6], p[6], p[7], FAKE if lse is None else lse, B, H, Lq, Lk, d, scale, dtype)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=3), A.ATTN_JVP_EINVAL),
    (dict(dtype=-1), A.ATTN_JVP_EINVAL),
    (dict(B=-1), A.ATTN_JVP_EINVAL),
    (dict(Lk=-3), A.ATTN_JVP_EINVAL),
    (dict(d=96), A.ATTN_JVP_EUNSUPPORTED),
    (dict(d=256), A.ATTN_JVP_EUNSUPPORTED),
    (dict(Lk=0), A.ATTN_JVP_EINVAL),
    (dict(scale=float("nan")), A.ATTN_JVP_EINVAL),
    (dict(scale=float("inf")), A.ATTN_JVP_EINVAL),
    (dict(scale=0.0), A.ATTN_JVP_EINVAL),
    (dict(scale=-0.1), A.ATTN_JVP_EINVAL),
    (dict(ptrs=[FAKE] * 5 + [0] + [FAKE] * 2), A.ATTN_JVP_EINVAL),
    (dict(ptrs=[FAKE] * 7 + [0]), A.ATTN_JVP_EINVAL),
    (dict(lse=0), A.ATTN_JVP_EINVAL),
    (dict(ptrs=[FAKE + 8] + [FAKE] * 7), A.ATTN_JVP_EALIGN),
    (dict(ptrs=[FAKE] * 7 + [FAKE + 4]), A.ATTN_JVP_EALIGN),
    (dict(lse=FAKE + 2), A.ATTN_JVP_EALIGN),
    (dict(Lq=1 << 23, d=128), A.ATTN_JVP_EUNSUPPORTED),
    (dict(Lk=1 << 23, d=64), A.ATTN_JVP_EUNSUPPORTED),
    (dict(B=1 << 20, H=1 << 12, Lq=256), A.ATTN_JVP_EUNSUPPORTED),
])
def test_invalid_arguments_are_rejected_on_host(lib, kw, status):
    assert call(**kw) == status
    assert A.attn_jvp_last_error() != ""


def test_zero_size_is_ok_without_pointers(lib):
    nul = [0] * 8
    assert call(B=0, ptrs=nul, lse=0) == A.ATTN_JVP_OK
    assert call(H=0, ptrs=nul, lse=0) == A.ATTN_JVP_OK
    assert call(Lq=0, Lk=0, ptrs=nul, lse=0) == A.ATTN_JVP_OK
    assert A.attn_jvp_last_error() == ""


def test_dimension_check_precedes_zero_size(lib):
    # an unsupported head dim is reported even when there is no work
    assert call(B=0, d=80, ptrs=[0] * 8, lse=0) == A.ATTN_JVP_EUNSUPPORTED


def test_fwd_rejects_bad_tensors_before_launch(lib):
    import torch

    q = torch.zeros(1, 1, 4, 64)
    with pytest.raises(ValueError):
        A.fwd(q, q, q, q, q, q.transpose(2, 3))
    with pytest.raises(TypeError):
        A.fwd(*(torch.zeros(1, 1, 4, 64, dtype=torch.float16),) * 6)


def test_null_key_tangents_must_come_in_pairs(lib):
    assert call(ptrs=[FAKE] * 4 + [0] + [FAKE] * 3) == A.ATTN_JVP_EINVAL
    assert "both be NULL" in A.attn_jvp_last_error()
    assert call(ptrs=[FAKE] * 5 + [0] + [FAKE] * 2) == A.ATTN_JVP_EINVAL


def test_frozen_context_passes_host_checks(lib):
    """tk = tv = NULL is a valid call: with no GPU it reaches the launch."""
    import torch

    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: this checks the no-device path only")
    assert call(ptrs=[FAKE] * 4 + [0, 0] + [FAKE] * 2) == A.ATTN_JVP_ELAUNCH


def test_no_device_returns_launch_error(lib):
    """With no GPU present a well-formed call reports ELAUNCH instead of aborting."""
    import torch

    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: this checks the no-device path only")
    assert call() == A.ATTN_JVP_ELAUNCH
    assert "HIP error" in A.attn_jvp_last_error()


def test_ctypes_signature_is_c_abi(lib):
    assert lib.attn_jvp_fwd.restype is ctypes.c_int
    assert len(lib.attn_jvp_fwd.argtypes) == 17
    assert len(lib.attn_jvp_fwd_part.argtypes) == 19
    assert len(lib.attn_jvp_merge.argtypes) == 13
    assert len(lib.attn_jvp_proj.argtypes) == 14
    assert len(lib.attn_jvp_rmsnorm_rope.argtypes) == 14


def test_merge_part_limit_matches_header():
    src = open(HEADER).read()
    assert re.search(r"#define ATTN_JVP_MAX_MERGE_PARTS (\d+)", src).group(1) == str(A.ATTN_JVP_MAX_MERGE_PARTS)


def call_part(Lk=8, kv_rows=8, tlse=None, **kw):
    p = [FAKE] * 9
    return A.attn_jvp_fwd_part(*p, FAKE if tlse is None else tlse, kw.get("B", 1), 1, 8, Lk, kv_rows,
                               kw.get("d", 64), 0.125, 0)


@pytest.mark.parametrize("kw,status", [
    (dict(Lk=8, kv_rows=7), A.ATTN_JVP_EINVAL),
    (dict(Lk=8, kv_rows=1 << 31), A.ATTN_JVP_EUNSUPPORTED),
    (dict(tlse=FAKE + 1), A.ATTN_JVP_EALIGN),
    (dict(d=32), A.ATTN_JVP_EUNSUPPORTED),
])
def test_fwd_part_rejects_invalid_arguments(lib, kw, status):
    assert call_part(**kw) == status
    assert A.attn_jvp_last_error() != ""


def call_merge(n=2, parts=None, out=None, rows=16, d=64, dtype=1):
    parts = parts if parts is not None else [[FAKE] * n for _ in range(4)]
    out = out if out is not None else [FAKE] * 4
    return A.attn_jvp_merge(n, *parts, *out, rows, d, dtype)


@pytest.mark.parametrize("kw,status", [
    (dict(n=0), A.ATTN_JVP_EINVAL),
    (dict(n=17), A.ATTN_JVP_EINVAL),
    (dict(dtype=3), A.ATTN_JVP_EINVAL),
    (dict(rows=-1), A.ATTN_JVP_EINVAL),
    (dict(d=100), A.ATTN_JVP_EUNSUPPORTED),
    (dict(parts=[[FAKE, FAKE], [FAKE, 0], [FAKE, FAKE], [FAKE, FAKE]]), A.ATTN_JVP_EINVAL),
    (dict(parts=[[FAKE, FAKE], [FAKE, FAKE], [FAKE, FAKE], None]), A.ATTN_JVP_EINVAL),
    (dict(out=[FAKE, FAKE, 0, FAKE]), A.ATTN_JVP_EINVAL),
    (dict(parts=[[FAKE, FAKE + 8], [FAKE, FAKE], [FAKE, FAKE], [FAKE, FAKE]]), A.ATTN_JVP_EALIGN),
    (dict(parts=[[FAKE, FAKE], [FAKE, FAKE], [FAKE, FAKE], [FAKE + 2, FAKE]]), A.ATTN_JVP_EALIGN),
    (dict(out=[FAKE, FAKE, FAKE, FAKE + 2]), A.ATTN_JVP_EALIGN),
    (dict(rows=1 << 40), A.ATTN_JVP_EUNSUPPORTED),
])
def test_merge_rejects_invalid_arguments(lib, kw, status):
    assert call_merge(**kw) == status
    assert A.attn_jvp_last_error() != ""


def test_merge_zero_rows_is_ok_without_pointers(lib):
    assert call_merge(rows=0, parts=[[0, 0]] * 4, out=[0] * 4) == A.ATTN_JVP_OK


def test_new_entry_points_report_launch_error_without_device(lib):
    import torch

    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: this checks the no-device path only")
    assert call_part() == A.ATTN_JVP_ELAUNCH
    assert call_merge() == A.ATTN_JVP_ELAUNCH


def call_proj(ptrs=None, B=1, L=8, D=64, n_out=3, H=2, d=64, dtype=1):
    p = ptrs if ptrs is not None else [FAKE] * 6
    return A.attn_jvp_proj(*p, B, L, D, n_out, H, d, dtype)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=3), A.ATTN_JVP_EINVAL),
    (dict(dtype=2), A.ATTN_JVP_EUNSUPPORTED),
    (dict(dtype=0), A.ATTN_JVP_EUNSUPPORTED),
    (dict(L=-1), A.ATTN_JVP_EINVAL),
    (dict(D=-64), A.ATTN_JVP_EINVAL),
    (dict(d=32), A.ATTN_JVP_EUNSUPPORTED),
    (dict(D=96), A.ATTN_JVP_EUNSUPPORTED),
    (dict(D=0), A.ATTN_JVP_EUNSUPPORTED),
    (dict(ptrs=[0] + [FAKE] * 5), A.ATTN_JVP_EINVAL),
    (dict(ptrs=[FAKE] * 4 + [0, FAKE]), A.ATTN_JVP_EINVAL),
    (dict(ptrs=[FAKE, 0] + [FAKE] * 4), A.ATTN_JVP_EINVAL),
    (dict(ptrs=[FAKE] * 5 + [0]), A.ATTN_JVP_EINVAL),
    (dict(ptrs=[FAKE, FAKE + 8] + [FAKE] * 4), A.ATTN_JVP_EALIGN),
    (dict(ptrs=[FAKE] * 3 + [FAKE + 2] + [FAKE] * 2), A.ATTN_JVP_EALIGN),
    (dict(L=1 << 20, D=1 << 12), A.ATTN_JVP_EUNSUPPORTED),
    (dict(D=1 << 22, L=1), A.ATTN_JVP_EUNSUPPORTED),
])
def test_proj_rejects_invalid_arguments(lib, kw, status):
    assert call_proj(**kw) == status
    assert A.attn_jvp_last_error() != ""


def test_proj_zero_size_is_ok_without_pointers(lib):
    for kw in (dict(B=0), dict(L=0), dict(n_out=0), dict(H=0)):
        assert call_proj(ptrs=[0] * 6, **kw) == A.ATTN_JVP_OK


def test_proj_without_tangent_or_bias_passes_host_checks(lib):
    import torch

    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: this checks the no-device path only")
    assert call_proj(ptrs=[FAKE, 0, FAKE, 0, FAKE, 0]) == A.ATTN_JVP_ELAUNCH
    assert call_proj() == A.ATTN_JVP_ELAUNCH


def test_sizes_one_past_the_stated_limits_are_rejected(lib):
    n = (1 << 29) // 128  # Lq*d or Lk*d = 2^29
    assert A.attn_jvp_fwd(*([FAKE] * 9), 1, 1, n, 8, 128, 0.1, 1) == A.ATTN_JVP_EUNSUPPORTED
    assert A.attn_jvp_fwd(*([FAKE] * 9), 1, 1, 8, n, 128, 0.1, 1) == A.ATTN_JVP_EUNSUPPORTED
    assert A.attn_jvp_proj(*([FAKE] * 6), 1, 1 << 18, 8192, 1, 2, 128, 1) == A.ATTN_JVP_EUNSUPPORTED  # L*D = 2^31


def test_absurd_sizes_are_rejected_without_overflow(lib):
    """Sizes whose products overflow 64 bits are rejected as unsupported (every
    factor is bounded before it is multiplied)."""
    big = (1 << 62) + 3
    assert A.attn_jvp_fwd(*([FAKE] * 9), 1, 1, big, 8, 128, 0.1, 1) == A.ATTN_JVP_EUNSUPPORTED
    assert A.attn_jvp_fwd(*([FAKE] * 9), 1, 1, 8, big, 64, 0.1, 0) == A.ATTN_JVP_EUNSUPPORTED
    assert A.attn_jvp_fwd(*([FAKE] * 9), big, big, 8, 8, 128, 0.1, 1) == A.ATTN_JVP_EUNSUPPORTED
    for kw in (dict(n_out=1 << 40, H=1 << 40), dict(L=big), dict(B=big), dict(D=big - 3),
               dict(n_out=(1 << 31) - 1, H=(1 << 31) - 1)):
        assert call_proj(**kw) == A.ATTN_JVP_EUNSUPPORTED, kw


def test_binding_rejects_host_tensors():
    """The torch wrappers refuse CPU tensors before any library call (their
    addresses would be host memory)."""
    import torch

    q = torch.zeros(1, 1, 8, 64)
    with pytest.raises(ValueError, match="GPU"):
        A.fwd(q, q, q, q, q, q)
    with pytest.raises(ValueError, match="GPU"):
        A.fwd_part(q, q, q, q, q, q, 0, 4)
    lse = torch.zeros(1, 1, 8)
    with pytest.raises(ValueError, match="GPU"):
        A.merge([(q, q, lse, lse)])
    x = torch.zeros(1, 8, 64, dtype=torch.bfloat16)
    w = torch.zeros(3 * 64, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        A.proj(x, x, w, n_out=3, heads=1)


def test_grids_of_2_24_workgroups_are_rejected_on_host(lib):
    """Every kernel launches a 1-D grid of 256-thread workgroups, and a launch
    keeps gridDim.x * 256 below 2^32: exactly 2^24 workgroups must fail the host
    check (EUNSUPPORTED, nothing launched), not the launch."""
    # attention: B*H*ceil(Lq/128) = 2^24
    assert call(B=1, H=1 << 24, Lq=1, Lk=1, d=64) == A.ATTN_JVP_EUNSUPPORTED
    assert "2^24" in A.attn_jvp_last_error()
    assert call(B=1 << 12, H=1 << 5, Lq=128 * (1 << 7), Lk=8, d=64) == A.ATTN_JVP_EUNSUPPORTED
    assert call_part(B=1 << 24) == A.ATTN_JVP_EUNSUPPORTED
    # merge: ceil(rows / (256 / (d / 8))) = 2^24 (16 rows per workgroup at d = 128)
    assert call_merge(rows=(1 << 24) * 16, d=128) == A.ATTN_JVP_EUNSUPPORTED
    assert call_merge(rows=(1 << 24) * 32, d=64) == A.ATTN_JVP_EUNSUPPORTED
    # projection: B*ceil(L/128)*ceil(n_out*H*d/256) = 2^24
    assert call_proj(B=1 << 24, L=1, n_out=1, H=2, d=128) == A.ATTN_JVP_EUNSUPPORTED
    assert call_proj(B=1 << 14, L=128 * 1024, D=64, n_out=1, H=2, d=128) == A.ATTN_JVP_EUNSUPPORTED


def test_grids_just_below_2_24_workgroups_pass_host_checks(lib):
    """2^24 - 1 workgroups is the largest grid: the call passes every host
    check and, with no GPU present, reaches the launch (ELAUNCH)."""
    import torch

    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: this checks the no-device path only")
    assert call(B=1, H=(1 << 24) - 1, Lq=1, Lk=1, d=64) == A.ATTN_JVP_ELAUNCH
    assert call_merge(rows=((1 << 24) - 1) * 16, d=128) == A.ATTN_JVP_ELAUNCH
    assert call_proj(B=(1 << 24) - 1, L=1, n_out=1, H=2, d=128) == A.ATTN_JVP_ELAUNCH


def call_nr(ptrs=None, B=1, H=2, L=8, d=64, eps=1e-6, dtype=1):
    p = ptrs if ptrs is not None else [FAKE] * 7
    return A.attn_jvp_rmsnorm_rope(*p, B, H, L, d, eps, dtype)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=3), A.ATTN_JVP_EINVAL),
    (dict(dtype=2), A.ATTN_JVP_EUNSUPPORTED),
    (dict(L=-1), A.ATTN_JVP_EINVAL),
    (dict(d=96), A.ATTN_JVP_EUNSUPPORTED),
    (dict(eps=-1e-6), A.ATTN_JVP_EINVAL),
    (dict(eps=float("nan")), A.ATTN_JVP_EINVAL),
    (dict(eps=float("inf")), A.ATTN_JVP_EINVAL),
    (dict(ptrs=[0] + [FAKE] * 6), A.ATTN_JVP_EINVAL),
    (dict(ptrs=[FAKE] * 2 + [0] + [FAKE] * 4), A.ATTN_JVP_EINVAL),
    (dict(ptrs=[FAKE, 0] + [FAKE] * 5), A.ATTN_JVP_EINVAL),
    (dict(ptrs=[FAKE] * 5 + [0, FAKE]), A.ATTN_JVP_EINVAL),
    (dict(ptrs=[FAKE + 8] + [FAKE] * 6), A.ATTN_JVP_EALIGN),
    (dict(ptrs=[FAKE] * 4 + [FAKE + 2] + [FAKE] * 2), A.ATTN_JVP_EALIGN),
    (dict(ptrs=[FAKE] * 6 + [FAKE + 4]), A.ATTN_JVP_EALIGN),
    (dict(B=1 << 12, H=1 << 12), A.ATTN_JVP_EUNSUPPORTED),
    (dict(H=1 << 20, L=1 << 10), A.ATTN_JVP_EUNSUPPORTED),
    (dict(L=1 << 31), A.ATTN_JVP_EUNSUPPORTED),
])
def test_rmsnorm_rope_rejects_invalid_arguments(lib, kw, status):
    """(dtype 2, float32 outputs from bf16 inputs, is for the attention outputs only.)"""
    assert call_nr(**kw) == status
    assert A.attn_jvp_last_error() != ""


def test_rmsnorm_rope_zero_size_and_optional_inputs(lib):
    import torch

    for kw in (dict(B=0), dict(H=0), dict(L=0)):
        assert call_nr(ptrs=[0] * 7, **kw) == A.ATTN_JVP_OK
    if torch.cuda.device_count() > 0:
        return
    # no tangent, no gain, no tables: every optional input may be NULL together
    assert call_nr(ptrs=[FAKE, 0, FAKE, 0, 0, 0, 0]) == A.ATTN_JVP_ELAUNCH
    assert call_nr(ptrs=[FAKE] * 7, dtype=0, d=128) == A.ATTN_JVP_ELAUNCH


def test_float32_outputs_from_bf16_pass_host_checks(lib):
    """dtype 2 (bf16 inputs, float32 O and tO; float32 partials merged into a
    bf16 result) is accepted by fwd, fwd_part and merge."""
    import torch

    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: this checks the no-device path only")
    assert call(dtype=2) == A.ATTN_JVP_ELAUNCH
    assert A.attn_jvp_fwd_part(*([FAKE] * 10), 1, 1, 8, 8, 8, 64, 0.125, 2) == A.ATTN_JVP_ELAUNCH
    assert call_merge(dtype=2) == A.ATTN_JVP_ELAUNCH
