"""GPU: every ragged tail position, against the fp64 oracle.

Each kernel masks the keys past Lk of its last tile and drops the query rows
past Lq of its last block, and the two attention kernels index keys in
different orders (the fp32 kernel in 16-key blocks whose registers follow the
fp64 matrix instruction's row order, 32-key tiles; the bf16 kernels in 64-key
tiles, pipelined at d = 128 and one tile at a time at d = 64).  These sweeps run
every key count up to two tiles and a tail, and every query count up to 40,
each against the oracle on every row, with and without the key-side tangents.
"""
import pytest
import torch

from workloads import custom_workload

from _parity import LSE_TOL, TOL, compare, device_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def A():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_forward_mode_attn_amd as A

    A.load_library()
    return A


def run_case(A, B, H, Lq, Lk, d, dtype, frozen, seed):
    std = {"q": 1.0, "k": 1.0, "v": 1.0, "tq": 1.0, "tk": 0.0 if frozen else 1.0, "tv": 0.0 if frozen else 1.0}
    w = custom_workload(B, H, Lq, Lk, d, dtype, seed_id=seed, std=std)
    print(f"case tail B{B} H{H} Lq{Lq} Lk{Lk} d{d} {dtype} frozen={frozen}", flush=True)
    x = device_inputs(w)
    tk, tv = (None, None) if frozen else (x["tk"], x["tv"])
    o, to, lse = A.fwd(x["q"], x["k"], x["v"], x["tq"], tk, tv, scale=w.scale)
    torch.cuda.synchronize()
    res = compare(w, o, to, lse, threads=2)
    ok = res["O"] <= TOL[dtype] and res["tO"] <= TOL[dtype] and res["lse"] <= LSE_TOL[dtype]
    if not ok:
        print(f"  O {res['O']:.3e} tO {res['tO']:.3e} lse {res['lse']:.3e}", flush=True)
    return ok


@pytest.mark.parametrize("d", [64, 128])
def test_fp32_every_key_count(A, d):
    """Lk = 1 .. 70: every position in the 16-key blocks and 32-key tiles."""
    bad = [Lk for Lk in range(1, 71) if not run_case(A, 1, 1, 37, Lk, d, "fp32", Lk % 3 == 0, 8000 + Lk)]
    assert not bad, bad


@pytest.mark.parametrize("d", [64, 128])
def test_bf16_every_key_count(A, d):
    """Lk = 1 .. 140: every position in the first two 64-key tiles and a tail."""
    bad = [Lk for Lk in range(1, 141) if not run_case(A, 1, 1, 70, Lk, d, "bf16", Lk % 3 == 0, 8100 + Lk)]
    assert not bad, bad


@pytest.mark.parametrize("dtype,d", [("fp32", 64), ("fp32", 128), ("bf16", 64), ("bf16", 128)])
def test_every_query_count(A, dtype, d):
    """Lq = 1 .. 40 over two heads: every row position in the first 16-row and
    32-row blocks of a wave."""
    bad = [Lq for Lq in range(1, 41) if not run_case(A, 1, 2, Lq, 50, d, dtype, Lq % 4 == 0, 8200 + Lq)]
    assert not bad, bad
