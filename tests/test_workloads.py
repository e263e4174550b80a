"""Host-side checks of the seeded inputs and of the oracle regression fixture."""
import json
import os

import numpy as np

from oracle import attention_jvp_head
from workloads import (
    WORKLOADS,
    bf16_bits_to_f32,
    custom_workload,
    f32_to_bf16_bits,
    head_array,
    head_upload,
    sample_rows,
    tq_head_scale,
)


def test_bf16_rounding_is_nearest_even():
    # 1 + 2^-8 is halfway between bf16 neighbours 1 and 1 + 2^-7: ties go to even (1).
    x = np.array([1.0, 1 + 2**-8, 1 + 3 * 2**-8, -2.5, 3.0e38, 1e-40, 0.0], dtype=np.float32)
    r = bf16_bits_to_f32(f32_to_bf16_bits(x))
    assert r[0] == 1.0 and r[1] == 1.0 and r[2] == 1 + 2**-6 and r[3] == -2.5
    assert np.isfinite(r[4]) and r[6] == 0.0
    # agrees with torch's own float32 -> bfloat16 conversion (round to nearest even)
    import torch

    y = np.random.default_rng(0).normal(size=4096).astype(np.float32) * 37.0
    want = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(f32_to_bf16_bits(y), want)


def test_generation_is_deterministic_and_per_head():
    w = WORKLOADS["image_self_bf16"]
    a = head_array(w, "q", 1, 3)
    b = head_array(w, "q", 1, 3)
    c = head_array(w, "q", 1, 4)
    assert a.shape == (w.Lq, w.d) and a.dtype == np.float32
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    assert np.array_equal(bf16_bits_to_f32(head_upload(w, "q", 1, 3)), a)
    assert abs(float(head_array(w, "tq", 0, 0).std()) - 0.5) < 0.01


def test_frozen_context_tangents_are_zero():
    w = WORKLOADS["text_cross_bf16"]
    assert not head_array(w, "tk", 0, 0).any() and not head_array(w, "tv", 1, 15).any()
    assert head_array(w, "tq", 0, 0).any()


def test_stress_workload_scales():
    w = WORKLOADS["video_cross_stress_bf16"]
    s = np.array([tq_head_scale(w, h) for h in range(w.H)])
    assert s.min() >= 1e-2 and s.max() <= 1e2 and s.max() / s.min() > 100
    k = head_array(w, "k", 0, 0)
    assert abs(float(k.std()) - np.sqrt(8.0)) < 0.05


def test_sample_rows_cover_edges():
    w = WORKLOADS["video_self_bf16"]
    r = sample_rows(w, 0, 7)
    assert r.size == 256 and np.all(np.diff(r) > 0)
    assert {0, 7, 120, 135, w.Lq - 1, w.Lq - 8} <= set(r.tolist())
    small = custom_workload(1, 1, 5, 5, 64, "fp32")
    assert sample_rows(small, 0, 0).tolist() == [0, 1, 2, 3, 4]


def test_oracle_regression_fixture():
    here = os.path.dirname(__file__)
    with open(os.path.join(here, "golden", "oracle_tiny_self_fp32_rows.json")) as f:
        g = json.load(f)
    w = WORKLOADS[g["workload"]]
    for e in g["heads"]:
        a = {t: head_array(w, t, e["b"], e["h"]) for t in ("q", "k", "v", "tq", "tk", "tv")}
        O, tO, lse = attention_jvp_head(a["q"], a["k"], a["v"], a["tq"], a["tk"], a["tv"], w.scale, rows=g["rows"])
        assert np.allclose(O, e["O"], rtol=0, atol=1e-13)
        assert np.allclose(tO, e["tO"], rtol=0, atol=1e-13)
        assert np.allclose(lse, e["lse"], rtol=0, atol=1e-13)


def test_key_ramp_scales_key_rows_only():
    import numpy as np

    from workloads import custom_workload, head_array

    flat = custom_workload(1, 1, 8, 40, 64, "fp32", seed_id=77)
    ramp = custom_workload(1, 1, 8, 40, 64, "fp32", seed_id=77, key_ramp=0.25)
    k0, k1 = head_array(flat, "k", 0, 0), head_array(ramp, "k", 0, 0)
    assert np.array_equal(k1, k0 * (1 + 0.25 * np.arange(40, dtype=np.float32))[:, None])
    for t in ("q", "v", "tq", "tk", "tv"):
        assert np.array_equal(head_array(flat, t, 0, 0), head_array(ramp, t, 0, 0))


def test_projection_inputs_are_seeded_bf16_values():
    import numpy as np

    from workloads import PROJ_WORKLOADS, bf16_bits_to_f32, custom_proj, f32_to_bf16_bits, proj_array, proj_host_inputs

    w = custom_proj(2, 33, 256, 3, 2, 64, seed_id=91)
    a, b = proj_host_inputs(w), proj_host_inputs(w)
    for t in ("x", "tx", "w", "bias"):
        assert np.array_equal(a[t], b[t]) and a[t].shape == w.shape(t)
        assert np.array_equal(bf16_bits_to_f32(f32_to_bf16_bits(a[t])), a[t])  # exactly bf16 values
    assert not np.array_equal(a["x"][0], a["x"][1]) and not np.array_equal(a["x"], a["tx"])
    assert abs(a["w"].std() * np.sqrt(w.D) - 1.0) < 0.02 and abs(a["bias"].std() - 0.1) < 0.02
    assert np.array_equal(proj_array(w, "x", 1), a["x"][1])
    frozen = custom_proj(1, 4, 64, 2, 1, 64, tangent=False, bias=False)
    f = proj_host_inputs(frozen)
    assert f["tx"] is None and f["bias"] is None
    video = PROJ_WORKLOADS["qkv_video_bf16"]
    assert video.F == 15360 and video.D == video.H * video.d
    assert video.flops == 4.0 * 32760 * 5120 * 15360


def test_norm_rope_inputs_are_seeded_and_rounded():
    import numpy as np

    from workloads import NORM_ROPE_WORKLOADS, custom_norm_rope, norm_rope_array, norm_rope_upload, rope_tables
    from workloads.inputs import bf16_bits_to_f32

    w = NORM_ROPE_WORKLOADS["q_image_bf16"]
    a = norm_rope_array(w, "x", 1, 3)
    assert a.shape == (w.L, w.d) and np.array_equal(a, norm_rope_array(w, "x", 1, 3))
    assert not np.array_equal(a, norm_rope_array(w, "x", 1, 2))
    assert np.array_equal(bf16_bits_to_f32(norm_rope_upload(w, "x", 1, 3)), a)
    g = norm_rope_array(w, "gamma")
    assert g.shape == (w.d,) and abs(float(g.mean()) - 1.0) < 0.05
    c, s = rope_tables(w)
    assert c.shape == (w.L, w.d // 2) and c.dtype == np.float32
    assert np.allclose(c[0], 1.0) and np.allclose(s[0], 0.0)       # position 0: no rotation
    assert np.allclose(c * c + s * s, 1.0, atol=1e-6)
    f = custom_norm_rope(1, 1, 3, 64, dtype="fp32", rope=False)
    assert rope_tables(f) == (None, None) and norm_rope_array(f, "x").dtype == np.float32
