"""Seeded synthetic inputs for the attention-JVP workloads.

This package holds shapes, value distributions, seeding and dtype rounding
only.  It contains none of the attention arithmetic, so that both the fp64
oracle (``oracle/``) and the HIP path can be fed from it without sharing any
computation.
"""
from .configs import WORKLOADS, TENSORS, Workload, custom_workload  # noqa: F401
from .inputs import (  # noqa: F401
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    head_array,
    head_upload,
    sample_rows,
    tq_head_scale,
)
from .norm_rope import (  # noqa: F401
    NORM_ROPE_TENSORS,
    NORM_ROPE_WORKLOADS,
    NormRopeWorkload,
    custom_norm_rope,
    norm_rope_array,
    norm_rope_upload,
    rope_tables,
)
from .proj import (  # noqa: F401
    PROJ_TENSORS,
    PROJ_WORKLOADS,
    ProjWorkload,
    custom_proj,
    proj_array,
    proj_host_inputs,
    proj_upload,
)
