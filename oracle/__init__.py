"""fp64 CPU oracle for the attention-JVP hot path (test infrastructure only).

Only the tests, the smoke check (`__graft_entry__.smoke`) and the benchmark's cpu_baseline leg may
import this package.  The product library never does.
"""
from .attn_jvp import attention_jvp, attention_jvp_head, merge_shards  # noqa: F401
from .norm_rope import norm_rope_jvp  # noqa: F401
from .proj import projection_jvp  # noqa: F401
