"""CPU fp64 oracle for the shared-expert SwiGLU MLP, the sharded MLA latent
projection and the replicated-vs-sharded layout choice (test infrastructure).

This package is test infrastructure. Only ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py`` may import it; the product path (the
HIP library and its Python binding) never does, and it shares no code with it.

Every function takes float64 numpy arrays (exact widenings of the fp32 or
bf16 values a GPU reads) and computes in float64 with no rounding to a
narrower type anywhere.
"""
from .swiglu_mlp import (  # noqa: F401
    silu,
    gate_up_act,
    down_proj,
    swiglu_mlp,
    rank_shard,
    rank_partial,
    slice_sum,
    rank_token_rows,
    feature_concat_design,
    rms_rescale_rows,
    shard_sequence_parallel_mlp,
)
from .mla_latent import (  # noqa: F401
    check_geometry,
    linear,
    merged_column_shard,
    gather_rank_major,
    restore_logical,
    sharded_projection,
)
from . import layout  # noqa: F401
