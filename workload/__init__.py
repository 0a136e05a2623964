"""Seeded synthetic inputs for absorbed MLA decode.

This package builds inputs only: page tables, pools, queries, scales, and
the inputs of the prepare step (weights, new rows, a RoPE cos / sin table).  It holds
none of the attention arithmetic, so both the GPU path's tests and the CPU
oracle can consume the same tensors without sharing any computation.
"""

from .gen import (  # noqa: F401
    DecodeInputs,
    CONFIGS,
    SWEEP_BATCHES,
    config_inputs,
    make_inputs,
    shard_from_full,
    local_lengths,
    ragged_lengths,
    softmax_scale_default,
    kv_bytes_per_token,
    PREPARE_CONFIGS,
    prepare_inputs,
)
