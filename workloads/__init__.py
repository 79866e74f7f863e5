"""Seeded synthetic inputs for paged-KV prefill attention.

This package only *creates* inputs: sequence lengths, bf16-valued Q/K/V, a
paged KV pool with randomly permuted block tables, and multimodal-prefix
ranges.  It performs none of the attention arithmetic, so both the CPU oracle
(``oracle/``) and the HIP path (``paged_kv_prefill_attention_amd``) can consume
the same inputs without sharing any of the method's code.
"""

from .synth import (  # noqa: F401
    CONFIGS,
    Workload,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    NAMED,
    TILE_SWEEP,
    make_config,
    make_named,
    make_sweep,
    make_workload,
)
