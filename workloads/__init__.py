"""Seeded synthetic workloads for the SALS decode path and post-prefill compaction.

This package only *draws inputs*: random low-rank key/value rows, projection
matrices, latent caches, queries and the VLM-shaped compaction cache. It holds
none of the method's arithmetic (no scoring, selection, reconstruction, RoPE,
attention or importance). Both the HIP path and the CPU oracle read the bytes
it produces, so they always see identical inputs.
"""

from .gen import (  # noqa: F401
    CONFIGS,
    CompactConfig,
    DecodeConfig,
    bf16_bits_to_f32,
    compact_case,
    decode_case,
    f32_to_bf16_bits,
    project_case,
    rng,
)
