"""Seeded synthetic omni-modal KV streams (inputs only; no quantization arithmetic).

Both the fp64 oracle and the HIP path consume the arrays produced here; this
package computes nothing that the method itself defines.
"""
from .streams import (  # noqa: F401
    CONFIGS,
    MOD_VIDEO,
    MOD_AUDIO,
    MOD_TEXT,
    StreamConfig,
    Workload,
    bf16_bits_to_f64,
    calibration_queries,
    f64_to_bf16_bits,
    generate,
    hadamard_value_bases,
    lloyd_max_codebook,
    lloyd_max_codebook_2bit,
    sylvester_hadamard,
    workload_digest,
)
