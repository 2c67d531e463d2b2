"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

Nothing in this package computes any step of the attention layer: it only
draws random tensors and converts them to storage formats (fp32 or the
16-bit bfloat16 bit pattern).
"""
from .inputs import (  # noqa: F401
    CONFIGS, Config, bf16_bits_from_f32, block_tensor, f32_from_bf16_bits, head_tensor,
    make_inputs, planted_positions, storage_to_f32,
)
