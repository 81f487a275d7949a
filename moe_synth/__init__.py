"""Seeded synthetic inputs for the MoE FFN forward.

This package only draws and encodes inputs (token activations, router logits,
expert weights, dropped-slot masks).  It computes no step of the forward pass:
routing, permutation, the expert FFNs and the combine live in the HIP library
(the product) and, independently, in the CPU oracle (test infrastructure).
Both sides read the arrays produced here and nothing else is shared.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    MoeConfig,
    bf16_bits_from_f32,
    bf16_bits_to_f32,
    deinterleave_rows,
    generate,
    interleave_rows,
    w4a8_sweep_tokens,
)
