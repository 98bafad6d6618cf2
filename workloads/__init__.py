"""Seeded synthetic inputs for gated retention (shared by tests, smoke and bench).

This package only draws random numbers and rounds them to the storage types.
It contains none of the retention arithmetic, so both the HIP path and the
fp64 oracle can be fed from it without sharing any computation.
"""
from .gret_inputs import (  # noqa: F401
    CONFIGS,
    LN_SHARP_GAMMA,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    gate_log_gamma,
    make_attention_inputs,
    make_decode_inputs,
    make_prefill_inputs,
    make_projection_inputs,
    prefill_head,
    slow_decay_log_gamma,
)
