"""Seeded synthetic inputs for the OneLA GDN decode step.

This package is shared by the tests, the bench and the smoke check. It holds
random draws, the bf16 encoding of inputs and the parent-selection rules of the
synthetic beam search, and none of the decode step's arithmetic.
"""
from .gen import (  # noqa: F401
    WORKLOADS,
    Shape,
    bf16_bits_to_f32,
    decode_inputs,
    f32_to_bf16_bits,
    gate_params,
    make_episode,
    make_raw_episode,
    prompt_tokens,
    shape_of,
)
