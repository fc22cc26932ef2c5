"""Seeded synthetic inputs for the WAITS prefill KV-selection path and for
decode attention over the compacted cache.

This package only draws random tensors and packs them; it holds none of the
method's arithmetic, so both the CPU oracle's tests and the GPU path's tests
and benchmark can use it without sharing any computation.
"""
from .gen import (  # noqa: F401
    ACTIONS,
    bf16_bits,
    bf16_bits_to_f32,
    make_prompt,
    make_batch,
    make_decode,
    Batch,
    DecodeInputs,
)
