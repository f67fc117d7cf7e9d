"""Seeded synthetic inputs for paged GQA decode attention.

This package only draws random numbers and lays them out as a paged KV cache;
it performs none of the attention arithmetic.  Both the CPU oracle (``oracle/``)
and the HIP library are fed from here, and neither imports the other.
"""
from .gen import (  # noqa: F401
    APPEND_CONFIGS,
    CONFIGS,
    PREFILL_CONFIGS,
    ROPE_THETA,
    AppendInputs,
    Case,
    PrefillInputs,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_append_case,
    make_append_config,
    make_append_inputs,
    make_case,
    make_config,
    make_prefill_case,
    make_prefill_config,
)
