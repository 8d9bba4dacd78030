"""Seeded synthetic inputs for the paged-KV attention hot path.

This package only draws numbers and lays them out (block tables, pool
contents, slot mappings).  It holds none of the attention arithmetic, so both
the CPU oracle (``oracle/``) and the HIP path can be fed from it without
sharing any computation.
"""
from .synth import (  # noqa: F401
    BF16_NAN,
    CONFIG_SEEDS,
    DecodeInputs,
    PrefillInputs,
    bf16_bits_from_f32,
    config,
    cu_seqlens_from_lens,
    decode_case,
    mixed_case,
    prefill_case,
    slot_for_position,
)
