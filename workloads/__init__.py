"""Seeded synthetic inputs shared by the GPU path's tests/bench and the CPU oracle.

This package draws random logits and per-row k / p controls. It holds none of
the selection method's arithmetic: no ordering, no thresholds, no softmax.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    EXTRA,
    Inputs,
    f32_to_bf16_bits,
    bf16_bits_to_f32,
    make_config,
    make_extra,
    make_rows,
    ROW_KINDS,
)
