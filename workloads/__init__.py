"""Seeded synthetic inputs for the block-sparse global attention path.

This package holds shapes, seeds and random draws only. It performs none of the
method's arithmetic (no pooling, scoring, selection or attention), so both the
HIP path and the CPU oracle can take their inputs from it without sharing any
computation.
"""
from .synthetic import (  # noqa: F401
    Layout,
    Workload,
    CONFIGS,
    config,
    generate,
    bf16_bits_from_float,
    float_from_bf16_bits,
    keep_from_sparsity,
)
