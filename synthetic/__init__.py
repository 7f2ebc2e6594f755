"""Seeded synthetic inputs for Split-KV block-sparse draft attention.

This package draws random numbers and lays them out; it holds none of the
method's arithmetic (no mask, no attention, no cost model, no plan).  Both the
CPU oracle (through the tests and the bench) and the HIP path consume exactly
the arrays produced here, so both sides see identical bf16 bit patterns.
"""
from .workloads import (  # noqa: F401
    CONFIGS, Config, Workload, make, make_custom, add_own_block,
    bf16_bits_from_f32, f64_from_bf16_bits, f32_from_bf16_bits,
)
