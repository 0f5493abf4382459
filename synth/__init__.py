"""Seeded synthetic inputs for MLA decode.

This package is shared by the tests, the benchmark and the oracle's callers.
It only draws random numbers and packs them into the stored formats
(fp32, bf16, fp8-e4m3 with a per-row fp32 scale, contiguous or paged cache
layouts).  It contains none of the attention arithmetic: decoding the stored
bits back to values is done independently by each consumer.
"""

from .rng import splitmix64_bits, uniform01, standard_normal, randint_uniform, permutation
from .encode import round_to_f32, f32_to_bf16_bits, bf16_bits_to_f32, quantize_rows_e4m3
from .workloads import (
    Workload,
    WORKLOADS,
    workload,
    MLAInputs,
    make_inputs,
    cache_bytes,
)

__all__ = [
    "splitmix64_bits",
    "uniform01",
    "standard_normal",
    "randint_uniform",
    "permutation",
    "round_to_f32",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "quantize_rows_e4m3",
    "Workload",
    "WORKLOADS",
    "workload",
    "MLAInputs",
    "make_inputs",
    "cache_bytes",
]
