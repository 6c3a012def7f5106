"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This package holds only input generation (counter-based random numbers and
their mapping to codes, scales and activations).  It contains none of the
matrix product's arithmetic and imports neither the oracle nor the HIP
library.
"""
from .gen import (  # noqa: F401
    rand_u32,
    binary_codes,
    ternary_codes,
    group_scales,
    normal_bf16,
    normal_f32,
    sign_bits,
    f32_to_bf16_bits,
    bf16_bits_to_f32,
    device_codes,
    device_scales,
    device_u32,
)
