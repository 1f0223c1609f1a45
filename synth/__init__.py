"""Seeded synthetic inputs shared by the oracle-side tests, the HIP-path tests and bench.py.

This package draws random numbers and nothing else: it holds none of the method's
arithmetic (no projection, no Sinkhorn, no top-k, no attention).
"""
from .configs import CONFIGS, Config, config_by_name  # noqa: F401
from .gen import (  # noqa: F401
    assign_inputs,
    qkv_inputs,
    bf16_round,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    random_groups,
    seed_streams,
)
