"""Seeded synthetic workloads shared by the oracle-side tests and the GPU path.

This package holds shapes and random inputs only; it contains none of the
attention method's arithmetic (no reorder, sampling, softmax or masking).
"""
from .configs import CONFIGS, Config, get_config  # noqa: F401
from .generator import bf16_round, bf16_bits, make_inputs, make_head  # noqa: F401
