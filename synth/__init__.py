"""Seeded synthetic inputs for the chunk-wise fast-weight update.

This package holds input recipes only (random draws, RMS row scaling, bf16
rounding of the drawn values). It contains none of the method's arithmetic, so
both the CPU oracle and the HIP path can take their inputs from it.
"""
from .workloads import (  # noqa: F401
    CONFIGS,
    Workload,
    bf16_round,
    bf16_bits,
    make_inputs,
    make_config,
    make_target_conv,
)
