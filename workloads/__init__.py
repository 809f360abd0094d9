"""Seeded synthetic inputs for the batched token sampler.

This package only draws input data (logits, per-row parameters, history ids).
It holds none of the sampler's arithmetic, so both the CPU oracle and the GPU
path can consume what it produces without sharing any method code.
"""

from .gen import (  # noqa: F401
    DRY_DTYPE,
    PARAMS_DTYPE,
    make_dry,
    V_DEFAULT,
    Workload,
    make_params,
    make_workload,
    f32_to_bf16_bits,
    bf16_bits_to_f32,
    WORKLOAD_NAMES,
)
