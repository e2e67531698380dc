"""Seeded synthetic inputs for the equivariant attention layer.

This package only draws geometry, features and weights.  It holds none of the
layer's arithmetic, so both the fp64 oracle (through the tests) and the HIP
path (through the tests and the benchmark) can take their inputs from it.
"""
from .generators import (  # noqa: F401
    CONFIGS,
    Workload,
    axis_lattice_geometry,
    bf16_round,
    block_weights_f32,
    bf16_to_f32,
    coincident_geometry,
    f32_to_bf16_bits,
    make_block_weights,
    make_config,
    so2_param_count,
)
