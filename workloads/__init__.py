"""Seeded synthetic workloads for the Dion / Orth-Dion step.

This package only draws inputs (shapes, random matrices, dtype rounding).  It
holds none of the step's arithmetic, and both the CPU oracle and the GPU path
consume exactly the bytes it produces.
"""
from .configs import (  # noqa: F401
    CONFIGS, MatrixSpec, Workload, config, stack_160m, stack_3b,
)
from .generators import (  # noqa: F401
    MatrixStream, bf16_bits_to_f32, conditioned_inputs, f32_to_bf16_bits,
    random_orthonormal, rng,
)
