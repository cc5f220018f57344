"""Seeded synthetic inputs shared by the oracle checks, the GPU tests and the bench.

This package only draws random tensors of the shapes and structure of the
video-DiT attention workloads (Q, K, V per head over a latent T x H x W grid).
It contains none of the routing or attention arithmetic: the oracle and the
HIP path both consume what it produces and never import each other.
"""

from .workloads import (  # noqa: F401
    WORKLOADS,
    Workload,
    Inputs,
    bf16_bits_to_f64,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_inputs,
    get_workload,
)
