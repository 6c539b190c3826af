"""Seeded synthetic inputs for the Muon step (weights, gradients, momenta).

This package is shared by the CPU oracle's tests and by the GPU path's tests
and benchmark.  It holds input generation and storage encoding only: none of
the optimizer's arithmetic lives here.
"""

from .gen import (  # noqa: F401
    ADAMW_WORKLOADS,
    WORKLOADS,
    AdamWWorkload,
    TensorSpec,
    adamw_workload,
    make_adamw_grad,
    make_adamw_param,
    MatSpec,
    Workload,
    bf16_bits_to_f32,
    encode_storage,
    expert_scale,
    gaussian,
    heavy_tail_grad,
    lowrank_noise_grad,
    make_grad,
    make_momentum,
    make_param,
    rng_for,
    workload,
)
