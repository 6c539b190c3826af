"""CPU float64 oracle for the Muon step.

TEST INFRASTRUCTURE ONLY: imported by the tests, the package smoke check and
the benchmark's CPU-baseline leg, never by the product path.
"""

from .muon_oracle import (  # noqa: F401
    BETA,
    NS_A,
    NS_B,
    NS_C,
    NS_EPS,
    NS_STEPS,
    Hyper,
    StepResult,
    block_corners,
    decode,
    frobenius_normalize,
    momentum_update,
    muon_overhead_fraction,
    muon_step,
    muon_step_matrix,
    muon_step_matrix_blocked,
    newton_schulz,
    ns_flops_dense,
    ns_flops_unique,
    ns_iterate,
    param_update,
    shape_scale,
    update_direction,
)
from .adamw_oracle import AdamWHyper, AdamWResult, adamw_step  # noqa: F401,E402
