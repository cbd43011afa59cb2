"""Seeded synthetic inputs for the Muon-step workloads.

This package holds input generation only (shapes, seeds, value
distributions).  It contains none of the optimizer's arithmetic, and is the
one module that both the float64 oracle's tests and the HIP path's tests and
benchmark draw inputs from.
"""
from .configs import CONFIGS, MatrixSpec, Workload, workload  # noqa: F401
from .gen import (  # noqa: F401
    bank_grads,
    bank_weights,
    grad_tensor,
    matrix_offsets,
    init_weight,
    seed_of,
    zero_experts,
)
