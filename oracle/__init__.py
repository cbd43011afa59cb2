"""Float64 CPU oracle of the Muon step (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package; the HIP library never does.
"""
from .muon_oracle import *  # noqa: F401,F403
from .muon_oracle import (  # noqa: F401
    FAST_COEFFS,
    HYBRID_SCHEDULE,
    STABLE_COEFFS,
    Hyper,
    StepRecord,
)
