"""fp64 CPU oracle for the Falcon forward pass and the Falcon-1 backward pass
(test infrastructure only).

Only the tests, the smoke check and the CPU-baseline leg of the benchmark
import this package; the HIP library never does.
"""
from .falcon_oracle import (F1, F2, F3, F1A, F2A, F3A, VARIANTS, WINDOW_VARIANTS, PER_COLUMN,
                            PHI_RMSNORM, PHI_IDENTITY, OracleState, OracleTrace,
                            falcon_forward, phi, window_lambda_max)
from .falcon_backward import falcon1_backward, phi_vjp

__all__ = ["F1", "F2", "F3", "F1A", "F2A", "F3A", "VARIANTS", "WINDOW_VARIANTS", "PER_COLUMN",
           "PHI_RMSNORM", "PHI_IDENTITY", "OracleState", "OracleTrace",
           "falcon_forward", "phi", "window_lambda_max", "falcon1_backward", "phi_vjp"]
