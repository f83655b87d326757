"""CPU oracle (test infrastructure only): see ``oracle/lapnys_oracle.py``."""

from .lapnys_oracle import (  # noqa: F401
    attention_problem,
    conjugate_gradient,
    forward,
    gaussian_kernel,
    laplacian_kernel,
    newton_schulz_inverse,
    pool_landmarks,
    refine_inverse,
    whiten_columns,
)
