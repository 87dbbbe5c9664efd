"""fp64 CPU oracle for Exact Flow Linear Attention (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this package. It shares no code with the HIP library.
"""
from .efla_oracle import (CHUNK, alpha, backward, chunk_forward, chunk_ut, coefficients, dphi,
                          euler_forward, forward, phi, rel_err, sequences)

__all__ = ["CHUNK", "alpha", "backward", "chunk_forward", "chunk_ut", "coefficients", "dphi",
           "euler_forward", "forward", "phi", "rel_err", "sequences"]
