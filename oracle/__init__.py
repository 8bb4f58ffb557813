"""Float64 CPU oracle of exact RoPE attention with learnable log-frequencies.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library or its binding.  It shares
no code with the HIP path.
"""
from .ref import (thetas, theta_hat, angles, rotate, unrotate, wedge, ref_fwd,
                  ref_bwd, ref_dense, ref_head_rows, dalpha_chain)
from .dtft import dalpha_dtft, offset_signal, surrogate, surrogate_slope

__all__ = ["thetas", "theta_hat", "angles", "rotate", "unrotate", "wedge", "ref_fwd",
           "ref_bwd", "ref_dense", "ref_head_rows", "dalpha_chain", "dalpha_dtft",
           "offset_signal", "surrogate", "surrogate_slope"]
