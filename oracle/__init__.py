"""CPU oracle for the Simple GLA mixer (float64, token by token).

TEST INFRASTRUCTURE ONLY: used by the tests, the package smoke check and the
benchmark's CPU-baseline leg.  The product path never imports it.
"""
from .gla_oracle import (forward, forward_packed, step, backward, conv1d_silu, state_bytes,  # noqa: F401
                         q16_encode, q16_decode, step_q16, Q16_MAX, Q16_NAN, gate_silu, forward_gated)
