"""fp64 CPU oracle for the TTT-with-KV-binding forward pass and the
backward of the per-token and large-chunk linear modes.

Test infrastructure only: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the library or its binding.
"""
from .ttt_oracle import (  # noqa: F401
    NORM_EPS,
    NS_COEFFS,
    NS_EPS,
    NS_STEPS,
    backward,
    forward,
    large_chunk_linear,
    large_chunk_linear_backward,
    large_chunk_swiglu,
    large_chunk_swiglu_backward,
    linear_binding_grad,
    linear_binding_loss,
    newton_schulz5,
    normalize_columns,
    per_token_linear,
    per_token_linear_backward,
    silu,
    silu_prime,
    silu_second,
    swiglu_read_backward,
    swiglu_step_vjp,
    swiglu_binding_grad,
    swiglu_binding_loss,
    swiglu_forward,
    swiglu_pack,
    swiglu_unpack,
)
