"""Float64 CPU oracle for exact softmax attention (test infrastructure only).

Only the test suite, the package smoke check and the benchmark's CPU-baseline leg import
this package. It shares no code with the GPU library and never calls it.
"""
from .fp8 import fp8_forward, round_e4m3  # noqa: F401
from .attention import (  # noqa: F401
    visibility,
    unit_forward,
    unit_backward,
    attention_forward,
    attention_backward,
    rows_forward,
    rows_backward_dq,
    keys_backward,
)
