"""Float64 CPU oracle for the fused linear cross-entropy + entropy head.

Test infrastructure only: the test suite, the smoke check and the benchmark's
CPU-baseline leg import this package. The GPU library never does.
"""
from .flce_oracle import (  # noqa: F401
    softcap,
    softcap_grad,
    logits,
    row_stats,
    forward,
    dlogits,
    backward,
    dhidden_rows,
    dweight_columns,
)
