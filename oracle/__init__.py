"""CPU oracle for the Dual-AR per-frame decode step.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this package.  The HIP library never
calls it, and it shares no code with the HIP library.
"""
from .dualar_oracle import (  # noqa: F401
    DualAROracle,
    Sampling,
    bf16_round,
    count_params,
    dequant_w4,
    embed_column,
    param_shapes,
    rope_table,
    sample_token,
)
