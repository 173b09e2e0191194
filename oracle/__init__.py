"""CPU oracle for the fused MXFP4 MoE forward.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product path.  It shares no code
with the HIP library.
"""
from .oracle import (  # noqa: F401
    lib_path,
    e2m1_value,
    e8m0_value,
    bf16_value,
    bf16_round,
    quant_block,
    quantize_rows,
    dequantize_rows,
    mx_dot,
    route,
    route_capacity,
    forward,
)
