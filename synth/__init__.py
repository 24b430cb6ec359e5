"""Seeded synthetic workloads for batched draft verification.

This package only draws random numbers: logits, draft tokens (the draft model's stand-in),
Saguaro sets chosen by that stand-in, and verification uniforms. It holds none of the
verification arithmetic, and both the HIP path and the oracle read its output.
"""
from .gen import (  # noqa: F401
    BF16,
    F32,
    VerifyBatch,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_branch_rows,
    make_branch_uniforms,
    make_verify_batch,
    workload,
    WORKLOADS,
)
