"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This package prepares inputs only. It holds none of the arithmetic of the
subgraphs being computed, so the oracle and the HIP path can both consume
its arrays without sharing any of each other's code.
"""
from .inputs import (  # noqa: F401
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    gemm_act_inputs,
    gemm_ln_inputs,
    gemm_softmax_gemm_inputs,
    gemm_softmax_inputs,
    layernorm_affine_inputs,
    layernorm_inputs,
    normal,
    pow_bcast_add_inputs,
    rmsnorm_inputs,
    softmax_inputs,
    uniform,
    WORKLOADS,
)
