"""Seeded input generators for the stitched / GEMM-fused subgraphs.

Recipe (the same for every caller):
  * Each tensor draws from its own stream: numpy PCG64 seeded with
    SeedSequence([seed, tensor_id]); tensor ids are fixed per workload.
  * Normals are drawn in float64, scaled as mean + std * z; uniforms are
    float64 on [lo, hi).  Both are then rounded to float32 (round to nearest
    even, numpy's cast).  bfloat16 tensors are rounded once more, fp32 -> bf16,
    round to nearest even.
  * "N(a, b)" takes b as the standard deviation; the gamma vector of the
    GEMM + LayerNorm workload is 1 + N(0, 0.1).

Every array returned is the exact stored value: fp32 arrays are what the GPU
reads, and each bf16 tensor comes as (uint16 bit patterns, their exact fp32
values).  Nothing here computes any part of a subgraph.
"""
from __future__ import annotations

import numpy as np

# Shapes of the five workloads, by what they are.
WORKLOADS = {
    "softmax_256x1024": dict(rows=256, cols=1024),
    "layernorm_750000x32": dict(rows=750000, cols=32),
    "pow_bcast_add_softmax_64x30000": dict(rows=64, cols=30000),
    "gemm_ln_4096x4096x1024": dict(M=4096, N=4096, K=1024),
    "gemm_softmax_8192x8192x128": dict(M=8192, N=8192, D=128),
    "gemm_softmax_gemm_8192x8192x128x128": dict(M=8192, N=8192, D=128, Dv=128),
    "rmsnorm_750000x32": dict(rows=750000, cols=32),
    "layernorm_affine_750000x32": dict(rows=750000, cols=32),
    "gemm_gelu_4096x4096x1024": dict(M=4096, N=4096, K=1024),
}


def _rng(seed: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(tensor_id)])))


def normal(seed: int, tensor_id: int, shape, mean: float = 0.0, std: float = 1.0) -> np.ndarray:
    """float32 array of N(mean, std^2) draws, rounded from float64 to nearest fp32."""
    z = _rng(seed, tensor_id).standard_normal(size=shape, dtype=np.float64)
    return (mean + std * z).astype(np.float32)


def uniform(seed: int, tensor_id: int, shape, lo: float, hi: float) -> np.ndarray:
    """float32 array of U[lo, hi) draws, rounded from float64 to nearest fp32."""
    u = _rng(seed, tensor_id).random(size=shape, dtype=np.float64)
    return (lo + (hi - lo) * u).astype(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bits.

    The inputs here are finite, so NaN handling is not needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact float32 values of bfloat16 bit patterns."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _bf16(x_f32: np.ndarray):
    bits = f32_to_bf16_bits(x_f32)
    return bits, bf16_bits_to_f32(bits)


def softmax_inputs(seed: int = 1, rows: int = 256, cols: int = 1024) -> dict:
    """Row softmax workload: X fp32 [rows x cols] ~ N(0, 1)."""
    return {"x": normal(seed, 0, (rows, cols))}


def layernorm_inputs(seed: int = 2, rows: int = 750000, cols: int = 32) -> dict:
    """Tall-skinny LayerNorm (no affine) workload: X fp32 [rows x cols] ~ U(-1, 1)."""
    return {"x": uniform(seed, 0, (rows, cols), -1.0, 1.0)}


def rmsnorm_inputs(seed: int = 7, rows: int = 750000, cols: int = 32) -> dict:
    """RMSNorm workload: X fp32 [rows x cols] ~ U(-1, 1), gain fp32 [cols] = 1 + N(0, 0.1), eps = 1e-5."""
    return {
        "x": uniform(seed, 0, (rows, cols), -1.0, 1.0),
        "gamma": (np.float64(1.0) + normal(seed, 1, (cols,), std=0.1).astype(np.float64)).astype(np.float32),
        "eps": 1e-5,
    }


def layernorm_affine_inputs(seed: int = 8, rows: int = 750000, cols: int = 32) -> dict:
    """Affine LayerNorm workload: X fp32 [rows x cols] ~ U(-1, 1), gamma = 1 + N(0, 0.1), beta ~ N(0, 0.1)."""
    return {
        "x": uniform(seed, 0, (rows, cols), -1.0, 1.0),
        "gamma": (np.float64(1.0) + normal(seed, 1, (cols,), std=0.1).astype(np.float64)).astype(np.float32),
        "beta": normal(seed, 2, (cols,), std=0.1),
        "eps": 1e-5,
    }


def pow_bcast_add_inputs(seed: int = 3, rows: int = 64, cols: int = 30000) -> dict:
    """Expensive elementwise -> broadcast workload: v fp32 [rows] ~ U(0.1, 2), X fp32 [rows x cols] ~ N(0, 1).

    The exponent is 1.5.
    """
    return {
        "v": uniform(seed, 0, (rows,), 0.1, 2.0),
        "x": normal(seed, 1, (rows, cols)),
        "p": 1.5,
    }


def gemm_ln_inputs(seed: int = 4, M: int = 4096, N: int = 4096, K: int = 1024, residual: bool = True) -> dict:
    """GEMM + bias + residual + LayerNorm workload.

    A bf16 [M x K] ~ N(0,1); W bf16 [K x N] ~ N(0, 0.02); bias, beta fp32 [N] ~ N(0, 0.1);
    gamma fp32 [N] = 1 + N(0, 0.1); R bf16 [M x N] ~ N(0, 1); eps = 1e-5.
    """
    a_bits, a = _bf16(normal(seed, 0, (M, K)))
    w_bits, w = _bf16(normal(seed, 1, (K, N), std=0.02))
    out = {
        "a_bits": a_bits, "a": a,
        "w_bits": w_bits, "w": w,
        "bias": normal(seed, 2, (N,), std=0.1),
        "gamma": (np.float64(1.0) + normal(seed, 3, (N,), std=0.1).astype(np.float64)).astype(np.float32),
        "beta": normal(seed, 4, (N,), std=0.1),
        "eps": 1e-5,
    }
    if residual:
        r_bits, r = _bf16(normal(seed, 5, (M, N)))
        out["r_bits"], out["r"] = r_bits, r
    else:
        out["r_bits"], out["r"] = None, None
    return out


def gemm_act_inputs(seed: int = 9, M: int = 4096, N: int = 4096, K: int = 1024, positive: bool = False) -> dict:
    """GEMM + bias + activation workload: A bf16 [M x K] ~ N(0, 1); W bf16 [K x N] ~ N(0, 0.02);
    bias fp32 [N] ~ N(0, 0.1) (the GEMM + LayerNorm workload's operands without the residual).

    ``positive``: A ~ U(0.5, 1.5), W ~ U(0, 0.02), bias ~ U(0, 0.1) instead, so every entry of
    A.W + bias is positive (the domain of an rsqrt epilogue)."""
    if positive:
        a_bits, a = _bf16(uniform(seed, 0, (M, K), 0.5, 1.5))
        w_bits, w = _bf16(uniform(seed, 1, (K, N), 0.0, 0.02))
        bias = uniform(seed, 2, (N,), 0.0, 0.1)
    else:
        a_bits, a = _bf16(normal(seed, 0, (M, K)))
        w_bits, w = _bf16(normal(seed, 1, (K, N), std=0.02))
        bias = normal(seed, 2, (N,), std=0.1)
    return {"a_bits": a_bits, "a": a, "w_bits": w_bits, "w": w, "bias": bias}


def gemm_softmax_inputs(seed: int = 5, M: int = 8192, N: int = 8192, D: int = 128) -> dict:
    """GEMM + scaled row softmax workload: Q bf16 [M x D], K bf16 [N x D], both ~ N(0, 1).

    The scale is the float32 value nearest 1/sqrt(D); both sides receive that stored value.
    """
    q_bits, q = _bf16(normal(seed, 0, (M, D)))
    k_bits, k = _bf16(normal(seed, 1, (N, D)))
    return {
        "q_bits": q_bits, "q": q,
        "k_bits": k_bits, "k": k,
        "scale": float(np.float32(1.0 / np.sqrt(np.float64(D)))),
    }


def gemm_softmax_gemm_inputs(seed: int = 6, M: int = 8192, N: int = 8192, D: int = 128, Dv: int = 128) -> dict:
    """Back-to-back GEMM workload, O = softmax(scale * Q.K^T).V: Q bf16 [M x D], K bf16 [N x D],
    V bf16 [N x Dv], all ~ N(0, 1).

    The scale is the float32 value nearest 1/sqrt(D); both sides receive that stored value.
    """
    q_bits, q = _bf16(normal(seed, 0, (M, D)))
    k_bits, k = _bf16(normal(seed, 1, (N, D)))
    v_bits, v = _bf16(normal(seed, 2, (N, Dv)))
    return {
        "q_bits": q_bits, "q": q,
        "k_bits": k_bits, "k": k,
        "v_bits": v_bits, "v": v,
        "scale": float(np.float32(1.0 / np.sqrt(np.float64(D)))),
    }
