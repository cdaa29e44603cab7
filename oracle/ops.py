"""Whole-array float64 operators the oracle composes.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Vocabulary, after the AStitch summary page ("Why this problem is worth
solving"): elementwise operators (cheap ones such as add and multiply,
expensive ones such as power and exp), reductions over a tensor dimension,
and broadcasts that replicate a value across a dimension.  Following the
ComFuse page (Frontend / Fusion Spec IR, the Phi patterns), a binary operator
against a lower-rank operand is a broadcast followed by the computation, a
one-dimensional parameter is a row-vector broadcast, and a constant is a
scalar broadcast.  Each broadcast below is written out explicitly with
np.broadcast_to so the reader sees which axis is replicated.

Every function takes and returns float64 arrays and materializes its result.
"""
from __future__ import annotations

import numpy as np


def f64(x) -> np.ndarray:
    """Widen stored values (fp32 or exact-bf16 fp32) to float64 exactly."""
    return np.asarray(x, dtype=np.float64)


# --- reductions over the last (row) dimension -------------------------------

def rowmax(x: np.ndarray) -> np.ndarray:
    """m_i = max_j x_ij."""
    return np.max(x, axis=1)


def rowsum(x: np.ndarray) -> np.ndarray:
    """s_i = sum_j x_ij."""
    return np.sum(x, axis=1)


# --- broadcasts ---------------------------------------------------------------

def bcast_col(c: np.ndarray, cols: int) -> np.ndarray:
    """B_ij = c_i: a per-row value replicated along the row."""
    return np.broadcast_to(c[:, None], (c.shape[0], cols))


def bcast_row(r: np.ndarray, rows: int) -> np.ndarray:
    """B_ij = r_j: a length-N vector replicated over every row (row-vector broadcast)."""
    return np.broadcast_to(r[None, :], (rows, r.shape[0]))


# --- binary elementwise ------------------------------------------------------

def add(x: np.ndarray, y: np.ndarray) -> np.ndarray:
    assert x.shape == y.shape
    return x + y


def sub(x: np.ndarray, y: np.ndarray) -> np.ndarray:
    assert x.shape == y.shape
    return x - y


def mul(x: np.ndarray, y: np.ndarray) -> np.ndarray:
    assert x.shape == y.shape
    return x * y


def div(x: np.ndarray, y: np.ndarray) -> np.ndarray:
    assert x.shape == y.shape
    return x / y


def sub_colvec(x: np.ndarray, c: np.ndarray) -> np.ndarray:
    """x_ij - c_i."""
    return sub(x, bcast_col(c, x.shape[1]))


def div_colvec(x: np.ndarray, c: np.ndarray) -> np.ndarray:
    """x_ij / c_i."""
    return div(x, bcast_col(c, x.shape[1]))


def mul_colvec(x: np.ndarray, c: np.ndarray) -> np.ndarray:
    """x_ij * c_i."""
    return mul(x, bcast_col(c, x.shape[1]))


def add_colvec(x: np.ndarray, c: np.ndarray) -> np.ndarray:
    """x_ij + c_i."""
    return add(x, bcast_col(c, x.shape[1]))


def add_rowvec(x: np.ndarray, r: np.ndarray) -> np.ndarray:
    """x_ij + r_j."""
    return add(x, bcast_row(r, x.shape[0]))


def mul_rowvec(x: np.ndarray, r: np.ndarray) -> np.ndarray:
    """x_ij * r_j."""
    return mul(x, bcast_row(r, x.shape[0]))


# --- unary elementwise -------------------------------------------------------

def map_exp(x: np.ndarray) -> np.ndarray:
    return np.exp(x)


def map_square(x: np.ndarray) -> np.ndarray:
    return x * x


def map_pow(x: np.ndarray, p: float) -> np.ndarray:
    return np.power(x, np.float64(p))


def map_rsqrt_eps(x: np.ndarray, eps: float) -> np.ndarray:
    """1 / sqrt(x + eps), with eps inside the root."""
    return 1.0 / np.sqrt(x + np.float64(eps))


def scale(x: np.ndarray, a: float) -> np.ndarray:
    """a * x for a scalar constant a (a scalar broadcast)."""
    return x * np.float64(a)


# --- contraction -------------------------------------------------------------

def transpose(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x.T)


def matmul(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Z_ij = sum_k a_ik b_kj in float64 (library dgemm as one step)."""
    assert a.ndim == 2 and b.ndim == 2 and a.shape[1] == b.shape[0]
    return a @ b


def map_relu(x: np.ndarray) -> np.ndarray:
    return np.maximum(x, 0.0)


def map_gelu_tanh(x: np.ndarray) -> np.ndarray:
    """0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))), the tanh form of GELU."""
    c = np.sqrt(np.float64(2.0) / np.pi)
    return 0.5 * x * (1.0 + np.tanh(c * (x + 0.044715 * x * x * x)))


def map_rsqrt(x: np.ndarray) -> np.ndarray:
    """1 / sqrt(x), no eps (inf at 0, nan below)."""
    return 1.0 / np.sqrt(x)


def map_silu(x: np.ndarray) -> np.ndarray:
    """x * sigmoid(x) = x / (1 + exp(-x))."""
    return x / (1.0 + np.exp(-x))
