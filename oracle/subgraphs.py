"""The five subgraphs, composed operator by operator in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Readings taken where the pages leave a point open (each is also listed with
its reason in the design notes):
  * LayerNorm uses the population variance (divide by the row length) with
    eps inside the square root; the residual is added before the statistics.
  * Softmax subtracts the row maximum before exp (a no-op in exact arithmetic).
  * The power result v_i^p is a per-row (column-vector) broadcast: Y_ij = X_ij + v_i^p.
  * bias, gamma and beta are length-N vectors broadcast over rows (row-vector
    broadcasts, indexed by the output column).
  * Q.K^T takes K row-major [N x D]; the scale multiplies the accumulator
    before the softmax.
  * The back-to-back product takes its second operand V row-major [N x Dv]
    (keys by output columns): O = S.V with S the scaled row softmax above.
  * The activation epilogue's GELU is the tanh form; SiLU is x * sigmoid(x);
    its rsqrt is 1/sqrt(u) with no eps (the norms' eps belongs to their stage).
  * RMSNorm divides by the root of the mean square (over the row length) plus
    eps; its gain gamma, like LayerNorm's gamma and beta, is a length-cols
    row-vector broadcast, and a missing gain is 1.
"""
from __future__ import annotations

import numpy as np

from . import ops


def softmax_rows(x) -> np.ndarray:
    """Row softmax as a chain of stages: max-reduce -> broadcast subtract -> exp -> sum-reduce -> broadcast divide.

    ComFuse, Stage-Stream Execution Model (stage chaining): each reduction ends
    a stage and its broadcast result feeds the next stage; softmax is named
    among the patterns the recursive split at reduction nodes covers
    (Frontend / Fusion Spec IR).  AStitch summary, "What people did before":
    a reduction feeding many consumers is the one-to-many pattern.
    """
    x = ops.f64(x)
    m = ops.rowmax(x)
    d = ops.sub_colvec(x, m)
    e = ops.map_exp(d)
    s = ops.rowsum(e)
    return ops.div_colvec(e, s)


def layernorm_rows(x, eps: float = 1e-5) -> np.ndarray:
    """LayerNorm without affine: row sum -> mean broadcast -> x - mean -> square -> row sum -> rsqrt(var + eps) -> multiply.

    ComFuse, Stage-Stream Execution Model, bypass path (Fig. 3): the stage-1
    value x feeds both the mean reduction and the stage-2 term x - mean;
    Frontend / Fusion Spec IR: LayerNorm reduces over its inputs and then
    normalizes the original values.
    """
    x = ops.f64(x)
    n = x.shape[1]
    s = ops.rowsum(x)
    mu = s / np.float64(n)
    c = ops.sub_colvec(x, mu)
    q = ops.map_square(c)
    var = ops.rowsum(q) / np.float64(n)
    r = ops.map_rsqrt_eps(var, eps)
    return ops.mul_colvec(c, r)


def pow_bcast_add_softmax(x, v, p: float = 1.5):
    """Y = X + broadcast_col(v^p), then the row softmax of Y.  Returns (softmax(Y), Y).

    AStitch summary, "What people did before": power -> broadcast -> add is
    the expensive-elementwise-feeding-a-broadcast pattern; the 64 x 30000 row
    reduction is its short-wide irregular shape.
    """
    x = ops.f64(x)
    v = ops.f64(v)
    pv = ops.map_pow(v, p)
    y = ops.add_colvec(x, pv)
    return softmax_rows(y), y


def gemm_ln(a, w, bias, r, gamma, beta, eps: float = 1e-5) -> np.ndarray:
    """Y = LayerNorm(A.W + bias + R) * gamma + beta over each output row.

    ComFuse, Stage-Stream Execution Model (Fig. 3): stage 1 forms
    x = alpha * Acc + Bias (alpha = 1 here) and the mean; later stages normalize.
    Frontend / Fusion Spec IR (Phi patterns): 1-D parameters are row-vector
    broadcasts.  ``r`` may be None (no residual).
    """
    z = ops.matmul(ops.f64(a), ops.f64(w))
    u = ops.add_rowvec(z, ops.f64(bias))
    if r is not None:
        u = ops.add(u, ops.f64(r))
    n = layernorm_rows(u, eps)
    return ops.add_rowvec(ops.mul_rowvec(n, ops.f64(gamma)), ops.f64(beta))


def gemm_softmax(q, k, scale: float) -> np.ndarray:
    """S = softmax(scale * Q.K^T) over each output row.

    ComFuse, B2BGEMM (eq. 3): the first MatMul's tile P is turned into
    S = F(P) by a fused epilogue; here F is the scaled row softmax, and the
    constant is a scalar broadcast (Phi patterns).
    """
    p = ops.matmul(ops.f64(q), ops.transpose(ops.f64(k)))
    s = ops.scale(p, scale)
    return softmax_rows(s)


def gemm_softmax_gemm(q, k, v, scale: float) -> np.ndarray:
    """O = softmax(scale * Q.K^T) . V: two MatMuls back to back with the softmax between them.

    ComFuse, B2BGEMM: the first MatMul's tile P becomes S = F(P) (eq. 3) with
    F the scaled row softmax, and the second MatMul multiplies S by W2 = V
    (eq. 4-5: partial products over the contraction dimension N1 summed into
    the output tile; here the whole sum is one matmul, eq. 6 shapes
    X = Q [M x K], W1 = K^T [K x N1], W2 = V [N1 x N2]).
    """
    s = gemm_softmax(q, k, scale)
    return ops.matmul(s, ops.f64(v))


def layernorm_affine_rows(x, gamma, beta, eps: float = 1e-5) -> np.ndarray:
    """LayerNorm followed by its affine map: LayerNorm(x) * gamma + beta per row.

    ComFuse, Frontend / Fusion Spec IR: LayerNorm among the stage DAGs the
    recursive split covers, and 1-D parameters as row-vector broadcasts (Phi
    patterns); the affine map is the output stage after the two reductions.
    """
    n = layernorm_rows(x, eps)
    return ops.add_rowvec(ops.mul_rowvec(n, ops.f64(gamma)), ops.f64(beta))


def rmsnorm_rows(x, gamma=None, eps: float = 1e-5) -> np.ndarray:
    """RMSNorm: square -> row sum -> mean -> rsqrt(ms + eps) -> multiply (-> times gamma).

    ComFuse, Stage-Stream Execution Model: one reduction stage whose broadcast
    result scales the original values held from the first stage (bypass path);
    the gain is a row-vector broadcast (Phi patterns).  ``gamma`` None means 1.
    """
    x = ops.f64(x)
    n = x.shape[1]
    ms = ops.rowsum(ops.map_square(x)) / np.float64(n)
    r = ops.map_rsqrt_eps(ms, eps)
    y = ops.mul_colvec(x, r)
    if gamma is not None:
        y = ops.mul_rowvec(y, ops.f64(gamma))
    return y


# activation name -> the ops function that computes it (looked up per call)
ACTIVATIONS = {"none": None, "relu": "map_relu", "gelu_tanh": "map_gelu_tanh", "silu": "map_silu",
               "square": "map_square", "rsqrt": "map_rsqrt"}


def gemm_act(a, w, bias, act: str) -> np.ndarray:
    """Y = act(A.W + bias): a GEMM with a unary-activation epilogue, per output element.

    ComFuse, Stage-Stream Execution Model (Fig. 3: x = alpha * Acc + Bias, alpha = 1)
    followed by one elementwise stage; Frontend / Fusion Spec IR names
    activations, rsqrt and squares among the unary operators that become
    computation nodes.  ``bias`` may be None.
    """
    z = ops.matmul(ops.f64(a), ops.f64(w))
    if bias is not None:
        z = ops.add_rowvec(z, ops.f64(bias))
    name = ACTIVATIONS[act]
    return z if name is None else getattr(ops, name)(z)
