"""Plant plausible mistakes in the oracle (CPU only) and check the pins catch each one.

A mistake counts as caught when at least one pin raises (a wrong value, a
non-finite value, or a shape error all count).
"""
import math

import numpy as np
import pytest

import oracle
from oracle import graph, ops, subgraphs
from tests import pins


def _graph_as_tile_swapped(kind, v, rows, cols):
    if kind == "row":
        return ops.bcast_row(v, rows)
    if kind == "vec":
        return ops.bcast_col(v, cols)
    return graph.np.full((rows, cols), v) if kind == "scalar" else v


def _ln_sample_variance(x, eps=1e-5):
    x = ops.f64(x)
    n = x.shape[1]
    mu = ops.rowsum(x) / n
    c = ops.sub_colvec(x, mu)
    var = ops.rowsum(ops.map_square(c)) / (n - 1)
    return ops.mul_colvec(c, ops.map_rsqrt_eps(var, eps))


def _ln_no_center_in_output(x, eps=1e-5):
    x = ops.f64(x)
    n = x.shape[1]
    mu = ops.rowsum(x) / n
    c = ops.sub_colvec(x, mu)
    var = ops.rowsum(ops.map_square(c)) / n
    return ops.mul_colvec(x, ops.map_rsqrt_eps(var, eps))


def _gemm_ln_residual_after_norm(a, w, bias, r, gamma, beta, eps=1e-5):
    z = ops.matmul(ops.f64(a), ops.f64(w))
    u = ops.add_rowvec(z, ops.f64(bias))
    nrm = subgraphs.layernorm_rows(u, eps)
    if r is not None:
        nrm = ops.add(nrm, ops.f64(r))
    return ops.add_rowvec(ops.mul_rowvec(nrm, ops.f64(gamma)), ops.f64(beta))


def _gemm_softmax_scale_after(q, k, scale):
    p = ops.matmul(ops.f64(q), ops.transpose(ops.f64(k)))
    return ops.scale(subgraphs.softmax_rows(p), scale)


def _b2b_softmax_over_keys_axis0(q, k, v, scale):
    s = ops.scale(ops.matmul(ops.f64(q), ops.transpose(ops.f64(k))), scale)
    e = np.exp(s - s.max(axis=0)[None, :])
    return ops.matmul(e / e.sum(axis=0)[None, :], ops.f64(v))


def _b2b_unnormalized(q, k, v, scale):
    s = ops.scale(ops.matmul(ops.f64(q), ops.transpose(ops.f64(k))), scale)
    return ops.matmul(np.exp(s - s.max(axis=1)[:, None]), ops.f64(v))


def _rms_centered(x, gamma=None, eps=1e-5):
    x = ops.f64(x)
    c = ops.sub_colvec(x, ops.rowsum(x) / x.shape[1])
    y = ops.mul_colvec(c, ops.map_rsqrt_eps(ops.rowsum(ops.map_square(c)) / x.shape[1], eps))
    return y if gamma is None else ops.mul_rowvec(y, ops.f64(gamma))


def _ln_affine_beta_scaled(x, gamma, beta, eps=1e-5):
    n = subgraphs.layernorm_rows(x, eps)
    return ops.mul_rowvec(ops.add_rowvec(n, ops.f64(beta)), ops.f64(gamma))


def _pow_row_broadcast(x, v, p=1.5):
    x = ops.f64(x)
    pv = ops.map_pow(ops.f64(v), p)
    y = ops.add(x, np.resize(pv, x.shape[1])[None, :].repeat(x.shape[0], axis=0))
    return subgraphs.softmax_rows(y), y


MUTANTS = {
    # reductions
    "rowsum_drops_last": (ops, "rowsum", lambda x: np.sum(x[:, :-1], axis=1)),
    "rowsum_drops_first": (ops, "rowsum", lambda x: np.sum(x[:, 1:], axis=1)),
    "rowmax_is_min": (ops, "rowmax", lambda x: np.min(x, axis=1)),
    "rowmax_is_zero": (ops, "rowmax", lambda x: np.zeros(x.shape[0])),
    "rowmax_over_columns": (ops, "rowmax", lambda x: np.resize(np.max(x, axis=0), x.shape[0])),
    # broadcasts / binary ops
    "sub_colvec_sign": (ops, "sub_colvec", lambda x, c: x + c[:, None]),
    "div_is_mul": (ops, "div_colvec", lambda x, c: x * c[:, None]),
    "mul_colvec_dropped": (ops, "mul_colvec", lambda x, c: x),
    "add_colvec_dropped": (ops, "add_colvec", lambda x, c: x),
    "add_rowvec_dropped": (ops, "add_rowvec", lambda x, r: x),
    "add_rowvec_sign": (ops, "add_rowvec", lambda x, r: x - r[None, :]),
    "add_rowvec_reversed": (ops, "add_rowvec", lambda x, r: x + r[::-1][None, :]),
    "mul_rowvec_dropped": (ops, "mul_rowvec", lambda x, r: x),
    "add_dropped": (ops, "add", lambda x, y: x),
    # unary
    "exp_is_exp2": (ops, "map_exp", lambda x: np.exp2(x)),
    "square_is_abs": (ops, "map_square", lambda x: np.abs(x)),
    "pow_is_square": (ops, "map_pow", lambda x, p: np.power(x, 2.0)),
    "pow_is_sqrt": (ops, "map_pow", lambda x, p: np.sqrt(x)),
    "rsqrt_eps_outside": (ops, "map_rsqrt_eps", lambda x, e: 1.0 / (np.sqrt(x) + e)),
    "rsqrt_no_eps": (ops, "map_rsqrt_eps", lambda x, e: 1.0 / np.sqrt(x)),
    "rsqrt_is_inverse": (ops, "map_rsqrt_eps", lambda x, e: 1.0 / (x + e)),
    "scale_ignored": (ops, "scale", lambda x, a: x),
    # contraction
    "matmul_transposed_b": (ops, "matmul", lambda a, b: a @ b.T),
    "matmul_drops_last_k": (ops, "matmul", lambda a, b: a[:, :-1] @ b[:-1, :]),
    "transpose_missing": (ops, "transpose", lambda x: x),
    # whole-subgraph readings
    "ln_sample_variance": (subgraphs, "layernorm_rows", _ln_sample_variance),
    "ln_scales_uncentered": (subgraphs, "layernorm_rows", _ln_no_center_in_output),
    "gemm_ln_residual_after_norm": (subgraphs, "gemm_ln", _gemm_ln_residual_after_norm),
    "gemm_softmax_scale_after": (subgraphs, "gemm_softmax", _gemm_softmax_scale_after),
    "pow_row_broadcast": (subgraphs, "pow_bcast_add_softmax", _pow_row_broadcast),
    "b2b_softmax_over_wrong_axis": (subgraphs, "gemm_softmax_gemm", _b2b_softmax_over_keys_axis0),
    "b2b_unnormalized": (subgraphs, "gemm_softmax_gemm", _b2b_unnormalized),
    "rmsnorm_centers": (subgraphs, "rmsnorm_rows", _rms_centered),
    "gelu_erf_constant_dropped": (ops, "map_gelu_tanh", lambda x: 0.5 * x * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * x))),
    "silu_sign": (ops, "map_silu", lambda x: x / (1.0 + np.exp(x))),
    "gelu_erf_form": (ops, "map_gelu_tanh", lambda x: 0.5 * x * (1.0 + np.vectorize(math.erf)(x / np.sqrt(2.0)))),
    "gelu_cubic_0_0447": (ops, "map_gelu_tanh",
                          lambda x: 0.5 * x * (1.0 + np.tanh(np.sqrt(2.0 / np.pi) * (x + 0.0447 * x ** 3)))),
    "silu_sigmoid_2x": (ops, "map_silu", lambda x: x / (1.0 + np.exp(-2.0 * x))),
    "relu_is_abs": (ops, "map_relu", lambda x: np.abs(x)),
    "rsqrt_is_sqrt": (ops, "map_rsqrt", lambda x: np.sqrt(x)),
    "rsqrt_with_eps": (ops, "map_rsqrt", lambda x: 1.0 / np.sqrt(x + 1e-5)),
    "ln_affine_beta_scaled": (subgraphs, "layernorm_affine_rows", _ln_affine_beta_scaled),
    "graph_broadcast_axes_swapped": (graph, "_as_tile", _graph_as_tile_swapped),
    "graph_div_is_mul": (graph, "_BINARY", {"add": ops.add, "sub": ops.sub, "mul": ops.mul, "div": ops.mul}),
    "graph_sub_reversed": (graph, "_BINARY", {"add": ops.add, "sub": lambda x, y: y - x, "mul": ops.mul,
                                              "div": ops.div}),
    "graph_silu_is_relu": (graph, "_UNARY", {**graph._UNARY, "silu": "map_relu"}),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    mod, attr, fn = MUTANTS[name]
    monkeypatch.setattr(mod, attr, fn)
    if mod is subgraphs:
        monkeypatch.setattr(oracle, attr, fn)
    caught = []
    with np.errstate(all="ignore"):
        for pin in pins.ALL_PINS:
            try:
                pin()
            except Exception as e:  # noqa: BLE001 - any failure is a catch
                caught.append((pin.__name__, type(e).__name__))
    assert caught, f"mutant {name} survived every pin"


@pytest.mark.parametrize("name", ["gelu_erf_form", "gelu_cubic_0_0447", "silu_sigmoid_2x",
                                  "gelu_erf_constant_dropped", "silu_sign"])
def test_activation_mutant_is_caught_by_an_independent_pin(name, monkeypatch):
    """Each plausible activation mistake is caught by a pin other than the GEMM + activation brute
    force (whose per-element activation restates the oracle's formula)."""
    mod, attr, fn = MUTANTS[name]
    monkeypatch.setattr(mod, attr, fn)
    caught = []
    with np.errstate(all="ignore"):
        for pin in pins.ALL_PINS:
            if pin.__name__ == "pin_gemm_act_brute_force":
                continue
            try:
                pin()
            except Exception:  # noqa: BLE001 - any failure is a catch
                caught.append(pin.__name__)
    assert caught, f"mutant {name} is caught only by the brute force"
