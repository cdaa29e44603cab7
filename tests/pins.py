"""Pins that tie the fp64 oracle to something other than itself.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with a
closed form, an invariant, a library routine or a brute-force evaluation on a
tiny input.  ``tests/test_oracle_pins.py`` runs them; ``tests/test_oracle_mutants.py``
plants plausible mistakes in the oracle (on the CPU) and checks that at least
one pin fails for every mistake.

The pages print no worked numerical example for these subgraphs, so no pin
compares against a printed value; the closed-form values used here are
derived in ``tests/golden/closed_forms.json``.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, rtol, atol=0.0, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = np.abs(a - b)
    bound = atol + rtol * np.abs(b)
    assert np.all(err <= bound), f"{what}: max err {err.max():.3e}"


# ----------------------------------------------------------------- brute force

def _bf_softmax(rows):
    """Direct definition exp(x_j) / sum_k exp(x_k), pure Python, no max shift."""
    out = []
    for row in rows:
        e = [math.exp(v) for v in row]
        s = math.fsum(e)
        out.append([v / s for v in e])
    return out


def _bf_layernorm(rows, eps):
    out = []
    for row in rows:
        n = len(row)
        mean = math.fsum(row) / n
        var = math.fsum((v - mean) ** 2 for v in row) / n
        out.append([(v - mean) / math.sqrt(var + eps) for v in row])
    return out


def _bf_matmul(a, b):
    m, k = len(a), len(a[0])
    n = len(b[0])
    return [[math.fsum(a[i][t] * b[t][j] for t in range(k)) for j in range(n)] for i in range(m)]


# --------------------------------------------------------------------- softmax

def pin_softmax_rows_sum_to_one():
    for shape in [(7, 13), (5, 1000), (3, 1)]:
        x = _rng(11).normal(size=shape) * 3.0
        y = oracle.softmax_rows(x)
        assert np.all(y > 0.0) and np.all(y <= 1.0), "softmax outside (0, 1]"
        assert np.max(np.abs(1.0 - y.sum(axis=1))) <= 1e-12, "softmax rows do not sum to 1"


def pin_softmax_constant_row():
    for n in [1, 7, 1024, 30000]:
        x = np.full((3, n), -2.75)
        y = oracle.softmax_rows(x)
        assert np.array_equal(y, np.full((3, n), 1.0 / n)), f"constant row n={n} is not 1/n"


def pin_softmax_one_hot():
    g = _golden()["softmax_one_hot"]
    n, t = g["n"], g["t"]
    x = np.zeros((n, n))
    for i in range(n):          # the hot entry moves along the diagonal: pins indexing
        x[i, i] = t
    y = oracle.softmax_rows(x)
    hot = 1.0 / (1.0 + (n - 1) * math.exp(-t))
    cold = math.exp(-t) * hot
    _close(np.diag(y), np.full(n, hot), 1e-14, what="one-hot hot entry")
    _close(y[~np.eye(n, dtype=bool)], np.full(n * (n - 1), cold), 1e-14, what="one-hot cold entries")
    _close([hot, cold], [g["hot"], g["cold"]], 1e-12, what="one-hot golden")


def pin_softmax_shift_invariance():
    x = _rng(12).normal(size=(9, 77))
    c = _rng(13).uniform(-50, 50, size=(9, 1))
    _close(oracle.softmax_rows(x + c), oracle.softmax_rows(x), 0.0, 1e-13, what="shift invariance")


def pin_softmax_brute_force():
    for n in range(1, 9):
        x = _rng(100 + n).normal(size=(3, n)) * 2.0
        _close(oracle.softmax_rows(x), _bf_softmax(x.tolist()), 1e-14, what=f"softmax brute n={n}")


def pin_softmax_large_inputs():
    """Entries near 1000 overflow exp unless the row maximum is subtracted first."""
    x = np.array([[1000.0, 999.0, 998.0], [1000.0, 0.0, -1000.0], [-1000.0, -1001.0, -999.0]])
    y = oracle.softmax_rows(x)
    d = np.array([[0.0, -1.0, -2.0], [0.0, -1000.0, -2000.0], [-1.0, -2.0, 0.0]])
    expect = [[math.exp(v) / math.fsum(math.exp(w) for w in row) for v in row] for row in d.tolist()]
    _close(y, expect, 1e-14, what="large-magnitude softmax")


# ------------------------------------------------------------------- LayerNorm

def pin_layernorm_invariants():
    eps = 1e-5
    for shape in [(5, 37), (4, 32), (3, 4096)]:
        x = _rng(21).uniform(-1, 1, size=shape)
        y = oracle.layernorm_rows(x, eps)
        var = np.var(x, axis=1)                     # library routine, ddof=0
        assert np.max(np.abs(y.mean(axis=1))) <= 1e-12, "LN mean is not 0"
        _close((y * y).mean(axis=1), var / (var + eps), 1e-12, what="LN mean of squares")


def pin_layernorm_constant_row():
    for val in [0.5, 3.0, -7.25]:
        x = np.full((2, 32), val)
        assert np.array_equal(oracle.layernorm_rows(x, 1e-5), np.zeros((2, 32))), "constant row is not 0"


def pin_layernorm_alternating():
    eps = 1e-5
    for a in [1e-3, 1.0, 7.0]:
        row = np.array([a if j % 2 == 0 else -a for j in range(32)])
        y = oracle.layernorm_rows(row[None, :], eps)
        _close(y[0], row / math.sqrt(a * a + eps), 1e-14, what=f"alternating a={a}")
    g = _golden()["layernorm_alternating"]
    y = oracle.layernorm_rows(np.array([[g["a"], -g["a"]] * 4]), g["eps"])
    _close(y[0], [g["value"], -g["value"]] * 4, 1e-14, what="alternating golden")


def pin_layernorm_numpy():
    eps = 1e-5
    x = _rng(22).normal(size=(6, 129))
    ref = (x - x.mean(axis=1, keepdims=True)) / np.sqrt(x.var(axis=1, keepdims=True) + eps)
    _close(oracle.layernorm_rows(x, eps), ref, 1e-12, 1e-14, what="LN vs numpy mean/var")


def pin_layernorm_brute_force():
    eps = 1e-5
    for shape in [(3, 5), (2, 2), (4, 9)]:
        x = _rng(23).normal(size=shape)
        _close(oracle.layernorm_rows(x, eps), _bf_layernorm(x.tolist(), eps), 1e-13, 1e-15,
               what=f"LN brute {shape}")


# ---------------------------------------------------------- pow-broadcast-add

def pin_pow_closed_forms():
    g = _golden()["pow_1_5"]
    v = np.array(g["v"])
    x = np.zeros((len(v), 3))
    _, y = oracle.pow_bcast_add_softmax(x, v, 1.5)
    _close(y, np.repeat(np.array(g["v_pow_1_5"])[:, None], 3, axis=1), 1e-15, what="v^1.5 closed forms")


def pin_pow_brute_force():
    for shape in [(3, 5), (7, 9)]:
        x = _rng(31).normal(size=shape)
        v = _rng(32).uniform(0.1, 2.0, size=shape[0])
        out, y = oracle.pow_bcast_add_softmax(x, v, 1.5)
        yb = [[x[i, j] + math.pow(v[i], 1.5) for j in range(shape[1])] for i in range(shape[0])]
        _close(y, yb, 1e-15, 1e-15, what=f"pow-bcast-add brute {shape}")
        _close(out, _bf_softmax(yb), 1e-14, what=f"softmax of Y brute {shape}")


def pin_pow_softmax_identity():
    """softmax(X + c_i) = softmax(X): the power stage cannot change the final output."""
    x = _rng(33).normal(size=(8, 300))
    v = _rng(34).uniform(0.1, 2.0, size=8)
    out, _ = oracle.pow_bcast_add_softmax(x, v, 1.5)
    _close(out, oracle.softmax_rows(x), 0.0, 1e-13, what="pow identity")


# ------------------------------------------------------------------- GEMMs

def pin_gemm_ones():
    for (m, n, k) in [(4, 6, 5), (3, 3, 1024)]:
        a, w = np.ones((m, k)), np.ones((k, n))
        bias, r = np.zeros(n), np.zeros((m, n))
        gamma = _rng(41).uniform(0.5, 1.5, size=n)
        beta = _rng(42).normal(size=n)
        y = oracle.gemm_ln(a, w, bias, r, gamma, beta, 1e-5)
        assert np.array_equal(y, np.repeat(beta[None, :], m, axis=0)), "ones GEMM+LN is not beta"
        s = oracle.gemm_softmax(np.ones((m, k)), np.ones((n, k)), 0.125)
        assert np.array_equal(s, np.full((m, n), 1.0 / n)), "ones GEMM+softmax is not 1/N"


def pin_gemm_softmax_zero_q():
    q, k = np.zeros((5, 16)), _rng(43).normal(size=(64, 16))
    assert np.array_equal(oracle.gemm_softmax(q, k, 0.25), np.full((5, 64), 1.0 / 64)), "Q=0 is not 1/N"


def pin_gemm_ln_brute_force():
    eps = 1e-5
    for (m, n, k) in [(3, 6, 4), (5, 5, 5), (2, 7, 3)]:
        rng = _rng(44 + m)
        a, w = rng.normal(size=(m, k)), rng.normal(size=(k, n))
        bias, gamma, beta = rng.normal(size=n), 1 + 0.1 * rng.normal(size=n), rng.normal(size=n)
        r = rng.normal(size=(m, n))
        z = _bf_matmul(a.tolist(), w.tolist())
        u = [[z[i][j] + bias[j] + r[i, j] for j in range(n)] for i in range(m)]
        nrm = _bf_layernorm(u, eps)
        yb = [[nrm[i][j] * gamma[j] + beta[j] for j in range(n)] for i in range(m)]
        _close(oracle.gemm_ln(a, w, bias, r, gamma, beta, eps), yb, 1e-12, 1e-13, what=f"GEMM+LN brute {m,n,k}")
        # without residual
        u0 = [[z[i][j] + bias[j] for j in range(n)] for i in range(m)]
        n0 = _bf_layernorm(u0, eps)
        y0 = [[n0[i][j] * gamma[j] + beta[j] for j in range(n)] for i in range(m)]
        _close(oracle.gemm_ln(a, w, bias, None, gamma, beta, eps), y0, 1e-12, 1e-13, what="GEMM+LN brute no R")


def pin_gemm_softmax_brute_force():
    for (m, n, d) in [(3, 5, 4), (4, 4, 4), (6, 2, 7)]:
        rng = _rng(50 + m)
        q, k = rng.normal(size=(m, d)), rng.normal(size=(n, d))
        sc = 1.0 / math.sqrt(d)
        kt = [[k[j, t] for j in range(n)] for t in range(d)]
        p = _bf_matmul(q.tolist(), kt)
        yb = _bf_softmax([[sc * v for v in row] for row in p])
        _close(oracle.gemm_softmax(q, k, sc), yb, 1e-13, what=f"GEMM+softmax brute {m,n,d}")


# -------------------------------------------------- back-to-back GEMM (softmax between)

def pin_b2b_brute_force():
    """O_ij = sum_n softmax_n(scale * q_i . k_n) v_nj, every sum written out in pure Python."""
    for (m, n, d, dv) in [(3, 5, 4, 2), (4, 4, 4, 4), (2, 7, 3, 5)]:
        rng = _rng(60 + m + n)
        q, k, v = rng.normal(size=(m, d)), rng.normal(size=(n, d)), rng.normal(size=(n, dv))
        sc = 1.0 / math.sqrt(d)
        kt = [[k[j, t] for j in range(n)] for t in range(d)]
        p = _bf_matmul(q.tolist(), kt)
        sm = _bf_softmax([[sc * x for x in row] for row in p])
        ob = _bf_matmul(sm, v.tolist())
        _close(oracle.gemm_softmax_gemm(q, k, v, sc), ob, 1e-12, 1e-14, what=f"B2B brute {m,n,d,dv}")


def pin_b2b_ones_v():
    """Every softmax row sums to one, so a V of ones gives an output of ones."""
    rng = _rng(64)
    q, k = rng.normal(size=(6, 16)), rng.normal(size=(40, 16))
    o = oracle.gemm_softmax_gemm(q, k, np.ones((40, 3)), 0.25)
    _close(o, np.ones((6, 3)), 0.0, 1e-14, what="B2B ones V")


def pin_b2b_zero_q():
    """Q = 0 makes every score equal: each output row is the column mean of V."""
    rng = _rng(65)
    k, v = rng.normal(size=(30, 8)), rng.normal(size=(30, 5))
    o = oracle.gemm_softmax_gemm(np.zeros((4, 8)), k, v, 0.5)
    _close(o, np.repeat(v.mean(axis=0)[None, :], 4, axis=0), 1e-13, 1e-15, what="B2B zero Q")


def pin_b2b_key_permutation():
    """Reordering the keys (rows of K and V together) leaves the output unchanged."""
    rng = _rng(66)
    q, k, v = rng.normal(size=(5, 12)), rng.normal(size=(33, 12)), rng.normal(size=(33, 7))
    perm = rng.permutation(33)
    _close(oracle.gemm_softmax_gemm(q, k[perm], v[perm], 0.3), oracle.gemm_softmax_gemm(q, k, v, 0.3),
           1e-12, 1e-14, what="B2B key permutation")


def pin_b2b_one_hot():
    """Orthogonal keys and a large scale: each row's softmax is one-hot, so the row copies one row of V."""
    n = 8
    k = np.eye(n)
    q = np.eye(n)[[3, 0, 7, 5]]
    v = _rng(67).normal(size=(n, 4))
    o = oracle.gemm_softmax_gemm(q, k, v, 100.0)
    _close(o, v[[3, 0, 7, 5]], 1e-12, 1e-12, what="B2B one-hot")


# ------------------------------------------------------- RMSNorm, affine LayerNorm

def _bf_rmsnorm(rows, eps, gamma=None):
    out = []
    for row in rows:
        n = len(row)
        ms = math.fsum(v * v for v in row) / n
        r = 1.0 / math.sqrt(ms + eps)
        out.append([v * r * (gamma[j] if gamma is not None else 1.0) for j, v in enumerate(row)])
    return out


def pin_rmsnorm_brute_force():
    for (m, n) in [(3, 5), (2, 32), (4, 1)]:
        rng = _rng(70 + n)
        x, g = rng.normal(size=(m, n)), 1.0 + 0.1 * rng.normal(size=n)
        _close(oracle.rmsnorm_rows(x, g, 1e-5), _bf_rmsnorm(x.tolist(), 1e-5, g.tolist()), 1e-13, 1e-15,
               what=f"RMSNorm brute {m,n}")
        _close(oracle.rmsnorm_rows(x, None, 1e-5), _bf_rmsnorm(x.tolist(), 1e-5), 1e-13, 1e-15,
               what=f"RMSNorm brute no gain {m,n}")


def pin_rmsnorm_closed_forms():
    """Constant row c: y = c / sqrt(c^2 + eps).  Any row: mean(y^2) = ms / (ms + eps) (no gain).
    A row and its negation map to negated outputs (no centering)."""
    c, eps = 0.75, 1e-5
    y = oracle.rmsnorm_rows(np.full((2, 16), c), None, eps)
    _close(y, np.full((2, 16), c / math.sqrt(c * c + eps)), 1e-15, what="RMSNorm constant row")
    x = _rng(72).uniform(-1, 1, size=(6, 32))
    ms = np.mean(x * x, axis=1)
    _close(np.mean(oracle.rmsnorm_rows(x, None, eps) ** 2, axis=1), ms / (ms + eps), 1e-13, what="RMSNorm mean square")
    _close(oracle.rmsnorm_rows(-x, None, eps), -oracle.rmsnorm_rows(x, None, eps), 0.0, 0.0, what="RMSNorm odd")


def pin_layernorm_affine_brute_force():
    for (m, n) in [(3, 6), (2, 32)]:
        rng = _rng(74 + n)
        x, g, b = rng.normal(size=(m, n)), 1.0 + 0.1 * rng.normal(size=n), 0.1 * rng.normal(size=n)
        nrm = _bf_layernorm(x.tolist(), 1e-5)
        yb = [[nrm[i][j] * g[j] + b[j] for j in range(n)] for i in range(m)]
        _close(oracle.layernorm_affine_rows(x, g, b, 1e-5), yb, 1e-13, 1e-15, what=f"affine LN brute {m,n}")


def pin_layernorm_affine_constant_row():
    """A constant row normalises to 0, so the output is beta."""
    b = _rng(76).normal(size=12)
    y = oracle.layernorm_affine_rows(np.full((3, 12), -2.5), _rng(77).normal(size=12), b, 1e-5)
    assert np.array_equal(y, np.repeat(b[None, :], 3, axis=0)), "affine LN constant row is not beta"


# ------------------------------------------------------- GEMM + activation

def _bf_act(v, act):
    if act == "none":
        return v
    if act == "relu":
        return v if v > 0 else 0.0
    if act == "gelu_tanh":
        return 0.5 * v * (1.0 + math.tanh(math.sqrt(2.0 / math.pi) * (v + 0.044715 * v ** 3)))
    if act == "silu":
        return v / (1.0 + math.exp(-v))
    if act == "rsqrt":
        return 1.0 / math.sqrt(v)
    return v * v


def pin_gemm_act_brute_force():
    for act in ["none", "relu", "gelu_tanh", "silu", "square"]:
        for (m, n, k) in [(3, 5, 4), (2, 7, 3)]:
            rng = _rng(80 + m + n)
            a, w, b = rng.normal(size=(m, k)), rng.normal(size=(k, n)), rng.normal(size=n)
            z = _bf_matmul(a.tolist(), w.tolist())
            yb = [[_bf_act(z[i][j] + b[j], act) for j in range(n)] for i in range(m)]
            _close(oracle.gemm_act(a, w, b, act), yb, 1e-13, 1e-14, what=f"GEMM+{act} brute {m,n,k}")
            y0 = [[_bf_act(z[i][j], act) for j in range(n)] for i in range(m)]
            _close(oracle.gemm_act(a, w, None, act), y0, 1e-13, 1e-14, what=f"GEMM+{act} brute no bias")


def pin_gemm_act_closed_forms():
    """Values the definitions fix: GELU and SiLU of 0 are 0 and tend to x for large x and to 0
    for large negative x; SiLU(x) - SiLU(-x) = x; ReLU(x) - ReLU(-x) = x; square of a ones GEMM is K^2."""
    x = np.array([[0.0, 30.0, -30.0, 1.5]])
    eye = np.eye(4)
    g = oracle.gemm_act(x, eye, None, "gelu_tanh")
    _close(g, [[0.0, 30.0, 0.0, g[0, 3]]], 0.0, 1e-12, what="GELU limits")
    s = oracle.gemm_act(x, eye, None, "silu")
    _close(s[0, :3], [0.0, 30.0, 0.0], 0.0, 1e-11, what="SiLU limits")
    v = _rng(82).normal(size=(3, 6))
    for act in ["silu", "relu"]:
        d = oracle.gemm_act(v, np.eye(6), None, act) - oracle.gemm_act(-v, np.eye(6), None, act)
        _close(d, v, 1e-14, 1e-15, what=f"{act} odd part")
    _close(oracle.gemm_act(np.ones((2, 9)), np.ones((9, 3)), None, "square"), np.full((2, 3), 81.0), 0.0, 0.0,
           what="square of ones")


def pin_activation_values():
    """GELU (tanh form) and SiLU at the points the golden file derives by hand in 50-digit decimal
    arithmetic (a route that shares nothing with the oracle's float64 formula), reached through
    the activation GEMM with an identity weight, so the values pass the epilogue unchanged."""
    gd = _golden()
    for key, act in (("gelu_tanh_values", "gelu_tanh"), ("silu_values", "silu")):
        x = np.array([gd[key]["x"]])
        y = oracle.gemm_act(x, np.eye(x.shape[1]), None, act)
        _close(y, [gd[key]["y"]], 1e-15, 1e-15, what=f"{act} at golden points")


def pin_gemm_act_rsqrt():
    """rsqrt epilogue: brute force on positive operands (every u > 0), and closed forms:
    a ones GEMM with K = 9 gives 1/3, with K = 4 exactly 0.5; a diagonal GEMM gives 1/sqrt of
    each entry (0.25 -> 2, 16 -> 0.25)."""
    for (m, n, k) in [(3, 5, 4), (2, 7, 3)]:
        rng = _rng(90 + m + n)
        a, w, b = rng.uniform(0.5, 1.5, (m, k)), rng.uniform(0.1, 1.0, (k, n)), rng.uniform(0.0, 1.0, n)
        z = _bf_matmul(a.tolist(), w.tolist())
        yb = [[_bf_act(z[i][j] + b[j], "rsqrt") for j in range(n)] for i in range(m)]
        _close(oracle.gemm_act(a, w, b, "rsqrt"), yb, 1e-13, 1e-14, what=f"GEMM+rsqrt brute {m,n,k}")
    _close(oracle.gemm_act(np.ones((2, 9)), np.ones((9, 3)), None, "rsqrt"), np.full((2, 3), 1.0 / 3.0), 0.0,
           0.0, what="rsqrt of a ones GEMM, K = 9")
    _close(oracle.gemm_act(np.ones((1, 4)), np.ones((4, 2)), np.zeros(2), "rsqrt"), [[0.5, 0.5]], 0.0, 0.0,
           what="rsqrt of a ones GEMM, K = 4")
    _close(oracle.gemm_act(np.array([[0.25, 16.0]]), np.eye(2), None, "rsqrt"), [[2.0, 0.25]], 0.0, 0.0,
           what="rsqrt of a diagonal GEMM")


def pin_graph_families_match_subgraphs():
    """The captured graph of every stage DAG, evaluated node by node, gives the subgraph oracle's
    values, with operands of add and mul in either order."""
    from oracle import graph
    from tests import graphs
    rng = _rng(100)
    rows, cols, k = 5, 12, 7
    x = rng.normal(size=(rows, cols))
    g, bt = 1.0 + 0.1 * rng.normal(size=cols), 0.1 * rng.normal(size=cols)
    v = rng.uniform(0.1, 2.0, rows)
    a, w, bias, r = rng.normal(size=(rows, k)), rng.normal(size=(k, cols)), rng.normal(size=cols), \
        rng.normal(size=(rows, cols))
    kk = rng.normal(size=(cols, k))
    ap, wp, bp = np.abs(a) + 0.5, np.abs(w), np.abs(bias)
    for cm in (False, True):
        cases = [
            (graphs.softmax(), [x], oracle.softmax_rows(x)),
            (graphs.layernorm(cols, 1e-5, False, cm), [x], oracle.layernorm_rows(x, 1e-5)),
            (graphs.layernorm(cols, 1e-5, True, cm), [x, g, bt], oracle.layernorm_affine_rows(x, g, bt, 1e-5)),
            (graphs.rmsnorm(cols, 1e-5, False, cm), [x], oracle.rmsnorm_rows(x, None, 1e-5)),
            (graphs.rmsnorm(cols, 1e-5, True, cm), [x, g], oracle.rmsnorm_rows(x, g, 1e-5)),
            (graphs.pow_softmax(1.5, cm), [x, v], oracle.pow_bcast_add_softmax(x, v, 1.5)[0]),
            (graphs.gemm_ln(cols, 1e-5, True, cm), [a, w, bias, r, g, bt], oracle.gemm_ln(a, w, bias, r, g, bt, 1e-5)),
            (graphs.gemm_ln(cols, 1e-5, False, cm), [a, w, bias, None, g, bt],
             oracle.gemm_ln(a, w, bias, None, g, bt, 1e-5)),
            (graphs.gemm_softmax(0.3, cm), [a, kk], oracle.gemm_softmax(a, kk, 0.3)),
        ]
        for act in oracle.ACTIVATIONS:
            aa, ww, bb = (ap, wp, bp) if act == "rsqrt" else (a, w, bias)
            cases.append((graphs.gemm_act(act, True, cm), [aa, ww, bb], oracle.gemm_act(aa, ww, bb, act)))
            cases.append((graphs.gemm_act(act, False, cm), [aa, ww], oracle.gemm_act(aa, ww, None, act)))
        for (nodes, t), args, want in cases:
            _close(graph.evaluate(nodes, t, args), want, 1e-12, 1e-14, what=f"graph of {nodes[t][0]} (commuted={cm})")


def pin_graph_brute_force():
    """A graph outside the stage DAGs, every broadcast kind and a per-row computation, against loops:
    y_ij = (x_ij - v_i) * r_j / 2 + 3 max_l x_il;  z_ij = sum_l a_il b_jl (the transposed MatMul)."""
    from oracle import graph
    rng = _rng(101)
    x, v, r = rng.normal(size=(4, 6)), rng.normal(size=4), rng.normal(size=6)
    nodes = [("input", -1, -1, 0, 0, 0.0), ("colvec", -1, -1, 0, 1, 0.0), ("rowvec", -1, -1, 0, 2, 0.0),
             ("const", -1, -1, 0, -1, 2.0), ("sub", 0, 1, 0, -1, 0.0), ("mul", 4, 2, 0, -1, 0.0),
             ("div", 5, 3, 0, -1, 0.0), ("rowmax", 0, -1, 0, -1, 0.0), ("const", -1, -1, 0, -1, 3.0),
             ("mul", 7, 8, 0, -1, 0.0), ("add", 6, 9, 0, -1, 0.0)]
    xs, vs, rs = x.tolist(), v.tolist(), r.tolist()
    want = [[(xs[i][j] - vs[i]) * rs[j] / 2.0 + 3.0 * max(xs[i]) for j in range(6)] for i in range(4)]
    _close(graph.evaluate(nodes, 10, [x, v, r]), want, 1e-14, 1e-15, what="graph brute force")
    a, b = rng.normal(size=(3, 5)), rng.normal(size=(4, 5))
    nodes = [("operand", -1, -1, 0, 0, 0.0), ("operand", -1, -1, 0, 1, 0.0), ("matmul", 0, 1, 1, -1, 0.0)]
    want = [[math.fsum(a[i, l] * b[j, l] for l in range(5)) for j in range(4)] for i in range(3)]
    _close(graph.evaluate(nodes, 2, [a, b]), want, 1e-13, 1e-15, what="graph transposed MatMul")


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
