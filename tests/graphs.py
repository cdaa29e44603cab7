"""Captured graphs of the library's stage DAGs as plain node tuples (op, in0, in1, attr, slot, value).

Shared by the oracle's graph pins (CPU) and the Fusion Spec IR tests, which
hand the same tuples to the product's binding and to oracle.graph.evaluate.
Slots: stitched graphs x=0 (gamma=1, beta=2 or v=1); GEMM graphs A=0, W=1,
bias=2, R=3, gamma=4, beta=5.
"""


class B:
    def __init__(self):
        self.nodes = []

    def add(self, op, a=-1, b=-1, attr=0, slot=-1, value=0.0):
        self.nodes.append((op, a, b, attr, slot, float(value)))
        return len(self.nodes) - 1

    def ph(self, op, slot):
        return self.add(op, slot=slot)

    def c(self, value):
        return self.add("const", value=value)


def softmax_chain(b, t):
    m = b.add("rowmax", t)
    e = b.add("exp", b.add("sub", t, m))
    return b.add("div", e, b.add("rowsum", e))


def layernorm_chain(b, u, cols, eps, affine=False, commuted=False, g=1, bt=2):
    mu = b.add("div", b.add("rowsum", u), b.c(cols))
    c = b.add("sub", u, mu)
    var = b.add("div", b.add("rowsum", b.add("square", c)), b.c(cols))
    ve = b.add("add", b.c(eps), var) if commuted else b.add("add", var, b.c(eps))
    r = b.add("rsqrt", ve)
    y = b.add("mul", r, c) if commuted else b.add("mul", c, r)
    if affine:
        gm = b.ph("rowvec", g)
        y = b.add("mul", gm, y) if commuted else b.add("mul", y, gm)
        be = b.ph("rowvec", bt)
        y = b.add("add", be, y) if commuted else b.add("add", y, be)
    return y


def softmax():
    b = B()
    return b.nodes, softmax_chain(b, b.ph("input", 0))


def layernorm(cols, eps=1e-5, affine=False, commuted=False):
    b = B()
    return b.nodes, layernorm_chain(b, b.ph("input", 0), cols, eps, affine, commuted)


def rmsnorm(cols, eps=1e-5, gain=False, commuted=False):
    b = B()
    x = b.ph("input", 0)
    ms = b.add("div", b.add("rowsum", b.add("square", x)), b.c(cols))
    r = b.add("rsqrt", b.add("add", ms, b.c(eps)))
    y = b.add("mul", r, x) if commuted else b.add("mul", x, r)
    if gain:
        y = b.add("mul", y, b.ph("rowvec", 1))
    return b.nodes, y


def pow_softmax(p=1.5, commuted=False):
    b = B()
    x = b.ph("input", 0)
    pv = b.add("pow", b.ph("colvec", 1), b.c(p))
    t = b.add("add", pv, x) if commuted else b.add("add", x, pv)
    return b.nodes, softmax_chain(b, t)


def gemm_ln(cols, eps=1e-5, residual=True, commuted=False):
    b = B()
    acc = b.add("matmul", b.ph("operand", 0), b.ph("operand", 1))
    u = b.add("add", b.ph("rowvec", 2), acc) if commuted else b.add("add", acc, b.ph("rowvec", 2))
    if residual:
        u = b.add("add", u, b.ph("tensor", 3))
    return b.nodes, layernorm_chain(b, u, cols, eps, True, commuted, g=4, bt=5)


def gemm_softmax(scale, commuted=False):
    b = B()
    acc = b.add("matmul", b.ph("operand", 0), b.ph("operand", 1), attr=1)
    t = b.add("mul", b.c(scale), acc) if commuted else b.add("mul", acc, b.c(scale))
    return b.nodes, softmax_chain(b, t)


def gemm_act(act, bias=True, commuted=False):
    b = B()
    u = b.add("matmul", b.ph("operand", 0), b.ph("operand", 1))
    if bias:
        u = b.add("add", b.ph("rowvec", 2), u) if commuted else b.add("add", u, b.ph("rowvec", 2))
    if act != "none":
        u = b.add(act, u)
    return b.nodes, u


# Graphs outside the library's stage DAGs (for the automatic stitcher).

def silu_ln_scaled(cols):
    """y = LayerNorm(silu(x) + b) * v_i, b a row vector (slot 1), v a per-row vector (slot 2)."""
    b = B()
    x = b.ph("input", 0)
    u = b.add("add", b.add("silu", x), b.ph("rowvec", 1))
    y = layernorm_chain(b, u, cols, 1e-5)
    return b.nodes, b.add("mul", y, b.ph("colvec", 2))


def softmax_temperature():
    """softmax(x * t_i), t a per-row temperature (slot 1)."""
    b = B()
    return b.nodes, softmax_chain(b, b.add("mul", b.ph("input", 0), b.ph("colvec", 1)))


def residual_ln(cols):
    """LayerNorm(x + r) * gamma + beta with two fp32 inputs: x (0), r (1); gamma (2), beta (3)."""
    b = B()
    u = b.add("add", b.ph("input", 0), b.ph("input", 1))
    return b.nodes, layernorm_chain(b, u, cols, 1e-5, True, g=2, bt=3)


def gelu_centered():
    """gelu(x) - rowmax(gelu(x)) + v_i^2 / 3 (v slot 1)."""
    b = B()
    gx = b.add("gelu_tanh", b.ph("input", 0))
    d = b.add("sub", gx, b.add("rowmax", gx))
    pv = b.add("div", b.add("pow", b.ph("colvec", 1), b.c(2.0)), b.c(3.0))
    return b.nodes, b.add("add", d, pv)


def rms_relu(cols):
    """relu(RMSNorm(x) * g) with g a row vector (slot 1)."""
    b = B()
    x = b.ph("input", 0)
    ms = b.add("div", b.add("rowsum", b.add("square", x)), b.c(cols))
    y = b.add("mul", b.add("mul", x, b.add("rsqrt", b.add("add", ms, b.c(1e-6)))), b.ph("rowvec", 1))
    return b.nodes, b.add("relu", y)
