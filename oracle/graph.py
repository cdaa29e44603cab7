"""A captured graph evaluated node by node in float64: the meaning a Fusion Spec IR must keep.

TEST INFRASTRUCTURE ONLY (see the package docstring).

ComFuse, Frontend / Fusion Spec IR: the graph G_epi that Phi lowers is a
list of operators with their data dependencies; Phi's closure property says
any graph it accepts keeps its semantics.  This module is that semantics
written out, independently of any lowering: each node is evaluated in order
from its inputs' values, with the broadcasts the Phi patterns name spelled
out (a constant is a scalar broadcast, a length-cols placeholder a
row-vector broadcast, a per-row value a column broadcast), so a lowered and
launched graph can be checked against it.

Nodes are tuples (op, in0, in1, attr, slot, value) with op a name:
  input, operand, tensor  2-D placeholders (args[slot])
  rowvec                  length-cols placeholder; colvec: one value per row
  const                   scalar `value`
  matmul                  in0 . in1 (attr 1: in0 . in1^T)
  add sub mul div pow     binary; exp square rsqrt relu gelu_tanh silu: unary
  rowsum rowmax           reductions over the row
"""
from __future__ import annotations

import numpy as np

from . import ops

_UNARY = {"exp": "map_exp", "square": "map_square", "rsqrt": "map_rsqrt", "relu": "map_relu",
          "gelu_tanh": "map_gelu_tanh", "silu": "map_silu"}
_BINARY = {"add": ops.add, "sub": ops.sub, "mul": ops.mul, "div": ops.div}


def _as_tile(kind, v, rows, cols):
    """The value as a [rows x cols] tile through the broadcast its kind calls for."""
    if kind == "tile":
        return v
    if kind == "row":
        return ops.bcast_col(v, cols)
    if kind == "vec":
        return ops.bcast_row(v, rows)
    return np.full((rows, cols), v)


def evaluate(nodes, terminal, args) -> np.ndarray:
    """Value of node `terminal`; args[slot] are the placeholders' stored values."""
    vals = []
    for (op, a, b, attr, slot, value) in nodes:
        if op in ("input", "operand", "tensor"):
            v = ("tile", ops.f64(args[slot]))
        elif op == "rowvec":
            v = ("vec", ops.f64(args[slot]))
        elif op == "colvec":
            v = ("row", ops.f64(args[slot]))
        elif op == "const":
            v = ("scalar", np.float64(value))
        elif op == "matmul":
            left, right = vals[a][1], vals[b][1]
            v = ("tile", ops.matmul(left, ops.transpose(right) if attr == 1 else right))
        elif op in _UNARY:
            kind, x = vals[a]
            v = (kind, getattr(ops, _UNARY[op])(x))
        elif op in ("rowsum", "rowmax"):
            kind, x = vals[a]
            assert kind == "tile"
            v = ("row", ops.rowsum(x) if op == "rowsum" else ops.rowmax(x))
        elif op == "pow":
            kind, x = vals[a]
            assert vals[b][0] == "scalar"
            v = (kind, ops.map_pow(x, float(vals[b][1])))
        else:
            (ka, xa), (kb, xb) = vals[a], vals[b]
            if "tile" in (ka, kb):
                rows, cols = (xa if ka == "tile" else xb).shape
                v = ("tile", _BINARY[op](_as_tile(ka, xa, rows, cols), _as_tile(kb, xb, rows, cols)))
            else:
                # per-row values with a per-row value or a constant
                n = xa.shape[0] if ka == "row" else xb.shape[0]
                xa = xa if ka == "row" else np.full(n, xa)
                xb = xb if kb == "row" else np.full(n, xb)
                v = ("row", _BINARY[op](xa, xb))
        vals.append(v)
    kind, out = vals[terminal]
    assert kind == "tile"
    return np.asarray(out)
