"""fp64 CPU oracle for the stitched and GEMM-fused subgraphs.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check in
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call anything in this package.  The library under
``broadcast_subgraphs_amd`` never does, and shares no code with it.

The oracle is the plain definition of each subgraph, evaluated one operator
at a time in float64: every operator is a whole-array function that
materializes its result, and the operators are composed in the order the
subgraph lists them.  Inputs are the exact stored fp32/bf16 values widened to
float64.  No blocking, fusion, online merging or reordering is done here; the
stitched kernels reach the same values (up to rounding) by a faster route.

Parity status: every function is pinned by closed forms, invariants, library
routines or brute force in ``tests/test_oracle_pins.py``; none is unpinned.
"""
from . import graph, ops  # noqa: F401
from .subgraphs import (  # noqa: F401
    ACTIVATIONS,
    gemm_act,
    gemm_ln,
    gemm_softmax,
    gemm_softmax_gemm,
    layernorm_affine_rows,
    layernorm_rows,
    pow_bcast_add_softmax,
    rmsnorm_rows,
    softmax_rows,
)
