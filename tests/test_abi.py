"""C-ABI checks that need no GPU: the library loads, exports every declared
symbol, and rejects invalid arguments before making any HIP call."""
import ctypes
import os

import pytest

import broadcast_subgraphs_amd as cf
from broadcast_subgraphs_amd import _lib

P = ctypes.c_void_p
A16 = 0x10000          # fake, 16-byte aligned addresses: never dereferenced,
B16 = 0x20000000       # validation rejects the call before any HIP call
C16 = 0x40000000


@pytest.fixture(scope="module")
def L():
    return cf.lib()


def test_exports_every_declared_symbol(L):
    names = cf.header_functions()
    assert len(names) >= 20
    for n in names:
        assert hasattr(L, n), f"libcf.so does not export {n}"
    # and the binding covers every declared function
    for n in names:
        assert n in _lib._SIGS, f"binding has no signature for {n}"


def test_status_strings(L):
    for s in range(7):
        assert cf.status_str(s).startswith(["CF_OK", "CF_EINVAL", "CF_EUNSUPPORTED", "CF_EALIGN",
                                            "CF_EWORKSPACE", "CF_EOCCUPANCY", "CF_EHIP"][s])
    assert cf.status_str(99) == "unknown cf_status"


def test_stitch_validation(L):
    z = ctypes.c_size_t(0)
    # null pointers
    assert L.cf_stitch_softmax(None, P(B16), 4, 4, None, z, None) == cf.CF_EINVAL
    assert L.cf_stitch_softmax(P(A16), None, 4, 4, None, z, None) == cf.CF_EINVAL
    # non-positive sizes
    assert L.cf_stitch_softmax(P(A16), P(B16), 0, 4, None, z, None) == cf.CF_EINVAL
    assert L.cf_stitch_layernorm(P(A16), P(B16), 4, -1, 1e-5, None, z, None) == cf.CF_EINVAL
    # aliasing input and output
    assert L.cf_stitch_softmax(P(A16), P(A16 + 8), 4, 4, None, z, None) == cf.CF_EINVAL
    # bad eps
    assert L.cf_stitch_layernorm(P(A16), P(B16), 4, 4, -1.0, None, z, None) == cf.CF_EINVAL
    assert L.cf_stitch_layernorm(P(A16), P(B16), 4, 4, float("nan"), None, z, None) == cf.CF_EINVAL
    # pow: v missing, y_pre aliasing y
    assert L.cf_stitch_pow_bcast_add(P(A16), None, 1.5, P(B16), None, 4, 4, None, z, None) == cf.CF_EINVAL
    assert L.cf_stitch_pow_bcast_add(P(A16), P(C16), 1.5, P(B16), P(B16), 4, 4, None, z, None) == cf.CF_EINVAL


def test_gemm_validation(L):
    z = ctypes.c_size_t(0)
    args = lambda A, W, Y, M, N, K, eps=1e-5: (P(A), P(W), P(C16), None, P(C16 + 0x1000), P(C16 + 0x2000),
                                               eps, P(Y), M, N, K, None, z, None)
    assert L.cf_gemm_ln(*args(A16, B16, C16 + 0x100000, 16, 12, 16)) == cf.CF_EUNSUPPORTED  # N % 8
    assert L.cf_gemm_ln(*args(A16, B16, C16 + 0x100000, 16, 16, 12)) == cf.CF_EUNSUPPORTED  # K % 8
    assert L.cf_gemm_ln(*args(A16 + 2, B16, C16 + 0x100000, 16, 16, 16)) == cf.CF_EALIGN
    assert L.cf_gemm_ln(*args(A16, B16, C16 + 0x100000, 0, 16, 16)) == cf.CF_EINVAL
    assert L.cf_gemm_ln(*args(A16, B16, C16 + 0x100000, 16, 16, 16, eps=-1.0)) == cf.CF_EINVAL
    # Y overlapping A
    assert L.cf_gemm_ln(*args(A16, B16, A16 + 64, 16, 16, 16)) == cf.CF_EINVAL
    assert L.cf_gemm_softmax(None, P(B16), 0.1, P(C16), 8, 8, 8, None, z, None) == cf.CF_EINVAL
    assert L.cf_gemm_softmax(P(A16), P(B16), float("inf"), P(C16), 8, 8, 8, None, z, None) == cf.CF_EINVAL
    assert L.cf_gemm_softmax(P(A16), P(B16), 0.1, P(C16), 8, 8, 6, None, z, None) == cf.CF_EUNSUPPORTED
    assert L.cf_gemm_softmax(P(A16), P(B16 + 4), 0.1, P(C16), 8, 8, 8, None, z, None) == cf.CF_EALIGN


def test_unfused_and_util_validation(L):
    z = ctypes.c_size_t(0)
    assert L.cf_unfused_stitch_softmax(None, P(B16), 4, 4, None, z, None) == cf.CF_EINVAL
    assert L.cf_unfused_stitch_layernorm(P(A16), P(B16), 4, 4, 1e-5, None, z, None) == cf.CF_EWORKSPACE
    assert L.cf_util_fill_f32(None, 4, 0.0, None) == cf.CF_EINVAL
    assert L.cf_util_copy_f32(P(A16), P(A16 + 4), 16, None) == cf.CF_EALIGN
    assert L.cf_util_copy_f32(P(A16), P(A16 + 16), 16, None) == cf.CF_EINVAL
    assert L.cf_graph_launch(None, None) == cf.CF_EINVAL
    assert L.cf_graph_destroy(None) == cf.CF_EINVAL


def test_workspace_query_rejects_bad_dims(L):
    bad = ctypes.c_size_t(-1).value
    assert L.cf_workspace_bytes(99, 4, 4, 0) == bad
    assert L.cf_workspace_bytes(cf.CF_OP_STITCH_SOFTMAX, 0, 4, 0) == bad
    assert L.cf_unfused_workspace_bytes(cf.CF_OP_GEMM_LN, 16, 16, 0) == bad
    # intermediates follow the 256-byte header and the 16384 eight-byte join words
    assert L.cf_unfused_workspace_bytes(cf.CF_OP_STITCH_SOFTMAX, 2, 3, 0) == 256 + 16384 * 8 + 2 * 256 + 2 * 256


def test_last_plan_is_a_string(L):
    s = cf.last_plan()
    assert isinstance(s, str)


def test_product_does_not_import_oracle():
    import os
    import re
    pkg = os.path.dirname(cf.__file__)
    for root, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".hpp", ".cpp", ".h")):
                txt = open(os.path.join(root, f)).read()
                assert not re.search(r"\boracle\b", txt), f"{f} mentions the oracle"


def test_spec_and_auto_validation_before_any_hip_call(L):
    from broadcast_subgraphs_amd._lib import GNode
    h = P()
    # null graph, bad terminal, non-positive sizes
    assert L.cf_spec_build(None, 1, 0, 4, 4, 0, ctypes.byref(h)) == cf.CF_EINVAL
    nodes = (GNode * 2)(GNode(cf.G_OPS["input"], -1, -1, 0, 0, 0.0), GNode(cf.G_OPS["exp"], 0, -1, 0, -1, 0.0))
    assert L.cf_spec_build(nodes, 2, 5, 4, 4, 0, ctypes.byref(h)) == cf.CF_EINVAL
    assert L.cf_spec_build(nodes, 2, 1, 0, 4, 0, ctypes.byref(h)) == cf.CF_EINVAL
    assert L.cf_spec_build(nodes, 2, 1, 4, 4, 0, None) == cf.CF_EINVAL
    # a valid S that no kernel implements (exp alone) is refused, not launched
    assert L.cf_spec_build(nodes, 2, 1, 4, 4, 0, ctypes.byref(h)) == cf.CF_EUNSUPPORTED
    assert L.cf_auto_build(None, 1, 0, 4, 4, ctypes.byref(h)) == cf.CF_EINVAL
    assert L.cf_auto_build(nodes, 2, 1, 4, 0, ctypes.byref(h)) == cf.CF_EINVAL
    # a built generated kernel rejects a missing argument and a null output before touching the device
    assert L.cf_auto_build(nodes, 2, 1, 4, 4, ctypes.byref(h)) == cf.CF_OK
    try:
        assert L.cf_auto_launch(h, None, 0, P(A16), None, 0, None) == cf.CF_EINVAL
        args = (P * 1)(P(B16))
        assert L.cf_auto_launch(h, args, 1, None, None, 0, None) == cf.CF_EINVAL
        # the output overlapping an input
        assert L.cf_auto_launch(h, args, 1, P(B16 + 16), None, 0, None) == cf.CF_EINVAL
    finally:
        L.cf_auto_free(h)
    assert L.cf_spec_launch(None, None, 0, P(A16), None, 0, None) == cf.CF_EINVAL


def test_bench_refuses_more_than_one_gpu():
    """bench.py runs on one GPU: --gpus above 1 exits with status 2 and a JSON error line,
    before touching torch or the device."""
    import json
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    p = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=root, timeout=120)
    assert p.returncode == 2
    msg = json.loads(p.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]
