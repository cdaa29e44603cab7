"""Fusion Spec IR on the GPU: a captured graph lowered, matched and launched gives the graph's
values (oracle.graph.evaluate) and the same bits as the entry point it dispatches to."""
import numpy as np
import pytest
import torch

import broadcast_subgraphs_amd as cf
import gen
import oracle
from tests import graphs
from tests.test_gpu_parity import TOL_BF16, TOL_F32, act_err, d32, dbf16, host, rownorm_err

pytestmark = pytest.mark.gpu


def _launch(g, args, out, rows, cols, k=0):
    nodes, t = g
    spec = cf.Spec(nodes, t, rows, cols, k)
    spec.launch(args, out)
    return host(out), spec.describe()


@pytest.mark.parametrize("commuted", [False, True])
@pytest.mark.parametrize("rows,cols", [(1000, 32), (7, 100), (3, 5000)])
def test_stitched_graphs(rows, cols, commuted):
    d = gen.layernorm_affine_inputs(seed=61, rows=rows, cols=cols)
    x, g, b = d["x"], d["gamma"], d["beta"]
    v = gen.pow_bcast_add_inputs(seed=62, rows=rows, cols=cols)["v"]
    X, G, Bt, V = d32(x), d32(g), d32(b), d32(v)
    cases = [
        (graphs.softmax(), [X], [x], lambda y: cf.cf_stitch_softmax(X, y)),
        (graphs.layernorm(cols, 1e-5, False, commuted), [X], [x], lambda y: cf.cf_stitch_layernorm(X, y, 1e-5)),
        (graphs.layernorm(cols, 1e-5, True, commuted), [X, G, Bt], [x, g, b],
         lambda y: cf.cf_stitch_layernorm_affine(X, G, Bt, y, 1e-5)),
        (graphs.rmsnorm(cols, 1e-5, False, commuted), [X], [x], lambda y: cf.cf_stitch_rmsnorm(X, None, y, 1e-5)),
        (graphs.rmsnorm(cols, 1e-5, True, commuted), [X, G], [x, g], lambda y: cf.cf_stitch_rmsnorm(X, G, y, 1e-5)),
        (graphs.pow_softmax(1.5, commuted), [X, V], [x, v], lambda y: cf.cf_stitch_pow_bcast_add(X, V, 1.5, y)),
    ]
    for gr, args, hargs, direct in cases:
        out = torch.full((rows, cols), float("nan"), device="cuda")
        got, desc = _launch(gr, args, out, rows, cols)
        want = oracle.graph.evaluate(gr[0], gr[1], hargs)
        assert rownorm_err(got, want) <= TOL_F32, desc["match"]
        ref = torch.full((rows, cols), float("nan"), device="cuda")
        direct(ref)
        assert np.array_equal(got, host(ref)), desc["match"]


@pytest.mark.parametrize("commuted", [False, True])
@pytest.mark.parametrize("M,N,K", [(300, 264, 72), (512, 1024, 256)])
def test_gemm_graphs(M, N, K, commuted):
    d = gen.gemm_ln_inputs(seed=63, M=M, N=N, K=K)
    A, W, Bias, R, G, Bt = (dbf16(d["a_bits"]), dbf16(d["w_bits"]), d32(d["bias"]), dbf16(d["r_bits"]),
                            d32(d["gamma"]), d32(d["beta"]))
    h = [d["a"], d["w"], d["bias"], d["r"], d["gamma"], d["beta"]]
    for res in (True, False):
        gr = graphs.gemm_ln(N, 1e-5, res, commuted)
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        got, desc = _launch(gr, [A, W, Bias, R if res else None, G, Bt], out, M, N, K)
        want = oracle.graph.evaluate(gr[0], gr[1], h)
        assert rownorm_err(got, want) <= TOL_BF16, desc["match"]
    for act in ["none", "relu", "gelu_tanh", "silu", "square", "rsqrt"]:
        q = gen.gemm_act_inputs(seed=64, M=M, N=N, K=K, positive=act == "rsqrt")
        A2, W2, B2 = dbf16(q["a_bits"]), dbf16(q["w_bits"]), d32(q["bias"])
        for bias in (True, False):
            gr = graphs.gemm_act(act, bias, commuted)
            out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            got, desc = _launch(gr, [A2, W2, B2 if bias else None], out, M, N, K)
            want = oracle.graph.evaluate(gr[0], gr[1], [q["a"], q["w"], q["bias"]])
            assert act_err(got, want) <= 1.0, desc["match"]
            ref = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
            cf.cf_gemm_act(A2, W2, B2 if bias else None, act, ref)
            assert torch.equal(out, ref)


def test_gemm_softmax_graph():
    M, N, D = 512, 1024, 128
    d = gen.gemm_softmax_inputs(seed=65, M=M, N=N, D=D)
    Q, Kt = dbf16(d["q_bits"]), dbf16(d["k_bits"])
    for cm in (False, True):
        gr = graphs.gemm_softmax(d["scale"], cm)
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        got, desc = _launch(gr, [Q, Kt], out, M, N, D)
        assert desc["match"]["call"] == "cf_gemm_softmax"
        want = oracle.graph.evaluate(gr[0], gr[1], [d["q"], d["k"]])
        assert rownorm_err(got, want) <= TOL_BF16


def test_spec_launch_rejects_missing_argument():
    nodes, t = graphs.layernorm(32, 1e-5, True)
    spec = cf.Spec(nodes, t, 16, 32)
    X = torch.zeros((16, 32), device="cuda")
    with pytest.raises(cf.CFError) as e:
        spec.launch([X, None, None], torch.empty_like(X))
    assert e.value.status == cf.CF_EINVAL
