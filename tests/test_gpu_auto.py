"""Automatically stitched kernels on the GPU against the graph oracle (oracle.graph.evaluate)."""
import numpy as np
import pytest
import torch

import broadcast_subgraphs_amd as cf
import gen
import oracle
from tests import graphs
from tests.test_gpu_parity import TOL_F32, d32, dbf16, host, rownorm_err

pytestmark = pytest.mark.gpu

SHAPES = [(1000, 32), (999, 36), (5, 3), (7, 100), (33, 1024), (33, 2048), (5, 1500), (34, 1025), (3, 5000),
          (4, 30000), (2, 32768), (4099, 33), (3, 32769), (2, 100000), (5, 70001), (600, 40000)]


def _inputs(rows, cols, seed):
    x = gen.normal(seed, 0, (rows, cols))
    r = gen.normal(seed, 1, (rows, cols))
    g = (1.0 + 0.1 * gen.normal(seed, 2, (cols,)).astype(np.float64)).astype(np.float32)
    bt = gen.normal(seed, 3, (cols,), std=0.1)
    v = gen.uniform(seed, 4, (rows,), 0.1, 2.0)
    return x, r, g, bt, v


def _cases(rows, cols, x, r, g, bt, v):
    return [
        ("softmax", graphs.softmax(), [x]),
        ("layernorm", graphs.layernorm(cols), [x]),
        ("layernorm_affine", graphs.layernorm(cols, 1e-5, True), [x, g, bt]),
        ("rmsnorm_gain", graphs.rmsnorm(cols, 1e-5, True), [x, g]),
        ("pow_softmax", graphs.pow_softmax(1.5), [x, v]),
        ("silu_ln_scaled", graphs.silu_ln_scaled(cols), [x, bt, v]),
        ("softmax_temperature", graphs.softmax_temperature(), [x, v]),
        ("residual_ln", graphs.residual_ln(cols), [x, r, g, bt]),
        ("gelu_centered", graphs.gelu_centered(), [x, v]),
        ("rms_relu", graphs.rms_relu(cols), [x, g]),
    ]


@pytest.mark.parametrize("rows,cols", SHAPES)
def test_auto_graphs(rows, cols):
    x, r, g, bt, v = _inputs(rows, cols, 70 + cols % 17)
    for name, (nodes, t), hargs in _cases(rows, cols, x, r, g, bt, v):
        a = cf.Auto(nodes, t, rows, cols)
        out = torch.full((rows, cols), float("nan"), device="cuda")
        ws = a.launch([d32(h) for h in hargs], out)
        got = host(out)
        if ws is not None:
            assert ws.error_word() == 0, "a cross-workgroup wait gave up"
        want = oracle.graph.evaluate(nodes, t, hargs)
        assert rownorm_err(got, want) <= TOL_F32, (name, a.describe()["mapping"])


@pytest.mark.parametrize("p", [2.0, 3.0, 0.0, -1.0, 1.5])
def test_auto_pow_on_signed_input(p):
    """pow(x, p) + a row statistic on N(0,1) input (negative bases): integral exponents give the
    real power for either sign, x^0 = 1, and the non-integral 1.5 gives NaN exactly where the
    oracle's real power does (negative x)."""
    rows, cols = 37, 515
    x = gen.normal(95, 0, (rows, cols))
    b = graphs.B()
    xi = b.ph("input", 0)
    pw = b.add("pow", xi, b.c(p))
    t = b.add("add", pw, b.add("div", b.add("rowsum", b.add("square", xi)), b.c(cols)))
    a = cf.Auto(b.nodes, t, rows, cols)
    out = torch.full((rows, cols), 7.0, device="cuda")
    a.launch([d32(x)], out)
    got = host(out).astype(np.float64)
    with np.errstate(invalid="ignore"):  # the real power of a negative base to 1.5 is NaN, as intended
        want = oracle.graph.evaluate(b.nodes, t, [x])
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert ok.any()
    assert rownorm_err(np.where(ok, got, 0.0), np.where(ok, want, 0.0)) <= TOL_F32


@pytest.mark.parametrize("act,key", [("gelu_tanh", "gelu_tanh_values"), ("silu", "silu_values")])
def test_auto_activation_at_golden_points(act, key):
    """The generated kernel's GELU (tanh form) and SiLU in fp32 at the points the golden file
    derives by hand: the erf form of GELU is 1.5e-4 away at x = 1, far outside fp32 rounding."""
    import json
    import os
    gd = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")))[key]
    xs = np.array(gd["x"], np.float32)
    rows, cols = 3, 64
    x = np.resize(xs, (rows, cols)).astype(np.float32)
    want = np.resize(np.array(gd["y"]), (rows, cols))
    b = graphs.B()
    t = b.add(act, b.ph("input", 0))
    out = torch.full((rows, cols), float("nan"), device="cuda")
    cf.Auto(b.nodes, t, rows, cols).launch([d32(x)], out)
    got = host(out).astype(np.float64)
    assert np.max(np.abs(got - want) / np.abs(want)) <= 2e-6


def test_auto_misaligned_takes_the_scalar_variant_and_repeats_bitwise():
    rows, cols = 513, 64
    x, r, g, bt, v = _inputs(rows, cols, 90)
    nodes, t = graphs.residual_ln(cols)
    a = cf.Auto(nodes, t, rows, cols)
    buf = torch.full((rows * cols + 1,), float("nan"), device="cuda")
    out = buf[1:].view(rows, cols)  # 4-byte aligned only
    args = [d32(x), d32(r), d32(g), d32(bt)]
    a.launch(args, out)
    got = host(out)
    assert rownorm_err(got, oracle.graph.evaluate(nodes, t, [x, r, g, bt])) <= TOL_F32
    out2 = torch.empty((rows, cols), device="cuda")
    a.launch(args, out2)
    a.launch(args, out2)
    assert np.array_equal(host(out2), got)  # the 16-byte variant computes the same bits


def test_auto_launch_rejects_overlap_and_missing_args():
    nodes, t = graphs.layernorm(32)
    a = cf.Auto(nodes, t, 16, 32)
    X = torch.zeros((16, 32), device="cuda")
    with pytest.raises(cf.CFError) as e:
        a.launch([X], X)
    assert e.value.status == cf.CF_EINVAL
    with pytest.raises(cf.CFError) as e:
        a.launch([], torch.empty_like(X))
    assert e.value.status == cf.CF_EINVAL


def test_auto_global_rows_in_several_rounds_repeat_bitwise():
    """More rows than one round of co-resident member workgroups: the row groups walk the rows,
    the join words and partial buffers are reused round after round, and a second launch on the
    same workspace gives the same bits (members merge partials in a fixed order)."""
    rows, cols = 3000, 40000
    x, r, g, bt, v = _inputs(rows, cols, 91)
    nodes, t = graphs.layernorm(cols, 1e-5, True)
    a = cf.Auto(nodes, t, rows, cols)
    assert a.describe()["mapping"]["workgroups_per_row"] == 5
    args = [d32(x), d32(g), d32(bt)]
    out = torch.empty((rows, cols), device="cuda")
    ws = a.launch(args, out)
    first = host(out)
    assert ws.error_word() == 0
    assert rownorm_err(first, oracle.graph.evaluate(nodes, t, [x, g, bt])) <= TOL_F32
    a.launch(args, out, ws=ws)
    assert np.array_equal(host(out), first)
    assert ws.error_word() == 0


def test_auto_global_scalar_form_matches_vector_form_bitwise():
    """The Global scheme's two kernel forms hold different numbers of member workgroups at once,
    so they walk the rows in rounds of different sizes; one workspace of workspace_bytes() serves
    both, and each row's partials merge in member order either way, so the bits agree."""
    rows, cols = 1500, 40000
    x, r, g, bt, v = _inputs(rows, cols, 92)
    nodes, t = graphs.layernorm(cols, 1e-5, True)
    a = cf.Auto(nodes, t, rows, cols)
    args = [d32(x), d32(g), d32(bt)]
    ws = cf.Workspace(a.workspace_bytes())
    buf = torch.full((rows * cols + 1,), float("nan"), device="cuda")
    out_s = buf[1:].view(rows, cols)  # 4-byte aligned only: the scalar form
    a.launch(args, out_s, ws=ws)
    got_s = host(out_s)
    assert ws.error_word() == 0
    assert rownorm_err(got_s, oracle.graph.evaluate(nodes, t, [x, g, bt])) <= TOL_F32
    out_v = torch.empty((rows, cols), device="cuda")
    a.launch(args, out_v, ws=ws)
    assert ws.error_word() == 0
    assert np.array_equal(host(out_v), got_s)


def test_auto_global_layouts_and_library_ops_share_a_workspace():
    """Two generated kernels with different member counts per row (5 and 8) and a library op that
    writes its own partials where the slots lie take turns on one workspace: each launch clears
    its slots and joins each row's members before reading one, so what the others left behind
    never passes for a fresh partial, and every repeat gives the first launch's bits."""
    ka = (700, 40000)
    kb = (300, 1 << 16)
    xa = gen.normal(93, 0, ka)
    xb = gen.softmax_inputs(seed=94, rows=kb[0], cols=kb[1])["x"]
    na, ta = graphs.layernorm(ka[1])
    nb, tb = graphs.softmax()
    a = cf.Auto(na, ta, *ka)
    b = cf.Auto(nb, tb, *kb)
    assert a.describe()["mapping"]["workgroups_per_row"] == 5
    assert b.describe()["mapping"]["workgroups_per_row"] == 8
    q = gen.gemm_softmax_inputs(seed=96, M=512, N=1024, D=128)
    ws = cf.Workspace(max(a.workspace_bytes(), b.workspace_bytes(),
                          cf.cf_workspace_bytes(cf.CF_OP_GEMM_SOFTMAX, 512, 1024, 128)))
    XA, XB = d32(xa), d32(xb)
    oa, ob = torch.empty(ka, device="cuda"), torch.empty(kb, device="cuda")
    a.launch([XA], oa, ws=ws)
    first_a = host(oa)
    assert rownorm_err(first_a, oracle.graph.evaluate(na, ta, [xa])) <= TOL_F32
    b.launch([XB], ob, ws=ws)
    first_b = host(ob)
    assert rownorm_err(first_b, oracle.graph.evaluate(nb, tb, [xb])) <= TOL_F32
    S = torch.empty((512, 1024), dtype=torch.bfloat16, device="cuda")
    for _ in range(2):
        cf.cf_gemm_softmax(dbf16(q["q_bits"]), dbf16(q["k_bits"]), q["scale"], S, ws=ws)
        for k, X, o, first in ((a, XA, oa, first_a), (b, XB, ob, first_b)):
            o.fill_(float("nan"))
            k.launch([X], o, ws=ws)
            assert np.array_equal(host(o), first)
            assert ws.error_word() == 0


def test_auto_wide_rows_without_reductions_need_no_workspace():
    """Element-wise work on rows of 40000 values: five member slices per row, no exchange, so no
    workspace; a Global kernel with reductions still runs exactly before and after it on one."""
    rows, cols = 300, 40000
    x = gen.normal(97, 0, (rows, cols))
    v = gen.normal(97, 1, (cols,))
    b = graphs.B()
    xi = b.ph("input", 0)
    t = b.add("mul", b.add("silu", xi), b.ph("rowvec", 1))
    e = cf.Auto(b.nodes, t, rows, cols)
    assert e.describe()["mapping"]["workgroups_per_row"] == 5
    assert e.workspace_bytes() == 0
    out = torch.full((rows, cols), float("nan"), device="cuda")
    assert e.launch([d32(x), d32(v)], out) is None
    assert rownorm_err(host(out), oracle.graph.evaluate(b.nodes, t, [x, v])) <= TOL_F32
    nodes, tl = graphs.layernorm(cols)
    ln = cf.Auto(nodes, tl, rows, cols)
    ws = cf.Workspace(ln.workspace_bytes())
    y = torch.empty((rows, cols), device="cuda")
    ln.launch([d32(x)], y, ws=ws)
    first = host(y)
    assert rownorm_err(first, oracle.graph.evaluate(nodes, tl, [x])) <= TOL_F32
    e.launch([d32(x), d32(v)], out)
    ln.launch([d32(x)], y, ws=ws)
    assert np.array_equal(host(y), first)
    assert ws.error_word() == 0


@pytest.mark.parametrize("name", ["layernorm_750000x32", "silu_ln_scaled_750000x32", "softmax_512x65536"])
def test_auto_bench_workloads_at_full_size(name):
    """The generated kernels the bench times, at the sizes it times them."""
    if name == "softmax_512x65536":
        rows, cols = 512, 1 << 16
        x = gen.softmax_inputs(seed=11, rows=rows, cols=cols)["x"]
        nodes, t = graphs.softmax()
        hargs = [x]
    else:
        rows, cols = 750000, 32
        d = gen.layernorm_affine_inputs(seed=10)
        v = gen.uniform(10, 5, (rows,), 0.1, 2.0)
        if name.startswith("silu"):
            nodes, t = graphs.silu_ln_scaled(cols)
            hargs = [d["x"], d["beta"], v]
        else:
            nodes, t = graphs.layernorm(cols)
            hargs = [d["x"]]
    a = cf.Auto(nodes, t, rows, cols)
    out = torch.full((rows, cols), float("nan"), device="cuda")
    ws = a.launch([d32(h) for h in hargs], out)
    got = host(out)
    if ws is not None:
        assert ws.error_word() == 0
    assert rownorm_err(got, oracle.graph.evaluate(nodes, t, hargs)) <= TOL_F32
