"""Fusion Spec IR on the host (no GPU): Phi's nested S, Psi's match and its refusals.

[ComFuse] Frontend / Fusion Spec IR: Phi lowers a captured graph into
S = <N, E, tau, A, C> with a nested S after each reduction; Psi maps S onto
a precompiled kernel.  cf_spec_build is host code only, so every check here
runs without a GPU.
"""
import pytest

import broadcast_subgraphs_amd as cf
from tests import graphs

ROWS, COLS, K = 64, 256, 128
ACTS = ["none", "relu", "gelu_tanh", "silu", "square", "rsqrt"]


def build(g, rows=ROWS, cols=COLS, k=0):
    nodes, t = g
    return cf.Spec(nodes, t, rows, cols, k)


def refused(g, status, rows=ROWS, cols=COLS, k=0):
    with pytest.raises(cf.CFError) as e:
        build(g, rows, cols, k)
    assert e.value.status == status, cf.status_str(e.value.status)


FAMILIES = [
    ("softmax", lambda cm: graphs.softmax(), 0, "cf_stitch_softmax", 3, {"x": 0}, {}),
    ("layernorm", lambda cm: graphs.layernorm(COLS, 1e-5, False, cm), 0, "cf_stitch_layernorm", 3, {"x": 0},
     {"eps": 1e-5}),
    ("layernorm_affine", lambda cm: graphs.layernorm(COLS, 2e-5, True, cm), 0, "cf_stitch_layernorm_affine", 3,
     {"x": 0, "gamma": 1, "beta": 2}, {"eps": 2e-5}),
    ("rmsnorm", lambda cm: graphs.rmsnorm(COLS, 1e-6, False, cm), 0, "cf_stitch_rmsnorm", 2, {"x": 0}, {"eps": 1e-6}),
    ("rmsnorm_gain", lambda cm: graphs.rmsnorm(COLS, 1e-6, True, cm), 0, "cf_stitch_rmsnorm", 2,
     {"x": 0, "gamma": 1}, {"eps": 1e-6}),
    ("pow_softmax", lambda cm: graphs.pow_softmax(1.5, cm), 0, "cf_stitch_pow_bcast_add", 3, {"x": 0, "v": 1},
     {"p": 1.5}),
    ("gemm_ln", lambda cm: graphs.gemm_ln(COLS, 1e-5, True, cm), K, "cf_gemm_ln", 3,
     {"A": 0, "W": 1, "bias": 2, "R": 3, "gamma": 4, "beta": 5}, {"eps": 1e-5}),
    ("gemm_ln_no_residual", lambda cm: graphs.gemm_ln(COLS, 1e-5, False, cm), K, "cf_gemm_ln", 3,
     {"A": 0, "W": 1, "bias": 2, "gamma": 4, "beta": 5}, {"eps": 1e-5}),
    ("gemm_softmax", lambda cm: graphs.gemm_softmax(0.125, cm), K, "cf_gemm_softmax", 3, {"A": 0, "W": 1},
     {"scale": 0.125}),
]


@pytest.mark.parametrize("commuted", [False, True])
@pytest.mark.parametrize("name,mk,k,call,depth,args,consts", FAMILIES, ids=[f[0] for f in FAMILIES])
def test_family_is_matched(name, mk, k, call, depth, args, consts, commuted):
    d = build(mk(commuted), k=k).describe()
    assert d["match"]["call"] == call, d["signature"]
    assert d["depth"] == depth and len(d["levels"]) == depth
    assert d["match"]["args"] == args
    assert d["match"]["constants"] == pytest.approx(consts, rel=1e-15)
    # every level but the last ends in its reduction; later levels start from entry placeholders
    for lv in d["levels"][:-1]:
        tau = next(n for n in lv["nodes"] if n["id"] == lv["tau"])
        assert tau["cat"] == "reduce"
    for lv in d["levels"][1:]:
        cats = {n["cat"] for n in lv["nodes"]}
        assert "stat" in cats and "pass" in cats
    # the parameter table holds each placeholder once, with its slot
    assert sorted(p["slot"] for p in d["params"]) == sorted(set(args.values()))


@pytest.mark.parametrize("bias", [False, True])
@pytest.mark.parametrize("act", ACTS)
def test_activation_family(act, bias):
    for cm in (False, True):
        d = build(graphs.gemm_act(act, bias, cm), k=K).describe()
        assert d["match"]["call"] == "cf_gemm_act" and d["match"]["act"] == act
        assert d["depth"] == 1
        want = {"A": 0, "W": 1, **({"bias": 2} if bias else {})}
        assert d["match"]["args"] == want


def test_layernorm_levels_in_detail():
    """LayerNorm lowers to three levels: the input and its row sum; the passthrough x, the mean
    from the statistic, x - mean, its square and the second row sum; the passthrough x - mean,
    the rsqrt from the statistic and the product."""
    d = build(graphs.layernorm(COLS)).describe()
    l0, l1, l2 = d["levels"]
    assert [n["cat"] for n in l0["nodes"]] == ["acc", "reduce"]
    c1 = [(n["cat"], n["op"]) for n in l1["nodes"]]
    assert ("pass", "-") in c1 and ("stat", "rowsum") in c1 and ("compute", "sub") in c1
    assert ("compute", "square") in c1 and c1[-1] == ("reduce", "rowsum")
    c2 = [(n["cat"], n["op"]) for n in l2["nodes"]]
    assert ("compute", "rsqrt") in c2 and c2[-1] == ("compute", "mul")
    # the passthrough of level 2 is x - mean, computed in level 1
    p2 = next(n for n in l2["nodes"] if n["cat"] == "pass")
    src = next(n for n in l1["nodes"] if n["id"] == p2["in"][0])
    assert src["op"] == "sub"
    # the row length appears as scalar broadcasts
    assert sum(n["cat"] == "bcast_scalar" for lv in d["levels"] for n in lv["nodes"]) == 3


def test_refusals():
    # the mean's divisor must be the row length
    refused(graphs.layernorm(COLS + 1), cf.CF_EUNSUPPORTED)
    # negative eps
    refused(graphs.layernorm(COLS, -1e-5), cf.CF_EUNSUPPORTED)
    # a GEMM family without its reduction depth, and a stitched one with one
    refused(graphs.gemm_softmax(0.1), cf.CF_EINVAL, k=0)
    refused(graphs.softmax(), cf.CF_EINVAL, k=K)
    # softmax with sub and exp in the wrong order: a valid S that no kernel implements
    b = graphs.B()
    x = b.ph("input", 0)
    m = b.add("rowmax", x)
    e = b.add("sub", b.add("exp", x), m)
    refused((b.nodes, b.add("div", e, b.add("rowsum", e))), cf.CF_EUNSUPPORTED)
    # variance by E[x^2] - E[x]^2: two reductions in one stage
    b = graphs.B()
    x = b.ph("input", 0)
    s1, s2 = b.add("rowsum", x), b.add("rowsum", b.add("square", x))
    refused((b.nodes, b.add("mul", x, b.add("sub", s2, s1))), cf.CF_EUNSUPPORTED)
    # an operand read outside its MatMul
    b = graphs.B()
    a, w = b.ph("operand", 0), b.ph("operand", 1)
    refused((b.nodes, b.add("add", b.add("matmul", a, w), a)), cf.CF_EUNSUPPORTED, k=K)
    # a forward reference, and an out-of-range terminal
    refused(([("exp", 1, -1, 0, -1, 0.0), ("input", -1, -1, 0, 0, 0.0)], 0), cf.CF_EINVAL)
    refused((graphs.softmax()[0], 99), cf.CF_EINVAL)
    # the output is a per-row value, not a tile
    b = graphs.B()
    refused((b.nodes, b.add("rowsum", b.ph("input", 0))), cf.CF_EUNSUPPORTED)
    # two roots
    b = graphs.B()
    refused((b.nodes, b.add("add", b.ph("input", 0), b.ph("input", 1))), cf.CF_EUNSUPPORTED)


def test_dead_nodes_are_ignored():
    nodes, t = graphs.softmax()
    nodes = list(nodes) + [("exp", 0, -1, 0, -1, 0.0), ("rowvec", -1, -1, 0, 7, 0.0)]
    d = build((nodes, t)).describe()
    assert d["match"]["call"] == "cf_stitch_softmax"
    assert [p["slot"] for p in d["params"]] == [0]
