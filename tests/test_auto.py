"""Automatic stitching on the host (no GPU): the schedule, the thread mapping, the generated kernel
(compiled with hiprtc for gfx950 here), and the graphs it refuses.

[AStitch] "Making it automatic" (dominants, index propagation, merging, locality check), "Four
stitching schemes", "Adaptive thread mapping".
"""
import pytest

import broadcast_subgraphs_amd as cf
from tests import graphs


def auto(g, rows, cols):
    nodes, t = g
    return cf.Auto(nodes, t, rows, cols)


@pytest.mark.parametrize("cols,lanes,frags,wg,waves", [
    (32, 8, 1, 256, 1), (33, 8, 2, 256, 1), (5, 8, 1, 256, 1), (1024, 64, 4, 256, 1), (1000, 64, 4, 256, 1),
    (1500, 128, 3, 256, 2), (2048, 128, 4, 256, 2),
    (4096, 256, 4, 256, 4), (30000, 1024, 8, 1024, 16), (32768, 1024, 8, 1024, 16)])
def test_thread_mapping_follows_the_row_length(cols, lanes, frags, wg, waves):
    d = auto(graphs.layernorm(cols), 100, cols).describe()
    m = d["mapping"]
    assert (m["lanes_per_row"], m["frags_per_lane"], m["workgroup"], m["waves_per_row"]) == (lanes, frags, wg, waves)
    assert m["rows_per_workgroup"] == wg // lanes
    assert lanes * frags * 4 >= cols
    # reductions cross waves through LDS only when a row spans several waves
    schemes = {e["scheme"] for e in d["edges"]}
    assert schemes == ({"local", "regional"} if waves > 1 else {"local"})
    assert d["kernels"] == 1 and d["code_bytes"] > 0


def test_regional_reduction_reads_the_waves_of_its_own_row():
    """Rows of 1025 to 2048 values take 128 lanes: two rows of two waves share a 256-lane
    workgroup, so each row's LDS combine starts at its own first wave (wave index with the
    low bit cleared), never at wave 0 for every row."""
    d = auto(graphs.layernorm(2048), 33, 2048)
    m = d.describe()["mapping"]
    assert (m["rows_per_workgroup"], m["waves_per_row"]) == (2, 2)
    src = d.source()
    assert src.count("red[slot][(threadIdx.x >> 6) & ~1u]") == 2 * 2  # two reductions, both variants
    assert "red[slot][0]" not in src


def test_pow_is_the_real_power():
    """pow in a generated kernel: integral exponents are real for negative bases (square and
    multiply), x^0 = 1 for every x, other exponents go through 2^(b log2 a)."""
    b = graphs.B()
    t = b.add("pow", b.ph("input", 0), b.c(3.0))
    src = auto((b.nodes, t), 8, 64).source()
    assert "cf_pow(" in src and "__builtin_rintf(b)" in src


def test_dominants_and_merge():
    d = auto(graphs.pow_softmax(1.5), 64, 30000).describe()
    kinds = [(x["op"], x["kind"]) for x in d["dominants"]]
    # v^p is computed once per row and broadcast; the two reductions and the output
    assert ("pow", "expensive_broadcast") in kinds
    assert kinds.count(("rowmax", "reduce")) == 1 and kinds.count(("rowsum", "reduce")) == 1
    assert kinds[-1][1] == "output"
    assert len(d["groups"]) == 1 and sorted(d["groups"][0]["dominants"]) == sorted(x["node"] for x in d["dominants"])
    assert [p["kind"] for p in d["params"]] == ["input", "colvec"]


def test_generated_source_has_both_variants():
    a = auto(graphs.softmax(), 256, 1024)
    src = a.source()
    name = a.describe()["kernel"]
    assert name.startswith("k_auto_") and name.endswith("_vec")
    assert name in src and name.replace("_vec", "_scalar") in src
    assert src.count("__shfl_xor") == 2 * 2 * 6  # two reductions of 64 lanes, in both variants


def test_refusals():
    with pytest.raises(cf.CFError) as e:
        auto(graphs.gemm_act("relu"), 64, 64)  # a MatMul root takes the GEMM entry points
    assert e.value.status == cf.CF_EUNSUPPORTED
    with pytest.raises(cf.CFError) as e:
        auto(graphs.layernorm(256 * 8192 + 1), 1, 256 * 8192 + 1)  # more than 256 member workgroups per row
    assert e.value.status == cf.CF_EUNSUPPORTED
    b = graphs.B()
    with pytest.raises(cf.CFError) as e:
        auto((b.nodes, b.add("rowsum", b.ph("input", 0))), 4, 8)  # a per-row output
    assert e.value.status == cf.CF_EUNSUPPORTED
    b = graphs.B()
    with pytest.raises(cf.CFError) as e:
        auto((b.nodes, b.add("exp", b.ph("input", 99))), 4, 8)  # slot out of range
    assert e.value.status == cf.CF_EINVAL
    b = graphs.B()
    with pytest.raises(cf.CFError) as e:
        auto((b.nodes, b.add("exp", b.ph("rowvec", 0))), 4, 8)  # no input tile to drive the rows
    assert e.value.status == cf.CF_EUNSUPPORTED


@pytest.mark.parametrize("cols,members", [(32769, 5), (100000, 13), (1 << 20, 128)])
def test_global_scheme_for_rows_wider_than_a_workgroup(cols, members):
    """Rows of more than 32768 values: slices of 256 lanes x 8 fragments, one workgroup each, and
    every reduction edge crosses workgroups (Global)."""
    d = auto(graphs.softmax(), 3, cols).describe()
    m = d["mapping"]
    assert (m["lanes_per_row"], m["frags_per_lane"], m["workgroups_per_row"]) == (256, 8, members)
    assert members * 256 * 8 * 4 >= cols > (members - 1) * 256 * 8 * 4
    red_edges = [e for e in d["edges"] if e["scheme"] != "local"]
    assert red_edges and all(e["scheme"] == "global" for e in red_edges)


def test_global_source_exchanges_tagged_partials():
    """Global scheme: each row reduction publishes the member's partial with one tagged store and
    takes every member's slot by the row's tag; one generation-counted join per launch (arrived on
    before the first loads, awaited at the first reduction) follows the clear of the member's
    slots, so nothing written before the launch can carry a tag it waits for."""
    src = auto(graphs.softmax(), 3, 100000).source()
    assert src.count("cf_put(pp + sl, tag,") == 2 * 2  # two reductions, in both variants
    assert src.count("cf_take(pp + q, tag,") == 2 * 2
    assert src.count("const unsigned tag = it_ + 1u;") == 2 * 2
    assert src.count("jold = cf_arrive(a.joins + rs)") == 2
    assert src.count("cf_await(a.joins + rs, jold") == 2
    for start in (0, src.index("_scalar(AutoArgs a)")):
        clear = src.index("__hip_atomic_store(a.slots", start)
        arrive = src.index("jold = cf_arrive", start)
        loop = src.index("for (long row = rs", start)
        first_take = src.index("cf_take(pp + q", start)
        await_ = src.index("cf_await(a.joins + rs, jold", start)
        assert clear < arrive < loop < await_ < first_take


def test_global_mapping_without_reductions_has_no_launch_join():
    """An element-wise graph on rows wider than a workgroup is cut into member slices like any
    Global graph, but with no reduction nothing crosses workgroups: the kernel arrives on no join
    word (an arrival never awaited would leave a shared word off by the member count)."""
    b = graphs.B()
    x = b.ph("input", 0)
    t = b.add("mul", b.add("silu", x), b.ph("rowvec", 1))
    a = auto((b.nodes, t), 3, 40000)
    assert a.describe()["mapping"]["workgroups_per_row"] == 5
    src = a.source()
    assert "cf_arrive(a.joins" not in src and "cf_await(a.joins" not in src and "cf_put(pp" not in src
