"""HIP path vs the fp64 oracle, through the C-ABI (needs an MI355X).

Error metric for every subgraph: per-row normalised max error
    err = max_i  max_j |g_ij - o_ij| / max_j |o_ij|
bounded by 1e-4 for the fp32 paths and 2e-2 for the bf16-output GEMM paths.
"""
import json

import numpy as np
import pytest
import torch

import broadcast_subgraphs_amd as cf
import gen
import oracle

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-4
TOL_BF16 = 2e-2


def rownorm_err(g, o):
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    assert g.shape == o.shape
    assert np.all(np.isfinite(g)), "non-finite GPU output"
    den = np.max(np.abs(o), axis=1)
    den[den == 0] = 1.0
    return float(np.max(np.max(np.abs(g - o), axis=1) / den))


def d32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def dbf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def host(t):
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def check_ws(ws):
    torch.cuda.synchronize()
    if ws is not None:
        assert ws.error_word() == 0, "a cross-workgroup wait gave up"


def empty_f32(rows, cols, misalign=False):
    if not misalign:
        return torch.full((rows, cols), float("nan"), dtype=torch.float32, device="cuda")
    buf = torch.full((rows * cols + 1,), float("nan"), dtype=torch.float32, device="cuda")
    return buf[1:].view(rows, cols)


# ------------------------------------------------------------------ softmax

SOFTMAX_SHAPES = [(256, 1024), (1, 1), (3, 5), (7, 13), (5, 64), (33, 100), (4099, 32), (17, 1000),
                  (9, 4096), (3, 16384), (4, 20000), (2, 65537), (1, 30000)]


@pytest.mark.parametrize("rows,cols", SOFTMAX_SHAPES)
def test_softmax(rows, cols):
    x = gen.softmax_inputs(seed=1, rows=rows, cols=cols)["x"]
    y = empty_f32(rows, cols)
    ws = cf.cf_stitch_softmax(d32(x), y)
    check_ws(ws)
    err = rownorm_err(host(y), oracle.softmax_rows(x))
    assert err <= TOL_F32, (err, cf.last_plan())


def test_softmax_misaligned_pointers():
    rows, cols = 6, 1024
    x = gen.softmax_inputs(seed=11, rows=rows, cols=cols)["x"]
    xb = torch.empty(rows * cols + 1, dtype=torch.float32, device="cuda")
    xb[1:] = d32(x).view(-1)
    xd = xb[1:].view(rows, cols)
    y = empty_f32(rows, cols, misalign=True)
    cf.cf_stitch_softmax(xd, y)
    assert '"frag_floats":1' in cf.last_plan()
    assert rownorm_err(host(y), oracle.softmax_rows(x)) <= TOL_F32


# ---------------------------------------------------------------- LayerNorm

LN_SHAPES = [(750000, 32), (1, 1), (5, 3), (1000, 32), (999, 36), (7, 100), (3, 1024), (4, 5000),
             (2, 30000), (3, 70001)]


@pytest.mark.parametrize("rows,cols", LN_SHAPES)
def test_layernorm(rows, cols):
    x = gen.layernorm_inputs(seed=2, rows=rows, cols=cols)["x"]
    y = empty_f32(rows, cols)
    ws = cf.cf_stitch_layernorm(d32(x), y, eps=1e-5)
    check_ws(ws)
    err = rownorm_err(host(y), oracle.layernorm_rows(x, 1e-5))
    assert err <= TOL_F32, (err, cf.last_plan())


def test_layernorm_constant_rows_are_zero():
    x = np.full((64, 32), 0.75, dtype=np.float32)
    y = empty_f32(64, 32)
    cf.cf_stitch_layernorm(d32(x), y, eps=1e-5)
    assert np.array_equal(host(y), np.zeros((64, 32), np.float32))


# -------------------------------------------------------- pow-broadcast-add

# RMSNorm and affine LayerNorm: every row plan (packed rows, 4-byte
# fragments for ragged rows, one row per workgroup, one wide row per
# workgroup, rows split across workgroups) and the full 750000 x 32 shape.
NORM_SHAPES = [(750000, 32), (1, 1), (5, 3), (1000, 32), (999, 36), (7, 100), (3, 1024), (4, 5000),
               (2, 30000), (3, 70001)]


@pytest.mark.parametrize("rows,cols", NORM_SHAPES)
def test_layernorm_affine(rows, cols):
    d = gen.layernorm_affine_inputs(seed=8, rows=rows, cols=cols)
    y = empty_f32(rows, cols)
    cf.cf_stitch_layernorm_affine(d32(d["x"]), d32(d["gamma"]), d32(d["beta"]), y, d["eps"])
    o = oracle.layernorm_affine_rows(d["x"], d["gamma"], d["beta"], d["eps"])
    err = rownorm_err(host(y), o)
    assert err <= TOL_F32, (err, cf.last_plan())


def test_layernorm_affine_wide_rows_plan():
    """A few rows of 30000: LayerNorm and RMSNorm hold each row in one 1024-lane
    workgroup (8 fragments per lane); affine LayerNorm, whose gain and bias
    fragments would not fit beside 8, splits the rows across workgroups."""
    rows, cols = 64, 30000
    d = gen.layernorm_affine_inputs(seed=18, rows=rows, cols=cols)
    y = empty_f32(rows, cols)
    cf.cf_stitch_layernorm(d32(d["x"]), y, d["eps"])
    p = json.loads(cf.last_plan())
    assert p["kernel"] == "k_rows" and p["lanes_per_row"] == 1024 and p["frags_per_lane"] == 8, p
    cf.cf_stitch_layernorm_affine(d32(d["x"]), d32(d["gamma"]), d32(d["beta"]), y, d["eps"])
    p = json.loads(cf.last_plan())
    assert p["kernel"] == "k_rows_split", p
    o = oracle.layernorm_affine_rows(d["x"], d["gamma"], d["beta"], d["eps"])
    assert rownorm_err(host(y), o) <= TOL_F32, p


@pytest.mark.parametrize("gain", [True, False])
@pytest.mark.parametrize("rows,cols", NORM_SHAPES)
def test_rmsnorm(rows, cols, gain):
    d = gen.rmsnorm_inputs(seed=7, rows=rows, cols=cols)
    g = d["gamma"] if gain else None
    y = empty_f32(rows, cols)
    cf.cf_stitch_rmsnorm(d32(d["x"]), d32(g) if gain else None, y, d["eps"])
    o = oracle.rmsnorm_rows(d["x"], g, d["eps"])
    err = rownorm_err(host(y), o)
    assert err <= TOL_F32, (err, cf.last_plan())


def test_norms_unfused_and_misaligned():
    rows, cols = 1000, 36
    d = gen.layernorm_affine_inputs(seed=8, rows=rows, cols=cols)
    y = empty_f32(rows, cols)
    cf.cf_stitch_layernorm_affine(d32(d["x"]), d32(d["gamma"]), d32(d["beta"]), y, d["eps"], unfused=True)
    assert rownorm_err(host(y), oracle.layernorm_affine_rows(d["x"], d["gamma"], d["beta"], d["eps"])) <= TOL_F32
    y = empty_f32(rows, cols, misalign=True)
    cf.cf_stitch_rmsnorm(d32(d["x"]), d32(d["gamma"]), y, d["eps"])
    assert json.loads(cf.last_plan())["frag_floats"] == 1
    assert rownorm_err(host(y), oracle.rmsnorm_rows(d["x"], d["gamma"], d["eps"])) <= TOL_F32
    y = empty_f32(rows, cols)
    cf.cf_stitch_rmsnorm(d32(d["x"]), None, y, d["eps"], unfused=True)
    assert rownorm_err(host(y), oracle.rmsnorm_rows(d["x"], None, d["eps"])) <= TOL_F32


POW_SHAPES = [(64, 30000), (3, 5), (7, 9), (64, 1024), (5, 20001), (1000, 32), (130, 8)]


@pytest.mark.parametrize("rows,cols", POW_SHAPES)
def test_pow_bcast_add(rows, cols):
    d = gen.pow_bcast_add_inputs(seed=3, rows=rows, cols=cols)
    y = empty_f32(rows, cols)
    ypre = empty_f32(rows, cols)
    ws = cf.cf_stitch_pow_bcast_add(d32(d["x"]), d32(d["v"]), d["p"], y, ypre)
    check_ws(ws)
    o, oy = oracle.pow_bcast_add_softmax(d["x"], d["v"], d["p"])
    assert rownorm_err(host(y), o) <= TOL_F32, cf.last_plan()
    assert rownorm_err(host(ypre), oy) <= TOL_F32, cf.last_plan()


def test_pow_bcast_add_without_y_pre():
    d = gen.pow_bcast_add_inputs(seed=33, rows=64, cols=30000)
    y = empty_f32(64, 30000)
    cf.cf_stitch_pow_bcast_add(d32(d["x"]), d32(d["v"]), d["p"], y, None)
    o, _ = oracle.pow_bcast_add_softmax(d["x"], d["v"], d["p"])
    assert rownorm_err(host(y), o) <= TOL_F32


# ---------------------------------------------------------------- GEMM + LN

GEMM_LN_SHAPES = [(300, 264, 72), (512, 1024, 256), (256, 128, 64), (17, 8, 8), (4096, 4096, 1024)]


def _gemm_ln_run(d, M, N, K, residual=True, unfused=False):
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")  # every element must be written
    ws = cf.cf_gemm_ln(dbf16(d["a_bits"]), dbf16(d["w_bits"]), d32(d["bias"]),
                       dbf16(d["r_bits"]) if residual else None, d32(d["gamma"]), d32(d["beta"]), Y,
                       eps=d["eps"], unfused=unfused)
    if not unfused:
        check_ws(ws)
    return host(Y)


@pytest.mark.parametrize("M,N,K", GEMM_LN_SHAPES)
def test_gemm_ln(M, N, K):
    d = gen.gemm_ln_inputs(seed=4, M=M, N=N, K=K)
    g = _gemm_ln_run(d, M, N, K)
    o = oracle.gemm_ln(d["a"], d["w"], d["bias"], d["r"], d["gamma"], d["beta"], d["eps"])
    err = rownorm_err(g, o)
    assert err <= TOL_BF16, (err, cf.last_plan())


def test_gemm_ln_default_plan_on_the_workload():
    """The 4096 x 4096 x 1024 workload runs on the 256 x 256 kernel, one tile per workgroup
    and a single launch (16 tiles per row block, all 256 tiles resident)."""
    d = gen.gemm_ln_inputs(seed=4, M=4096, N=4096, K=64)  # the workload's output shape, a short K
    _gemm_ln_run(d, 4096, 4096, 64)
    p = json.loads(cf.last_plan())
    assert (p["kernel"], p["tile"][:2], p["row_group"]) == ("k_gemm_ln3", [256, 256], 16), p
    assert p["rounds"] == 1, p


def test_gemm_ln_no_residual():
    M, N, K = 300, 264, 72
    d = gen.gemm_ln_inputs(seed=44, M=M, N=N, K=K, residual=False)
    g = _gemm_ln_run(d, M, N, K, residual=False)
    o = oracle.gemm_ln(d["a"], d["w"], d["bias"], None, d["gamma"], d["beta"], d["eps"])
    assert rownorm_err(g, o) <= TOL_BF16


def test_gemm_ln_ones_gives_beta_exactly():
    """A = W = 1, bias = 0, R = 0: every row of A.W is K, so y = beta_j (bf16-rounded) exactly."""
    M, N, K = 512, 4096, 1024
    d = gen.gemm_ln_inputs(seed=4, M=M, N=N, K=K)
    one = gen.f32_to_bf16_bits(np.ones(1, np.float32))[0]
    zero = gen.f32_to_bf16_bits(np.zeros(1, np.float32))[0]
    d["a_bits"] = np.full((M, K), one, np.uint16)
    d["w_bits"] = np.full((K, N), one, np.uint16)
    d["r_bits"] = np.full((M, N), zero, np.uint16)
    d["bias"] = np.zeros(N, np.float32)
    g = _gemm_ln_run(d, M, N, K)
    beta_bf16 = gen.bf16_bits_to_f32(gen.f32_to_bf16_bits(d["beta"]))
    assert np.array_equal(g, np.repeat(beta_bf16[None, :], M, axis=0))


# ----------------------------------------------------------- GEMM + softmax

GEMM_SM_SHAPES = [(300, 264, 72), (512, 1024, 128), (256, 128, 64), (17, 8, 8), (8192, 8192, 128)]


def _gemm_sm_run(d, M, N, D, unfused=False):
    S = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")  # every element must be written
    ws = cf.cf_gemm_softmax(dbf16(d["q_bits"]), dbf16(d["k_bits"]), d["scale"], S, unfused=unfused)
    if not unfused:
        check_ws(ws)
    return host(S)


@pytest.mark.parametrize("M,N,D", GEMM_SM_SHAPES)
def test_gemm_softmax(M, N, D):
    d = gen.gemm_softmax_inputs(seed=5, M=M, N=N, D=D)
    g = _gemm_sm_run(d, M, N, D)
    o = oracle.gemm_softmax(d["q"], d["k"], d["scale"])
    err = rownorm_err(g, o)
    assert err <= TOL_BF16, (err, cf.last_plan())
    rs = g.astype(np.float64).sum(axis=1)
    assert np.max(np.abs(rs - 1.0)) <= 8e-3  # bf16 rounding of each term is within 2^-9 relative


def test_gemm_softmax_zero_q_is_exact():
    """Q = 0: every score is equal, so every output is 1/8192 = 2^-13, exact in bf16."""
    M, N, D = 512, 8192, 128
    d = gen.gemm_softmax_inputs(seed=5, M=M, N=N, D=D)
    d["q_bits"] = np.zeros((M, D), np.uint16)
    g = _gemm_sm_run(d, M, N, D)
    assert np.array_equal(g, np.full((M, N), 2.0 ** -13, np.float32))


# Back-to-back GEMM with the softmax between: ragged tails on every axis, a
# single strip per row (one 64-key tile), several strips per row block, strips
# of an odd number of tiles (3 per strip with a ragged last tile; 3 per strip
# with a last strip of 1), and the full 8192 x 8192 x 128 x 128 workload.
B2B_SHAPES = [(300, 264, 72, 40), (512, 1024, 128, 128), (17, 8, 8, 8), (130, 40, 32, 16),
              (1000, 2056, 128, 64), (8192, 1496, 128, 128), (4096, 2536, 96, 72), (8192, 8192, 128, 128)]


def _b2b_run(d, M, N, D, Dv, unfused=False, ws=None):
    O = torch.full((M, Dv), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = cf.cf_gemm_softmax_gemm(dbf16(d["q_bits"]), dbf16(d["k_bits"]), dbf16(d["v_bits"]), d["scale"], O,
                                 ws=ws, unfused=unfused)
    if not unfused:
        check_ws(ws)
    return host(O)


@pytest.mark.parametrize("M,N,D,Dv", B2B_SHAPES)
def test_gemm_softmax_gemm(M, N, D, Dv):
    d = gen.gemm_softmax_gemm_inputs(seed=6, M=M, N=N, D=D, Dv=Dv)
    g = _b2b_run(d, M, N, D, Dv)
    o = oracle.gemm_softmax_gemm(d["q"], d["k"], d["v"], d["scale"])
    err = rownorm_err(g, o)
    assert err <= TOL_BF16, (err, cf.last_plan())


def test_gemm_softmax_gemm_plan_uses_strips():
    """The 8192-row workload runs several strips per row block in one round, and
    a 40-key row runs one strip (the direct commit)."""
    d = gen.gemm_softmax_gemm_inputs(seed=6, M=1024, N=8192, D=128, Dv=128)
    _b2b_run(d, 1024, 8192, 128, 128)
    p = json.loads(cf.last_plan())
    assert p["kernel"] == "k_gemm_b2b" and p["row_group"] > 1 and p["rounds"] == 1, p
    d = gen.gemm_softmax_gemm_inputs(seed=6, M=130, N=40, D=32, Dv=16)
    _b2b_run(d, 130, 40, 32, 16)
    assert json.loads(cf.last_plan())["row_group"] == 1, cf.last_plan()


def test_gemm_softmax_gemm_unfused():
    M, N, D, Dv = 512, 1024, 128, 128
    d = gen.gemm_softmax_gemm_inputs(seed=6, M=M, N=N, D=D, Dv=Dv)
    g = _b2b_run(d, M, N, D, Dv, unfused=True)
    o = oracle.gemm_softmax_gemm(d["q"], d["k"], d["v"], d["scale"])
    assert rownorm_err(g, o) <= TOL_BF16


def test_gemm_softmax_gemm_negative_scale_and_zero_q():
    M, N, D, Dv = 256, 1000, 64, 96
    d = gen.gemm_softmax_gemm_inputs(seed=7, M=M, N=N, D=D, Dv=Dv)
    d["scale"] = -abs(d["scale"])
    o = oracle.gemm_softmax_gemm(d["q"], d["k"], d["v"], d["scale"])
    assert rownorm_err(_b2b_run(d, M, N, D, Dv), o) <= TOL_BF16, cf.last_plan()
    d["q_bits"] = np.zeros_like(d["q_bits"])
    d["q"] = np.zeros_like(d["q"])
    o = oracle.gemm_softmax_gemm(d["q"], d["k"], d["v"], d["scale"])
    assert rownorm_err(_b2b_run(d, M, N, D, Dv), o) <= TOL_BF16, cf.last_plan()


def _b2b_inputs_from(q32, k32, v32, scale):
    qb, kb, vb = (gen.f32_to_bf16_bits(np.ascontiguousarray(x, np.float32)) for x in (q32, k32, v32))
    return {"q_bits": qb, "q": gen.bf16_bits_to_f32(qb), "k_bits": kb, "k": gen.bf16_bits_to_f32(kb),
            "v_bits": vb, "v": gen.bf16_bits_to_f32(vb), "scale": float(np.float32(scale))}


def test_gemm_softmax_gemm_rising_max():
    """Key magnitudes ramp up along the row, with a large scale: each row's max
    grows by far more than 2^8 across a strip's tiles, so the running reference
    moves (and the accumulator is rescaled) mid-strip, and the strips' maxima
    differ widely at the commit."""
    M, N, D, Dv = 512, 4096, 64, 64
    ramp = (1.0 + 6.0 * np.arange(N) / N).astype(np.float32)
    d = _b2b_inputs_from(gen.normal(11, 0, (M, D)), gen.normal(11, 1, (N, D)) * ramp[:, None],
                         gen.normal(11, 2, (N, Dv)), 0.5)
    g = _b2b_run(d, M, N, D, Dv)
    o = oracle.gemm_softmax_gemm(d["q"], d["k"], d["v"], d["scale"])
    assert rownorm_err(g, o) <= TOL_BF16, cf.last_plan()


def test_gemm_softmax_gemm_zero_scale_is_the_mean():
    """scale = 0: every weight is 1/N, so each output row is the column mean of V."""
    M, N, D, Dv = 256, 2048, 32, 32
    d = gen.gemm_softmax_gemm_inputs(seed=12, M=M, N=N, D=D, Dv=Dv)
    d["scale"] = 0.0
    g = _b2b_run(d, M, N, D, Dv)
    o = np.repeat(d["v"].astype(np.float64).mean(axis=0)[None, :], M, axis=0)
    assert rownorm_err(g, o) <= TOL_BF16


def test_gemm_softmax_gemm_deterministic_on_one_workspace():
    """Fixed strip order in the partial-output sum: repeated calls (one workspace)
    give identical bits, also after a plain softmax call used the same join words."""
    M, N, D, Dv = 1024, 8192, 128, 128
    d = gen.gemm_softmax_gemm_inputs(seed=8, M=M, N=N, D=D, Dv=Dv)
    need = max(cf.cf_workspace_bytes(cf.CF_OP_GEMM_SOFTMAX_GEMM, M, N, D),
               cf.cf_workspace_bytes(cf.CF_OP_GEMM_SOFTMAX, M, N, D))
    ws = cf.Workspace(need)
    a = _b2b_run(d, M, N, D, Dv, ws=ws)
    S = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    cf.cf_gemm_softmax(dbf16(d["q_bits"]), dbf16(d["k_bits"]), d["scale"], S, ws=ws)
    b = _b2b_run(d, M, N, D, Dv, ws=ws)
    assert np.array_equal(a, b)


def test_gemm_softmax_gemm_rejects():
    q = torch.zeros((64, 32), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((64, 32), dtype=torch.bfloat16, device="cuda")
    v12 = torch.zeros((64, 12), dtype=torch.bfloat16, device="cuda")
    o12 = torch.zeros((64, 12), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(cf.CFError) as e:
        cf.cf_gemm_softmax_gemm(q, k, v12, 0.1, o12)
    assert e.value.status == cf.CF_EUNSUPPORTED
    v = torch.zeros((64, 16), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(cf.CFError) as e:
        cf.cf_gemm_softmax_gemm(q, k, v, 0.1, v[:, :16])  # O aliases V
    assert e.value.status == cf.CF_EINVAL
    q136 = torch.zeros((64, 136), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(cf.CFError) as e:
        cf.cf_gemm_softmax_gemm(q136, q136, v, 0.1, torch.zeros((64, 16), dtype=torch.bfloat16, device="cuda"))
    assert e.value.status == cf.CF_EUNSUPPORTED


# ------------------------------------------------ GEMM + unary activation

ACTS = ["none", "relu", "gelu_tanh", "silu", "square", "rsqrt"]
GEMM_ACT_SHAPES = [(300, 264, 72), (17, 8, 8), (512, 1024, 256), (129, 136, 1032), (8300, 4096, 64)]


def act_err(g, o):
    """max_ij |g - o| / (2^-8 |o_ij| + 2^-12 max|o|): at most 1 passes.

    bf16 rounding to nearest moves a value by at most 2^-9 of itself; the
    2^-12 max|o| floor covers the fp32 accumulation and the activation's
    fp32 evaluation near zero crossings."""
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    assert g.shape == o.shape
    assert np.all(np.isfinite(g)), "non-finite GPU output"
    floor = 2.0 ** -12 * max(float(np.max(np.abs(o))), 1e-30)
    return float(np.max(np.abs(g - o) / (2.0 ** -8 * np.abs(o) + floor)))


def _gemm_act_run(d, M, N, act, bias=True, unfused=False):
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    ws = cf.cf_gemm_act(dbf16(d["a_bits"]), dbf16(d["w_bits"]), d32(d["bias"]) if bias else None, act, Y,
                        unfused=unfused)
    check_ws(ws)
    return host(Y)


def _act_inputs(act, seed, M, N, K):
    # rsqrt is defined on positive values: its operands make every A.W + bias positive
    return gen.gemm_act_inputs(seed=seed, M=M, N=N, K=K, positive=act == "rsqrt")


@pytest.mark.parametrize("algo", [0, 1])
@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("M,N,K", GEMM_ACT_SHAPES)
def test_gemm_act(monkeypatch, M, N, K, act, algo):
    monkeypatch.setenv("CF_GEMM_ACT_ALGO", str(algo))
    d = _act_inputs(act, 9, M, N, K)
    g = _gemm_act_run(d, M, N, act)
    o = oracle.gemm_act(d["a"], d["w"], d["bias"], act)
    assert act_err(g, o) <= 1.0, (act_err(g, o), cf.last_plan())


@pytest.mark.parametrize("act", ["gelu_tanh", "silu", "rsqrt"])
def test_gemm_act_full_size(act):
    M, N, K = 4096, 4096, 1024
    d = _act_inputs(act, 9, M, N, K)
    g = _gemm_act_run(d, M, N, act)
    plan = json.loads(cf.last_plan())
    assert plan["kernel"] == "k_gemm_act2" and plan["schedule"] == "independent-tiles", plan
    o = oracle.gemm_act(d["a"], d["w"], d["bias"], act)
    assert act_err(g, o) <= 1.0, act_err(g, o)


@pytest.mark.parametrize("act", ACTS)
def test_gemm_act_no_bias_and_unfused(act):
    M, N, K = 300, 264, 72
    d = _act_inputs(act, 19, M, N, K)
    o = oracle.gemm_act(d["a"], d["w"], None, act)
    assert act_err(_gemm_act_run(d, M, N, act, bias=False), o) <= 1.0
    assert act_err(_gemm_act_run(d, M, N, act, bias=False, unfused=True), o) <= 1.0
    o = oracle.gemm_act(d["a"], d["w"], d["bias"], act)
    assert act_err(_gemm_act_run(d, M, N, act, unfused=True), o) <= 1.0


@pytest.mark.parametrize("act", ACTS)
def test_gemm_act_ones_are_exact(act):
    """A = W = 1, bias = 0: every u is K = 1024, and act(1024) is a bf16 value
    (1024, 2^20 for the square, 2^-5 for rsqrt): the output is exact.  For the
    gated forms the gate's exponent is far below the exp2 range, so the gate is 1."""
    M, N, K = 256, 512, 1024
    one = gen.f32_to_bf16_bits(np.ones(1, np.float32))[0]
    d = {"a_bits": np.full((M, K), one, np.uint16), "w_bits": np.full((K, N), one, np.uint16),
         "bias": np.zeros(N, np.float32)}
    g = _gemm_act_run(d, M, N, act)
    want = {"square": float(K) ** 2, "rsqrt": 1.0 / 32.0}.get(act, float(K))
    assert np.all(g == want)


@pytest.mark.parametrize("cfg", range(1, 6))
def test_gemm_act_every_tile_config(monkeypatch, cfg):
    """The round-based kernel (128-wide tiles, two workgroups per CU) in every tile configuration."""
    monkeypatch.setenv("CF_GEMM_ACT_ALGO", "0")
    monkeypatch.setenv("CF_GEMM_ACT_CFG", str(cfg))
    M, N, K = 300, 264, 72
    d = gen.gemm_act_inputs(seed=29, M=M, N=N, K=K)
    g = _gemm_act_run(d, M, N, "gelu_tanh")
    o = oracle.gemm_act(d["a"], d["w"], d["bias"], "gelu_tanh")
    assert act_err(g, o) <= 1.0, cf.last_plan()


ACT2_SHAPES = [(300, 264, 72), (17, 8, 8), (129, 136, 1032), (4133, 8192, 128), (4133, 4096, 192)]


@pytest.mark.parametrize("cfg", range(4))
@pytest.mark.parametrize("M,N,K", ACT2_SHAPES)
def test_gemm_act_large_tiles(monkeypatch, cfg, M, N, K):
    """The large-tile kernel (one 8-wave workgroup per CU) in every ring
    configuration: ragged edges, more tiles than workgroups (the next tile's
    first stages prefetched during the epilogue when the stage count allows),
    and each activation across the configurations."""
    monkeypatch.setenv("CF_GEMM_ACT_ALGO", "1")
    monkeypatch.setenv("CF_GEMM_ACT_CFG", str(cfg))
    act = ACTS[(cfg + K) % len(ACTS)]
    d = _act_inputs(act, 39, M, N, K)
    g = _gemm_act_run(d, M, N, act)
    plan = json.loads(cf.last_plan())
    assert plan["kernel"] == "k_gemm_act2", plan
    o = oracle.gemm_act(d["a"], d["w"], d["bias"], act)
    assert act_err(g, o) <= 1.0, (act, act_err(g, o), plan)


@pytest.mark.parametrize("act", ACTS)
def test_gemm_act_large_tiles_full_size_no_bias(monkeypatch, act):
    monkeypatch.setenv("CF_GEMM_ACT_ALGO", "1")
    M, N, K = 4096, 4096, 1024
    d = _act_inputs(act, 49, M, N, K)
    g = _gemm_act_run(d, M, N, act, bias=act != "none")
    o = oracle.gemm_act(d["a"], d["w"], d["bias"] if act != "none" else None, act)
    assert act_err(g, o) <= 1.0, act_err(g, o)


def test_gemm_act_rejects():
    A = torch.zeros((64, 32), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((32, 64), dtype=torch.bfloat16, device="cuda")
    Y = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros(65, dtype=torch.float32, device="cuda")
    assert cf.cf_workspace_bytes(cf.CF_OP_GEMM_ACT, 64, 64, 32) == 0
    with pytest.raises(cf.CFError) as e:
        cf.cf_gemm_act(A, W, b[:64], 6, Y)  # no such activation
    assert e.value.status == cf.CF_EINVAL
    with pytest.raises(cf.CFError) as e:
        cf.cf_gemm_act(A, W, b[1:], "relu", Y)  # bias not 16-byte aligned
    assert e.value.status == cf.CF_EALIGN
    with pytest.raises(cf.CFError) as e:
        cf.cf_gemm_act(A, A, b[:64], "relu", A)  # Y aliases A
    assert e.value.status == cf.CF_EINVAL
    W12 = torch.zeros((32, 12), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(cf.CFError) as e:
        cf.cf_gemm_act(A, W12, None, "relu", torch.zeros((64, 12), dtype=torch.bfloat16, device="cuda"))
    assert e.value.status == cf.CF_EUNSUPPORTED


# Every GEMM epilogue schedule the planner can pick (forced through its
# CF_GEMM_ALGO override): 0 one join per round, 1 joins overlapped with
# MainLoops, 2 softmax by strips.
SCHEDULE_SHAPES = [(300, 264, 72), (512, 1024, 128), (17, 8, 8), (1000, 2056, 128)]


@pytest.mark.parametrize("algo", [0, 1])
@pytest.mark.parametrize("M,N,K", SCHEDULE_SHAPES)
def test_gemm_ln_every_schedule(monkeypatch, algo, M, N, K):
    monkeypatch.setenv("CF_GEMM_ALGO", str(algo))
    d = gen.gemm_ln_inputs(seed=6, M=M, N=N, K=K)
    g = _gemm_ln_run(d, M, N, K)
    o = oracle.gemm_ln(d["a"], d["w"], d["bias"], d["r"], d["gamma"], d["beta"], d["eps"])
    assert rownorm_err(g, o) <= TOL_BF16, cf.last_plan()


@pytest.mark.parametrize("algo", [0, 1, 2])
@pytest.mark.parametrize("M,N,D", SCHEDULE_SHAPES)
def test_gemm_softmax_every_schedule(monkeypatch, algo, M, N, D):
    monkeypatch.setenv("CF_GEMM_ALGO", str(algo))
    d = gen.gemm_softmax_inputs(seed=7, M=M, N=N, D=D)
    g = _gemm_sm_run(d, M, N, D)
    o = oracle.gemm_softmax(d["q"], d["k"], d["scale"])
    assert rownorm_err(g, o) <= TOL_BF16, cf.last_plan()


@pytest.mark.parametrize("cfg", range(8))
@pytest.mark.parametrize("M,N,K", [(512, 1024, 256), (300, 264, 72)])
def test_gemm_ln_every_tile_config(monkeypatch, cfg, M, N, K):
    """Every tile configuration of the overlapped GEMM+LN kernel (forced through
    the planner's CF_GEMM_LN_CFG override), including the one-tile-at-a-time
    8-wave configuration whose epilogue scratch lives in the idle ring."""
    monkeypatch.setenv("CF_GEMM_LN_CFG", str(cfg))
    d = gen.gemm_ln_inputs(seed=9, M=M, N=N, K=K)
    g = _gemm_ln_run(d, M, N, K)
    o = oracle.gemm_ln(d["a"], d["w"], d["bias"], d["r"], d["gamma"], d["beta"], d["eps"])
    assert rownorm_err(g, o) <= TOL_BF16, cf.last_plan()


@pytest.mark.parametrize("cfg", [0, 7])
def test_gemm_ln_one_tile_at_a_time_rounds(monkeypatch, cfg):
    """More 256 x 256 tiles than resident workgroups: whole row blocks per
    round (one kernel round after another, or one launch per round), the
    epilogue scratch in the ring; ragged last row block and column tile."""
    monkeypatch.setenv("CF_GEMM_LN_CFG", str(cfg))
    M, N, K = 256 * 40 - 37, 2048 - 120, 64
    d = gen.gemm_ln_inputs(seed=10, M=M, N=N, K=K)
    g = _gemm_ln_run(d, M, N, K)
    assert json.loads(cf.last_plan())["rounds"] >= 2, cf.last_plan()
    o = oracle.gemm_ln(d["a"], d["w"], d["bias"], d["r"], d["gamma"], d["beta"], d["eps"])
    assert rownorm_err(g, o) <= TOL_BF16, cf.last_plan()


def test_gemm_softmax_negative_scale():
    """A negative scale flips which raw score is the row maximum."""
    M, N, D = 256, 1000, 64
    d = gen.gemm_softmax_inputs(seed=8, M=M, N=N, D=D)
    d["scale"] = -abs(d["scale"])
    g = _gemm_sm_run(d, M, N, D)
    o = oracle.gemm_softmax(d["q"], d["k"], d["scale"])
    assert rownorm_err(g, o) <= TOL_BF16, cf.last_plan()


def test_fused_after_unfused_on_one_workspace():
    """The unfused chains' intermediates never touch the join words: a fused
    call on a workspace an unfused call just used still joins correctly."""
    M, N, D = 512, 1024, 128
    q = gen.gemm_softmax_inputs(seed=5, M=M, N=N, D=D)
    need = max(cf.cf_unfused_workspace_bytes(cf.CF_OP_GEMM_SOFTMAX, M, N, D),
               cf.cf_workspace_bytes(cf.CF_OP_GEMM_SOFTMAX, M, N, D))
    ws = cf.Workspace(need)
    S = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    cf.cf_gemm_softmax(dbf16(q["q_bits"]), dbf16(q["k_bits"]), q["scale"], S, ws=ws, unfused=True)
    cf.cf_gemm_softmax(dbf16(q["q_bits"]), dbf16(q["k_bits"]), q["scale"], S, ws=ws)
    check_ws(ws)
    o = oracle.gemm_softmax(q["q"], q["k"], q["scale"])
    assert rownorm_err(host(S), o) <= TOL_BF16


# ------------------------------------------------------------- determinism

def test_deterministic_runs():
    x = gen.pow_bcast_add_inputs(seed=3)
    y1, y2 = empty_f32(64, 30000), empty_f32(64, 30000)
    cf.cf_stitch_pow_bcast_add(d32(x["x"]), d32(x["v"]), 1.5, y1)
    cf.cf_stitch_pow_bcast_add(d32(x["x"]), d32(x["v"]), 1.5, y2)
    assert torch.equal(y1, y2)
    d = gen.gemm_ln_inputs(seed=4, M=1024, N=4096, K=256)
    assert np.array_equal(_gemm_ln_run(d, 1024, 4096, 256), _gemm_ln_run(d, 1024, 4096, 256))
    q = gen.gemm_softmax_inputs(seed=5, M=1024, N=8192, D=128)
    assert np.array_equal(_gemm_sm_run(q, 1024, 8192, 128), _gemm_sm_run(q, 1024, 8192, 128))


# ------------------------------------------------------------ metamorphic

def test_row_permutation():
    rng = np.random.default_rng(0)
    d = gen.pow_bcast_add_inputs(seed=3)
    perm = rng.permutation(64)
    y, yp = empty_f32(64, 30000), empty_f32(64, 30000)
    cf.cf_stitch_pow_bcast_add(d32(d["x"]), d32(d["v"]), 1.5, y)
    cf.cf_stitch_pow_bcast_add(d32(d["x"][perm]), d32(d["v"][perm]), 1.5, yp)
    assert np.array_equal(host(y)[perm], host(yp))
    M, N, K = 512, 1024, 128
    g = gen.gemm_ln_inputs(seed=4, M=M, N=N, K=K)
    p = rng.permutation(M)
    base = _gemm_ln_run(g, M, N, K)
    g2 = dict(g)
    g2["a_bits"], g2["r_bits"] = g["a_bits"][p], g["r_bits"][p]
    assert np.array_equal(base[p], _gemm_ln_run(g2, M, N, K))


def test_column_permutation_gemm():
    rng = np.random.default_rng(1)
    M, N, K = 256, 1024, 128
    g = gen.gemm_ln_inputs(seed=4, M=M, N=N, K=K)
    p = rng.permutation(N)
    base = _gemm_ln_run(g, M, N, K)
    g2 = dict(g)
    g2["w_bits"], g2["r_bits"] = g["w_bits"][:, p], g["r_bits"][:, p]
    g2["bias"], g2["gamma"], g2["beta"] = g["bias"][p], g["gamma"][p], g["beta"][p]
    assert rownorm_err(_gemm_ln_run(g2, M, N, K), base[:, p]) <= TOL_BF16
    q = gen.gemm_softmax_inputs(seed=5, M=M, N=N, D=128)
    sb = _gemm_sm_run(q, M, N, 128)
    q2 = dict(q)
    q2["k_bits"] = q["k_bits"][p]
    assert rownorm_err(_gemm_sm_run(q2, M, N, 128), sb[:, p]) <= TOL_BF16


# ------------------------------------------------- unfused chains and graphs

def test_unfused_chains_match_oracle():
    x = gen.softmax_inputs(seed=1)["x"]
    y = empty_f32(256, 1024)
    cf.cf_stitch_softmax(d32(x), y, unfused=True)
    assert rownorm_err(host(y), oracle.softmax_rows(x)) <= TOL_F32
    x = gen.layernorm_inputs(seed=2, rows=10000)["x"]
    y = empty_f32(10000, 32)
    cf.cf_stitch_layernorm(d32(x), y, unfused=True)
    assert rownorm_err(host(y), oracle.layernorm_rows(x)) <= TOL_F32
    d = gen.pow_bcast_add_inputs(seed=3)
    y, yp = empty_f32(64, 30000), empty_f32(64, 30000)
    cf.cf_stitch_pow_bcast_add(d32(d["x"]), d32(d["v"]), 1.5, y, yp, unfused=True)
    o, oy = oracle.pow_bcast_add_softmax(d["x"], d["v"], 1.5)
    assert rownorm_err(host(y), o) <= TOL_F32 and rownorm_err(host(yp), oy) <= TOL_F32
    g = gen.gemm_ln_inputs(seed=4, M=512, N=1024, K=256)
    o = oracle.gemm_ln(g["a"], g["w"], g["bias"], g["r"], g["gamma"], g["beta"])
    assert rownorm_err(_gemm_ln_run(g, 512, 1024, 256, unfused=True), o) <= TOL_BF16
    q = gen.gemm_softmax_inputs(seed=5, M=512, N=1024, D=128)
    o = oracle.gemm_softmax(q["q"], q["k"], q["scale"])
    assert rownorm_err(_gemm_sm_run(q, 512, 1024, 128, unfused=True), o) <= TOL_BF16


def test_graph_replay_is_bitwise_equal_to_stream_launch():
    d = gen.gemm_softmax_inputs(seed=5, M=512, N=1024, D=128)
    Q, K = dbf16(d["q_bits"]), dbf16(d["k_bits"])
    S1 = torch.empty((512, 1024), dtype=torch.bfloat16, device="cuda")
    S2 = torch.zeros_like(S1)
    ws = cf.Workspace(cf.cf_unfused_workspace_bytes(cf.CF_OP_GEMM_SOFTMAX, 512, 1024, 128))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        cf.cf_gemm_softmax(Q, K, d["scale"], S1, ws=ws, unfused=True)
        s.synchronize()
        cf.cf_graph_begin()
        cf.cf_gemm_softmax(Q, K, d["scale"], S2, ws=ws, unfused=True)
        h = cf.cf_graph_end()
        for _ in range(3):
            S2.zero_()
            cf.cf_graph_launch(h)
            s.synchronize()
            assert torch.equal(S1, S2)
        cf.cf_graph_destroy(h)


def test_one_workspace_shared_by_every_op():
    """Any later call of any op accepts a workspace earlier calls left behind."""
    big = max(cf.cf_workspace_bytes(op, *dims) for op, dims in [
        (cf.CF_OP_STITCH_SOFTMAX, (4, 20000, 0)), (cf.CF_OP_STITCH_LAYERNORM, (3, 70001, 0)),
        (cf.CF_OP_STITCH_POW_BCAST_ADD, (64, 30000, 0)), (cf.CF_OP_GEMM_LN, (512, 1024, 128)),
        (cf.CF_OP_GEMM_SOFTMAX, (512, 1024, 128))])
    ws = cf.Workspace(big)
    s = gen.softmax_inputs(seed=1, rows=4, cols=20000)["x"]
    l = gen.layernorm_inputs(seed=2, rows=3, cols=70001)["x"]
    p = gen.pow_bcast_add_inputs(seed=3)
    g = gen.gemm_ln_inputs(seed=4, M=512, N=1024, K=128)
    q = gen.gemm_softmax_inputs(seed=5, M=512, N=1024, D=128)
    og = oracle.gemm_ln(g["a"], g["w"], g["bias"], g["r"], g["gamma"], g["beta"])
    oq = oracle.gemm_softmax(q["q"], q["k"], q["scale"])
    for _ in range(2):
        for step in range(5):
            if step == 0:
                y = empty_f32(4, 20000)
                cf.cf_stitch_softmax(d32(s), y, ws=ws)
                err = rownorm_err(host(y), oracle.softmax_rows(s))
            elif step == 1:
                Y = torch.empty((512, 1024), dtype=torch.bfloat16, device="cuda")
                cf.cf_gemm_ln(dbf16(g["a_bits"]), dbf16(g["w_bits"]), d32(g["bias"]), dbf16(g["r_bits"]),
                              d32(g["gamma"]), d32(g["beta"]), Y, ws=ws)
                err = rownorm_err(host(Y), og) / TOL_BF16 * TOL_F32
            elif step == 2:
                y = empty_f32(3, 70001)
                cf.cf_stitch_layernorm(d32(l), y, ws=ws)
                err = rownorm_err(host(y), oracle.layernorm_rows(l))
            elif step == 3:
                S = torch.empty((512, 1024), dtype=torch.bfloat16, device="cuda")
                cf.cf_gemm_softmax(dbf16(q["q_bits"]), dbf16(q["k_bits"]), q["scale"], S, ws=ws)
                err = rownorm_err(host(S), oq) / TOL_BF16 * TOL_F32
            else:
                y = empty_f32(64, 30000)
                cf.cf_stitch_pow_bcast_add(d32(p["x"]), d32(p["v"]), 1.5, y, ws=ws)
                err = rownorm_err(host(y), oracle.pow_bcast_add_softmax(p["x"], p["v"], 1.5)[0])
            assert ws.error_word() == 0, f"step {step}: a join gave up"
            assert err <= TOL_F32, (step, err)


def test_single_row_and_minimal_gemms(monkeypatch):
    """One output row (and the smallest legal N, K) through every fused GEMM."""
    for M, N, K in [(1, 8, 8), (1, 264, 72), (2, 136, 1032)]:
        d = gen.gemm_ln_inputs(seed=71, M=M, N=N, K=K)
        assert rownorm_err(_gemm_ln_run(d, M, N, K), oracle.gemm_ln(d["a"], d["w"], d["bias"], d["r"], d["gamma"],
                                                                   d["beta"], d["eps"])) <= TOL_BF16
        q = gen.gemm_softmax_inputs(seed=72, M=M, N=N, D=K)
        assert rownorm_err(_gemm_sm_run(q, M, N, K), oracle.gemm_softmax(q["q"], q["k"], q["scale"])) <= TOL_BF16
        for algo in (0, 1):
            monkeypatch.setenv("CF_GEMM_ACT_ALGO", str(algo))
            g = gen.gemm_act_inputs(seed=73, M=M, N=N, K=K)
            assert act_err(_gemm_act_run(g, M, N, "silu"), oracle.gemm_act(g["a"], g["w"], g["bias"], "silu")) <= 1.0
        if K <= 128:
            b = gen.gemm_softmax_gemm_inputs(seed=74, M=M, N=N, D=K, Dv=8)
            assert rownorm_err(_b2b_run(b, M, N, K, 8), oracle.gemm_softmax_gemm(b["q"], b["k"], b["v"], b["scale"])) \
                <= TOL_BF16


@pytest.mark.parametrize("M,N,K", [(1024, 4096, 1024), (2048, 2048, 2048)])
def test_gemm_ln_small_grid_takes_the_128_tiles(M, N, K):
    """Fewer 256 x 256 tiles than half the CUs: the planner takes 128 x 128 tiles at two
    workgroups per CU (the large tiles would leave most CUs idle); parity against the oracle."""
    d = gen.gemm_ln_inputs(seed=13, M=M, N=N, K=K)
    g = _gemm_ln_run(d, M, N, K)
    p = json.loads(cf.last_plan())
    assert p["kernel"] == "k_gemm_ln2" and p["tile"][:2] == [128, 128], p
    o = oracle.gemm_ln(d["a"], d["w"], d["bias"], d["r"], d["gamma"], d["beta"], d["eps"])
    assert rownorm_err(g, o) <= TOL_BF16, cf.last_plan()


def test_gemm_act_small_grid_takes_the_128_tiles():
    """Fewer 256 x 256 tiles than three quarters of the CUs: the planner takes the 128 x 128
    kernel at two workgroups per CU; parity against the oracle."""
    M, N, K = 1024, 4096, 1024
    d = _act_inputs("gelu_tanh", 59, M, N, K)
    g = _gemm_act_run(d, M, N, "gelu_tanh")
    plan = json.loads(cf.last_plan())
    assert plan["kernel"] == "k_gemm" and plan["tile"][:2] == [128, 128], plan
    o = oracle.gemm_act(d["a"], d["w"], d["bias"], "gelu_tanh")
    assert act_err(g, o) <= 1.0, act_err(g, o)


@pytest.mark.parametrize("M,N,D", [(4096, 4096, 128), (8192, 2048, 128)])
def test_gemm_softmax_strips_hold_four_tiles(M, N, D):
    """The strip planner keeps at least four 128-column tiles per strip (fewer, longer strips
    where the rows would allow more); parity against the oracle on sampled rows."""
    d = gen.gemm_softmax_inputs(seed=14, M=M, N=N, D=D)
    g = _gemm_sm_run(d, M, N, D)
    p = json.loads(cf.last_plan())
    assert p["kernel"] == "k_gemm_sm3" and p["row_group"] == N // 128 // 4, p
    rows = np.arange(0, M, 37)
    o = oracle.gemm_softmax(np.asarray(d["q"])[rows], d["k"], d["scale"])
    assert rownorm_err(g[rows], o) <= TOL_BF16, cf.last_plan()
