"""The seeded input generator: determinism, distributions and bf16 rounding (CPU only)."""
import numpy as np
import torch

import gen


def test_deterministic_and_independent_streams():
    a = gen.normal(7, 0, (1000,))
    b = gen.normal(7, 0, (1000,))
    c = gen.normal(7, 1, (1000,))
    assert np.array_equal(a, b)
    assert not np.array_equal(a, c)
    assert a.dtype == np.float32


def test_distributions():
    z = gen.normal(1, 0, (200000,), mean=1.0, std=0.1).astype(np.float64)
    assert abs(z.mean() - 1.0) < 2e-3 and abs(z.std() - 0.1) < 2e-3
    u = gen.uniform(2, 0, (200000,), -1.0, 1.0).astype(np.float64)
    assert u.min() >= -1.0 and u.max() < 1.0
    assert abs(u.mean()) < 1e-2 and abs(u.var() - 1.0 / 3.0) < 1e-2


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(1 << 20) * np.exp2(rng.integers(-40, 40, 1 << 20))).astype(np.float32)
    # ties: low 16 bits exactly 0x8000, both parities of the kept lsb
    ties = (np.arange(4096, dtype=np.uint32) << np.uint32(16)) | np.uint32(0x8000)
    ties = ties.view(np.float32)
    ties = ties[np.isfinite(ties)]
    for arr in (x, ties):
        ours = gen.f32_to_bf16_bits(arr)
        ref = torch.from_numpy(arr).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(ours, ref)
        back = gen.bf16_bits_to_f32(ours)
        assert np.array_equal(back, torch.from_numpy(arr).to(torch.bfloat16).float().numpy())


def test_workload_shapes():
    d = gen.softmax_inputs(rows=4, cols=9)
    assert d["x"].shape == (4, 9)
    d = gen.pow_bcast_add_inputs(rows=3, cols=11)
    assert d["v"].shape == (3,) and d["x"].shape == (3, 11)
    assert d["v"].min() >= 0.1 and d["v"].max() < 2.0
    d = gen.gemm_ln_inputs(M=16, N=32, K=8)
    assert d["a_bits"].shape == (16, 8) and d["w_bits"].shape == (8, 32) and d["r_bits"].shape == (16, 32)
    assert np.array_equal(gen.bf16_bits_to_f32(d["a_bits"]), d["a"])
    d = gen.gemm_softmax_inputs(M=8, N=16, D=4)
    assert d["k_bits"].shape == (16, 4)
    assert d["scale"] == float(np.float32(0.5))
    d = gen.gemm_softmax_gemm_inputs(M=8, N=16, D=4, Dv=12)
    assert d["q_bits"].shape == (8, 4) and d["k_bits"].shape == (16, 4) and d["v_bits"].shape == (16, 12)
    assert np.array_equal(gen.bf16_bits_to_f32(d["v_bits"]), d["v"])
    assert d["scale"] == float(np.float32(0.5))
    d = gen.rmsnorm_inputs(rows=5, cols=7)
    assert d["x"].shape == (5, 7) and d["gamma"].shape == (7,) and d["x"].dtype == np.float32
    d = gen.layernorm_affine_inputs(rows=5, cols=7)
    assert d["gamma"].shape == (7,) and d["beta"].shape == (7,)
    d = gen.gemm_act_inputs(M=16, N=24, K=8)
    assert d["a_bits"].shape == (16, 8) and d["w_bits"].shape == (8, 24) and d["bias"].shape == (24,)


def test_gemm_act_positive_inputs_are_positive():
    d = gen.gemm_act_inputs(M=16, N=24, K=8, positive=True)
    assert d["a"].min() >= 0.5 and d["w"].min() >= 0.0 and d["bias"].min() >= 0.0
    assert d["a"].max() <= 1.5 and d["w"].max() <= 0.02
