"""The allocation-free GEMM + LayerNorm entry point (cf_gemm_ln_noalloc), through the C-ABI, against
cf_gemm_ln on the same inputs: two calls in a row, the second on a smaller shape, each bit-equal to
the workspace entry point and within the bf16 tolerance of the fp64 oracle; and the refusal of a
shape whose partials exceed the static scratch."""
import numpy as np
import pytest
import torch

import broadcast_subgraphs_amd as cf
import gen
import oracle
from tests.test_gpu_parity import TOL_BF16, d32, dbf16, host, rownorm_err

pytestmark = pytest.mark.gpu


def _args(d, M, N):
    return (dbf16(d["a_bits"]), dbf16(d["w_bits"]), d32(d["bias"]), dbf16(d["r_bits"]), d32(d["gamma"]),
            d32(d["beta"]))


def test_noalloc_matches_workspace_entry_point_twice():
    for seed, (M, N, K) in ((301, (2048, 4096, 1024)), (302, (300, 264, 72))):
        d = gen.gemm_ln_inputs(seed=seed, M=M, N=N, K=K)
        args = _args(d, M, N)
        y_ws = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        cf.cf_gemm_ln(*args, y_ws, eps=d["eps"])
        y_na = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        cf.cf_gemm_ln_noalloc(*args, y_na, eps=d["eps"])
        got = host(y_na)
        assert np.array_equal(got, host(y_ws)), (M, N, K)
        o = oracle.gemm_ln(d["a"], d["w"], d["bias"], d["r"], d["gamma"], d["beta"], d["eps"])
        assert rownorm_err(got, o) <= TOL_BF16, (M, N, K)


def test_noalloc_refuses_shapes_beyond_the_scratch():
    M, N, K = 131072, 4096, 64  # M x (N / 128) x 16 bytes of partials: 64 MiB > 16 MiB
    A = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    W = torch.empty((K, N), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros(N, dtype=torch.float32, device="cuda")
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(cf.CFError) as e:
        cf.cf_gemm_ln_noalloc(A, W, v, None, v, v, Y)
    assert e.value.status == cf.CF_EWORKSPACE
    torch.cuda.synchronize()
    assert torch.isnan(Y[:4096]).all()
