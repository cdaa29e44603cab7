"""The oracle against closed forms, invariants, library routines and brute force (CPU only)."""
import pytest

from tests import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


def test_every_subgraph_is_pinned():
    names = {p.__name__ for p in pins.ALL_PINS}
    for prefix in ["pin_softmax", "pin_layernorm", "pin_pow", "pin_gemm_ln", "pin_gemm_softmax", "pin_b2b", "pin_rmsnorm",
                   "pin_layernorm_affine", "pin_gemm_act"]:
        assert any(n.startswith(prefix) for n in names), prefix
