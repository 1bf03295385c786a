"""The CPU oracle against what the pages and the mathematics fix (no GPU)."""
import numpy as np
import pytest

import workloads
from oracle import moe_oracle
from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(moe_oracle)


def test_workload_recipe_is_reproducible():
    wl = workloads.workload(1)
    a = workloads.make_inputs(wl)
    b = workloads.make_inputs(wl)
    for k in ("fused_ctx", "gate_logits", "W", "b", "d_out"):
        assert np.array_equal(getattr(a, k), getattr(b, k))
    assert a.fused_ctx.dtype == np.float32 and a.fused_ctx.shape == (64, 5, 128)
    assert set(np.unique(a.gate_logits)) <= {-2.0, -1.0, 0.0, 1.0, 2.0}


def test_tiny_ref_tie_rate():
    """Integer logits in {-2..2} over 4 experts tie at the max with probability 0.36."""
    inp = workloads.make_inputs(workloads.workload(1))
    G = inp.gate_logits.reshape(-1, 4)
    ties = ((G == G.max(axis=1, keepdims=True)).sum(axis=1) > 1).mean()
    assert 0.25 < ties < 0.47


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 3.0e-5], dtype=np.float32)
    bits = workloads.f32_to_bf16_bits(x)
    back = workloads.bf16_bits_to_f32(bits)
    assert back[0] == 1.0
    assert back[1] == 1.0            # tie -> even mantissa
    assert back[2] == 1.0 + 2 ** -6  # tie -> even (rounds up)
    assert back[3] == 1.0
    assert back[4] == -2.5
    assert abs(back[5] - 3.0e-5) <= 3.0e-5 * 2 ** -8


def test_imbalanced_skew_matches_pages():
    """The skewed workload reproduces the routing skew reported for the adaptive-lambda
    page (one expert near 80 %, the other seven under 5 % each)."""
    wl = workloads.workload(3, B=2048)
    inp = workloads.make_inputs(wl)
    idx = moe_oracle.route(inp.gate_logits, 8)
    share = np.bincount(idx, minlength=8) / idx.size
    assert 0.75 < share[4] < 0.9
    assert (np.delete(share, 4) < 0.05).all()
