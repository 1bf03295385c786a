"""The comparison rules themselves (CPU): they accept rounding and reject real errors."""
import numpy as np
import pytest

from tests import compare as C


def test_elementwise_accepts_rounding_rejects_errors():
    o = np.linspace(-3, 3, 101)
    C.elementwise("ok", o.astype(np.float32), o)
    with pytest.raises(AssertionError):
        C.elementwise("bad", o + 1e-3, o)
    with pytest.raises(AssertionError):
        C.elementwise("nan", np.where(o > 0, np.nan, o), o)


def test_per_expert_scaled_tolerates_cancellation():
    rng = np.random.default_rng(0)
    o = rng.standard_normal((2, 16, 16)) * 100
    o[0, 0, 0] = 1e-9  # a cancelled entry: absolute error at the slice's scale is fine
    g = o.copy()
    g[0, 0, 0] = 1e-3
    C.per_expert_scaled("dW", g, o)
    g[1, 3, 3] += 0.5  # a real error
    with pytest.raises(AssertionError):
        C.per_expert_scaled("dW", g, o)


def test_frac_ulp_and_exact():
    C.frac_ulp("frac", np.float32([0.25, 0.5, 0.25]), [1, 2, 1], 4)
    with pytest.raises(AssertionError):
        C.frac_ulp("frac", np.float32([0.2500001, 0.5, 0.25]), [1, 2, 1], 4)
    with pytest.raises(AssertionError):
        C.exact("perm", np.array([0, 2, 1]), np.array([0, 1, 2]))
