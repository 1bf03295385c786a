"""Pins of the adaptive-lambda oracle against the page's worked example and regimes (CPU)."""
import json
import math
import os

import pytest

from oracle import lambda_controller as L

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "lambda_controller_worked.json")


def test_page_worked_example():
    g = json.load(open(GOLDEN))
    for row in g["printed"]:
        lam = L.lambda_eff(row["ent_ema"], g["K"], g["floor"], g["max_extra"], g["target_frac"])
        # printed to 3 significant digits: agree to half a unit in the last printed place
        assert abs(lam - row["lambda_eff"]) <= 0.5e-4, (row, lam)


def test_regimes():
    K = 8
    tgt = L.entropy_target(K)
    assert abs(tgt - 0.7 * math.log(8)) < 1e-15
    assert L.lambda_eff(math.log(K), K) == L.FLOOR                    # deeply above target (bootstrap ln K)
    assert L.lambda_eff(tgt + 0.1, K) == L.FLOOR                      # above target
    assert L.lambda_eff(tgt, K) == L.FLOOR                            # at target
    assert abs(L.lambda_eff(tgt / 2, K) - (L.FLOOR + L.MAX_EXTRA / 2)) < 1e-15   # half collapse
    assert abs(L.lambda_eff(0.0, K) - (L.FLOOR + L.MAX_EXTRA)) < 1e-15          # full collapse


def test_monotone_non_increasing_in_entropy():
    vals = [L.lambda_eff(e / 100.0, 8) for e in range(0, 300)]
    assert all(a >= b for a, b in zip(vals, vals[1:]))
    assert min(vals) == L.FLOOR and max(vals) == pytest.approx(L.FLOOR + L.MAX_EXTRA)
