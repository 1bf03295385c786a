"""Comparison rules between the HIP path and the fp64 oracle.

fp32 (relative 1e-4, absolute 1e-5):
  * routing outputs (expert_idx, counts, offsets, perm): bit-exact;
  * frac: counts / T within one fp32 ulp;
  * routed_ctx, d_fused_ctx, loss, mean_prob, probs: elementwise |g - o| <= 1e-5 + 1e-4 |o|;
  * d_W, d_b: sums over up to ~1e5 tokens with random signs, where fp32 rounding of any
    summation order grows with sqrt(count) * |terms| rather than with |o|; elementwise
    |g - o| <= 1e-5 s + 1e-4 max(|o|, s), s = RMS of the oracle's slice for that expert;
  * d_gate_logits: its entries are of order lambda N_E / T (far below 1e-5), so the
    comparison is made on dG * T / (lambda N_E) with the elementwise rule.
bf16 storage: every float output within 2e-2 max(|o|, s).
"""
from __future__ import annotations

import numpy as np

RTOL, ATOL = 1e-4, 1e-5
BF16_TOL = 2e-2


def _report(name, bad, err):
    return f"{name}: {int(bad.sum())} of {bad.size} outside tolerance, max err {float(np.max(err)) if err.size else 0:.3e}"


def elementwise(name, g, o, rtol=RTOL, atol=ATOL):
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    assert g.shape == o.shape, f"{name}: shape {g.shape} vs {o.shape}"
    assert np.isfinite(g).all(), f"{name}: non-finite values in GPU output"
    err = np.abs(g - o)
    bad = ~(err <= atol + rtol * np.abs(o))
    assert not bad.any(), _report(name, bad, err)


def per_expert_scaled(name, g, o, rtol=RTOL, atol=ATOL):
    """d_W [N_E, H, H] / d_b [N_E, H]: tolerance scaled by each expert slice's RMS."""
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    assert g.shape == o.shape, f"{name}: shape {g.shape} vs {o.shape}"
    assert np.isfinite(g).all(), f"{name}: non-finite values in GPU output"
    for e in range(o.shape[0]):
        s = float(np.sqrt(np.mean(o[e] ** 2)))
        err = np.abs(g[e] - o[e])
        bad = ~(err <= atol * s + rtol * np.maximum(np.abs(o[e]), s))
        assert not bad.any(), _report(f"{name}[expert {e}]", bad, err)


def bf16_scaled(name, g, o, tol=BF16_TOL, per_expert=False):
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    assert g.shape == o.shape, f"{name}: shape {g.shape} vs {o.shape}"
    assert np.isfinite(g).all(), f"{name}: non-finite values in GPU output"
    slices = [(slice(None),)] if not per_expert else [(e,) for e in range(o.shape[0])]
    for sl in slices:
        s = float(np.sqrt(np.mean(o[sl] ** 2))) if o[sl].size else 0.0
        err = np.abs(g[sl] - o[sl])
        bad = ~(err <= tol * np.maximum(np.abs(o[sl]), s))
        assert not bad.any(), _report(f"{name}{sl}", bad, err)


def frac_ulp(name, g, counts, T):
    g = np.asarray(g, dtype=np.float32)
    ref = (np.asarray(counts, dtype=np.float64) / T)
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    err = np.abs(g.astype(np.float64) - ref)
    bad = ~(err <= ulp)
    assert not bad.any(), _report(name, bad, err)


def exact(name, g, o):
    g = np.asarray(g)
    o = np.asarray(o)
    assert g.shape == o.shape, f"{name}: shape {g.shape} vs {o.shape}"
    if not np.array_equal(g, o):
        bad = g != o
        first = np.argwhere(bad)[:5].tolist()
        raise AssertionError(f"{name}: {int(bad.sum())} of {bad.size} differ; first at {first}")
