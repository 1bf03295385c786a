"""Pins for the oracles of reduce_axis0, the horizon mean collapse and the softmax-CE head (CPU)."""
import json
import math
import os

import numpy as np
import pytest

from oracle import next_rows as N

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "softmax_ce_worked.json")


# ---------------------------------------------------------------- reduce_axis0
def test_reduce_axis0_brute_and_invariants():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((37, 11))
    brute = [sum(x[r, j] for r in range(37)) for j in range(11)]
    assert np.allclose(N.reduce_axis0(x), brute, rtol=0, atol=1e-12)
    assert np.array_equal(N.reduce_axis0(np.ones((5, 3))), [5.0, 5.0, 5.0])
    assert np.array_equal(N.reduce_axis0(x[:1]), x[0])                  # one row: identity
    # the MoE use: per-token dW scratch [T, N_E, H, H] collapses to the expert dW
    T, NE, H = 6, 2, 3
    idx = np.array([0, 1, 1, 0, 1, 1])
    dy, xx = rng.standard_normal((T, H)), rng.standard_normal((T, H))
    scratch = np.zeros((T, NE, H, H))
    for t in range(T):
        scratch[t, idx[t]] = np.outer(dy[t], xx[t])
    dW = N.reduce_axis0(scratch.reshape(T, -1)).reshape(NE, H, H)
    assert np.allclose(dW[1], dy[idx == 1].T @ xx[idx == 1])


# ---------------------------------------------------------------- horizon mean collapse
def test_horizon_mean_brute_and_adjoint():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 5, 4))
    brute = [[sum(x[b, h, k] for h in range(5)) / 5 for k in range(4)] for b in range(3)]
    assert np.allclose(N.horizon_mean_fwd(x), brute, atol=1e-15)
    d = rng.standard_normal((3, 4))
    # adjoint identity <fwd(x), d> = <x, bwd(d)>
    assert abs(np.sum(N.horizon_mean_fwd(x) * d) - np.sum(x * N.horizon_mean_bwd(d, 5))) < 1e-12
    assert np.allclose(N.horizon_mean_fwd(np.ones((2, 7, 3)) * 2.5), 2.5)


# ---------------------------------------------------------------- softmax-CE head
def test_softmax_ce_uniform_logits_page_value():
    g = json.load(open(GOLDEN))
    A = g["A"]
    logits = np.full((4, 5, A), 0.37)
    labels = np.arange(20).reshape(4, 5) % A
    ce, grad = N.softmax_ce(logits, labels)
    assert np.allclose(ce, math.log(A), atol=1e-14)
    assert abs(round(float(ce[0, 0]), g["uniform_ce_printed_decimals"]) - g["uniform_ce"]) < 1e-12
    assert np.abs(grad.sum(axis=-1)).max() < 1e-15


def test_softmax_ce_rowsum_sentinel_and_floor():
    rng = np.random.default_rng(2)
    logits = rng.standard_normal((6, 3, 21)) * 4
    labels = rng.integers(0, 21, size=(6, 3))
    labels[2, 1] = -1
    ce, grad = N.softmax_ce(logits, labels)
    assert np.abs(grad.sum(axis=-1)).max() < 1e-15
    assert ce[2, 1] == 0.0 and np.all(grad[2, 1] == 0.0)
    # label logit far below the others: p underflows and the 1e-30 floor caps the loss
    z = np.zeros((1, 1, 21)); z[0, 0, 3] = -2000.0
    ce2, _ = N.softmax_ce(z, np.array([[3]]))
    assert abs(ce2[0, 0] - 30 * math.log(10)) < 1e-9


def test_softmax_ce_central_fd():
    rng = np.random.default_rng(3)
    B, NH, A = 3, 2, 21
    logits = rng.standard_normal((B, NH, A))
    labels = rng.integers(0, A, size=(B, NH))
    labels[1, 0] = -1
    _, grad = N.softmax_ce(logits, labels)
    eps = 1e-6

    def loss(z):
        return N.softmax_ce(z, labels)[0].sum() / B   # the loss whose gradient is the head's grad

    fd = np.zeros_like(logits)
    for ix in np.ndindex(logits.shape):
        zp = logits.copy(); zp[ix] += eps
        zm = logits.copy(); zm[ix] -= eps
        fd[ix] = (loss(zp) - loss(zm)) / (2 * eps)
    assert np.allclose(grad, fd, rtol=1e-6, atol=1e-9)


def test_softmax_ce_brute_small():
    logits = np.array([[[1.0, 2.0, 0.5]], [[-1.0, -1.0, 3.0]]])
    labels = np.array([[1], [0]])
    ce, grad = N.softmax_ce(logits, labels)
    for b in range(2):
        z = logits[b, 0]
        p = [math.exp(v - max(z)) for v in z]
        s = sum(p)
        p = [v / s for v in p]
        assert abs(ce[b, 0] + math.log(p[labels[b, 0]])) < 1e-14
        for a in range(3):
            assert abs(grad[b, 0, a] - (p[a] - (a == labels[b, 0])) / 2) < 1e-15
