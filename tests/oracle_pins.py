"""Pins that tie the CPU oracle to the mathematics, written over an implementation.

Each ``pin_*`` takes an object with the oracle's functions (route, group, forward,
backward, backward_entries, aux, softmax) and raises AssertionError when it disagrees with a value
that the pages or the mathematics fix.  tests/test_oracle.py runs them against the
oracle; tests/test_oracle_mutants.py runs them against copies of the oracle with a
planted mistake and checks that some pin fails.

Pages cited: the MoE-gate commit page "11b96dac6a" (summary, ARCHITECTURE,
PERFORMANCE, NUMGRAD blocks) and the softmax/cross-entropy page "6cfd7e6691"
(its analytic oracles: uniform logits give a closed form, softmax-gradient rows
sum to zero, central finite differences).
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch

import workloads
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, rtol=1e-12, atol=1e-12, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.isfinite(a).all(), f"{what}: non-finite values"
    err = np.abs(a - b)
    bad = ~(err <= atol + rtol * np.abs(b))
    assert not bad.any(), f"{what}: {bad.sum()} mismatches, max err {err.max():.3e}"


def _tiny(seed, B=2, NH=3, H=4, NE=3, ints=False):
    r = _rng(seed)
    X = r.standard_normal((B, NH, H))
    if ints:
        G = r.integers(-2, 3, size=(B, NH, NE)).astype(np.float64)
    else:
        G = r.standard_normal((B, NH, NE))
    W = r.uniform(-1, 1, (NE, H, H))
    b = r.uniform(-1, 1, (NE, H))
    dY = r.standard_normal((B, NH, H))
    return X, G, W, b, dY


# ---------------------------------------------------------------- routing / grouping

def pin_route_first_occurrence(impl):
    """Top-1 with lowest-index ties equals numpy's first-occurrence argmax."""
    G = _rng(1).integers(-2, 3, size=(4000, 5)).astype(np.float64)
    got = impl.route(G, 5)
    assert np.array_equal(got, np.argmax(G, axis=1)), "route != first-occurrence argmax"
    ties = (G == G.max(axis=1, keepdims=True)).sum(axis=1) > 1
    assert ties.mean() > 0.3, "fixture should hold many ties"


def pin_route_all_ties(impl):
    G = np.full((7, 6), 0.25)
    assert (impl.route(G, 6) == 0).all(), "all-tie rows must pick expert 0"
    G = np.array([[0.0, 3.0, 1.0, 3.0], [5.0, 1.0, 5.0, 5.0], [-1.0, -2.0, -3.0, -1.0]])
    assert list(impl.route(G, 4)) == [1, 0, 0]


def pin_route_brute(impl):
    inp = workloads.make_inputs(workloads.workload(1))
    G = inp.gate_logits.reshape(-1, 4)
    assert list(impl.route(G, 4)) == brute.route(G.tolist())


def pin_group(impl):
    idx = _rng(2).integers(0, 6, size=3001).astype(np.int32)
    idx[idx == 3] = 5  # expert 3 empty
    counts, offsets, perm = impl.group(idx, 6)
    assert np.array_equal(counts, np.bincount(idx, minlength=6))
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(np.sort(perm), np.arange(idx.size)), "perm is not a permutation"
    ref = np.lexsort((np.arange(idx.size), idx))  # by expert, then by token
    assert np.array_equal(perm, ref), "perm is not the stable by-expert order"
    bc, bo, bp = brute.group(idx.tolist(), 6)
    assert list(counts) == bc and list(offsets) == bo and list(perm) == bp


# ---------------------------------------------------------------- forward

def _linear(x, w, b):
    return torch.nn.functional.linear(torch.from_numpy(x), torch.from_numpy(w),
                                      torch.from_numpy(b)).numpy()


def pin_fwd_single_expert_is_linear(impl):
    """N_E = 1 reduces the gate to one dense linear layer, y = W x + b."""
    X, G, W, b, _ = _tiny(3, B=5, NH=4, H=8, NE=1)
    Y = impl.forward(X, G, W, b).routed_ctx
    _close(Y, _linear(X.reshape(-1, 8), W[0], b[0]), what="N_E=1 vs F.linear")


def pin_fwd_identity(impl):
    X, G, _, _, _ = _tiny(4, H=6, NE=3)
    W = np.stack([np.eye(6)] * 3)
    Y = impl.forward(X, G, W, np.zeros((3, 6))).routed_ctx
    _close(Y, X.reshape(-1, 6), what="W=I, b=0")


def pin_fwd_select_dense(impl):
    """Every expert applied densely, then the top-1 one selected per token."""
    X, G, W, b, _ = _tiny(5, B=3, NH=5, H=6, NE=4)
    Xf = X.reshape(-1, 6)
    dense = np.stack([_linear(Xf, W[e], b[e]) for e in range(4)], axis=1)  # [T, NE, H]
    pick = np.argmax(G.reshape(-1, 4), axis=1)
    _close(impl.forward(X, G, W, b).routed_ctx, dense[np.arange(Xf.shape[0]), pick], what="select")


def pin_fwd_brute(impl):
    X, G, W, b, _ = _tiny(6, ints=True)
    f = impl.forward(X, G, W, b)
    idx, Y = brute.forward(X.reshape(-1, 4).tolist(), G.reshape(-1, 3).tolist(), W.tolist(), b.tolist())
    assert list(f.expert_idx) == idx
    _close(f.routed_ctx, Y, what="fwd vs brute")


def pin_golden_worked_example(impl):
    with open(os.path.join(GOLDEN, "tiny_gate_worked.json")) as fh:
        g = json.load(fh)
    X, G, W, b, dY = (np.array(g[k], dtype=np.float64) for k in ("fused_ctx", "gate_logits", "W", "b", "d_out"))
    ex = g["expected"]
    f = impl.forward(X, G, W, b)
    assert list(f.expert_idx) == ex["expert_idx"]
    assert list(f.counts) == ex["counts"] and list(f.offsets) == ex["offsets"] and list(f.perm) == ex["perm"]
    _close(f.routed_ctx, ex["routed_ctx"], what="golden routed_ctx")
    bw = impl.backward(dY, X, W, f.expert_idx)
    _close(bw.d_fused_ctx, ex["d_fused_ctx"], what="golden d_fused_ctx")
    _close(bw.d_W, ex["d_W"], what="golden d_W")
    _close(bw.d_b, ex["d_b"], what="golden d_b")


# ---------------------------------------------------------------- backward

def _loss_exp(impl, X, G, W, b, dY):
    return float(np.sum(dY.reshape(-1, W.shape[1]) * impl.forward(X, G, W, b).routed_ctx))


def pin_bwd_central_fd(impl):
    """L = sum(dY * Y) is linear in W, b, X, so central differences equal the
    analytic gradients up to rounding (a stricter form of the page's numgrad check)."""
    X, G, W, b, dY = _tiny(7)
    f = impl.forward(X, G, W, b)
    bw = impl.backward(dY, X, W, f.expert_idx)
    eps = 1e-6

    def fd(arr, setter):
        out = np.zeros_like(arr)
        for ix in np.ndindex(arr.shape):
            a = arr.copy(); a[ix] += eps
            lp = _loss_exp(impl, *setter(a))
            a[ix] -= 2 * eps
            lm = _loss_exp(impl, *setter(a))
            out[ix] = (lp - lm) / (2 * eps)
        return out

    _close(bw.d_W, fd(W, lambda a: (X, G, a, b, dY)), rtol=1e-6, atol=1e-7, what="FD dW")
    _close(bw.d_b, fd(b, lambda a: (X, G, W, a, dY)), rtol=1e-6, atol=1e-7, what="FD db")
    _close(bw.d_fused_ctx.reshape(X.shape), fd(X, lambda a: (a, G, W, b, dY)), rtol=1e-6, atol=1e-7, what="FD dX")


def pin_bwd_single_expert_autograd(impl):
    """N_E = 1: textbook dense-linear backward via torch autograd in fp64."""
    X, G, W, b, dY = _tiny(8, B=4, NH=3, H=5, NE=1)
    x = torch.from_numpy(X.reshape(-1, 5)).requires_grad_()
    w = torch.from_numpy(W[0].copy()).requires_grad_()
    bb = torch.from_numpy(b[0].copy()).requires_grad_()
    torch.nn.functional.linear(x, w, bb).backward(torch.from_numpy(dY.reshape(-1, 5)))
    bw = impl.backward(dY, X, W, impl.route(G, 1))
    _close(bw.d_fused_ctx, x.grad.numpy(), what="autograd dX")
    _close(bw.d_W[0], w.grad.numpy(), what="autograd dW")
    _close(bw.d_b[0], bb.grad.numpy(), what="autograd db")


def pin_bwd_inactive_zero(impl):
    X, G, W, b, dY = _tiny(9, B=4, NH=5, H=4, NE=4)
    G[..., 2] = -1e6
    bw = impl.backward(dY, X, W, impl.route(G, 4))
    assert np.all(bw.d_W[2] == 0.0) and np.all(bw.d_b[2] == 0.0), "inactive expert must get exact zeros"
    assert not np.signbit(bw.d_W[2]).any() and not np.signbit(bw.d_b[2]).any(), "zeros must be +0.0"


def pin_bwd_accumulate(impl):
    X, G, W, b, dY = _tiny(10)
    idx = impl.route(G, 3)
    prev = _rng(11).standard_normal((6, 4))
    a = impl.backward(dY, X, W, idx).d_fused_ctx
    c = impl.backward(dY, X, W, idx, prev).d_fused_ctx
    _close(c, a + prev, what="accumulate dX")


def pin_bwd_brute(impl):
    X, G, W, b, dY = _tiny(12, ints=True)
    idx = impl.route(G, 3)
    bw = impl.backward(dY, X, W, idx)
    dX, dW, db = brute.backward(dY.reshape(-1, 4).tolist(), X.reshape(-1, 4).tolist(), W.tolist(), list(idx))
    _close(bw.d_fused_ctx, dX, what="brute dX")
    _close(bw.d_W, dW, what="brute dW")
    _close(bw.d_b, db, what="brute db")


def pin_bwd_entries_brute(impl):
    """Selected d_W / d_b entries equal the loop-only oracle's, empty expert included."""
    X, G, W, b, dY = _tiny(13, B=3, NH=4, H=5, NE=4, ints=True)
    G[..., 3] = -10.0  # expert 3 gets no tokens
    idx = impl.route(G, 4)
    _, dW, db = brute.backward(dY.reshape(-1, 5).tolist(), X.reshape(-1, 5).tolist(), W.tolist(), list(idx))
    dW, db = np.array(dW), np.array(db)
    rows, cols = [4, 0, 2], [1, 3]
    for e in range(4):
        w, bb = impl.backward_entries(dY.reshape(-1, 5)[:, rows], X.reshape(-1, 5)[:, cols], idx, e)
        _close(w, dW[e][np.ix_(rows, cols)], what=f"entries dW[{e}]")
        _close(bb, db[e][rows], what=f"entries db[{e}]")


def pin_ste_gate_gets_no_expert_gradient(impl):
    """FD of the expert-path loss w.r.t. the gate logits is 0 wherever a small
    perturbation cannot change the argmax (the ARCHITECTURE block's STE)."""
    X, G, W, b, dY = _tiny(13, B=3, NH=4, H=4, NE=3)
    eps = 1e-4
    s = np.sort(G.reshape(-1, 3), axis=1)
    safe = (s[:, -1] - s[:, -2]) > 2 * eps
    assert safe.sum() >= 6
    for t in np.nonzero(safe)[0]:
        for j in range(3):
            Gp = G.reshape(-1, 3).copy(); Gp[t, j] += eps
            Gm = G.reshape(-1, 3).copy(); Gm[t, j] -= eps
            d = _loss_exp(impl, X, Gp, W, b, dY) - _loss_exp(impl, X, Gm, W, b, dY)
            assert d == 0.0, "gate logit received a gradient through the expert path"


# ---------------------------------------------------------------- aux

def pin_softmax_library(impl):
    import scipy.special
    G = _rng(14).standard_normal((50, 7)) * 30
    G[:10] += 900.0   # large logits: only the max-shifted form stays finite
    G[10:20] -= 900.0
    _close(impl.softmax(G, 7), scipy.special.softmax(G, axis=1), rtol=1e-12, atol=1e-15, what="softmax")


def pin_aux_uniform_counts(impl):
    """Equal counts: the loss is lambda exactly and the gradient vanishes."""
    G = _rng(15).standard_normal((40, 4))
    a = impl.aux(G, np.array([10, 10, 10, 10]), 0.02)
    assert abs(a.loss - 0.02) < 1e-15
    assert np.abs(a.d_gate_logits).max() < 1e-18


def pin_aux_uniform_probs(impl):
    """Constant logits: p = 1/N_E, so L = lambda and dG[t,j] = (lambda/T)(frac_j - 1/N_E)."""
    T, NE, lam = 30, 5, 0.03
    G = np.full((T, NE), 1.7)
    counts = np.array([12, 0, 9, 6, 3])
    a = impl.aux(G, counts, lam)
    assert abs(a.loss - lam) < 1e-15
    _close(a.d_gate_logits, np.tile((lam / T) * (counts / T - 1.0 / NE), (T, 1)), rtol=1e-12, atol=1e-18,
           what="uniform-p dG")


def pin_aux_collapse(impl):
    """Every token on one expert with a one-hot softmax: L -> lambda * N_E."""
    T, NE, lam = 16, 8, 0.01
    G = np.zeros((T, NE)); G[:, 4] = 800.0
    counts = np.zeros(NE, dtype=np.int64); counts[4] = T
    a = impl.aux(G, counts, lam)
    assert abs(a.loss - lam * NE) < 1e-15


def pin_aux_bounds_and_rowsum(impl):
    """0 < L <= lambda*N_E; each row of dG sums to zero (softmax-Jacobian rows,
    the same invariant the softmax/cross-entropy page asserts)."""
    inp = workloads.make_inputs(workloads.workload(1))
    f = impl.forward(inp.fused_ctx, inp.gate_logits, inp.W, inp.b)
    a = impl.aux(inp.gate_logits, f.counts, 0.01)
    assert 0.0 < a.loss <= 0.01 * 4
    scale = np.abs(a.d_gate_logits).max()
    assert scale > 0
    assert np.abs(a.d_gate_logits.sum(axis=1)).max() < 1e-12 * scale
    _close(a.frac, f.counts / 320.0, what="frac")
    _close(a.probs.sum(axis=1), np.ones(320), what="softmax rows")


def pin_aux_central_fd(impl):
    """Central differences of L(G) with the counts frozen match dG."""
    G = _rng(16).standard_normal((6, 4))
    counts = np.array([3, 1, 0, 2])
    lam = 0.05
    a = impl.aux(G, counts, lam)
    eps = 1e-5
    fd = np.zeros_like(G)
    for ix in np.ndindex(G.shape):
        Gp = G.copy(); Gp[ix] += eps
        Gm = G.copy(); Gm[ix] -= eps
        fd[ix] = (impl.aux(Gp, counts, lam).loss - impl.aux(Gm, counts, lam).loss) / (2 * eps)
    _close(a.d_gate_logits, fd, rtol=1e-6, atol=1e-11, what="aux FD")


def pin_aux_brute(impl):
    G = _rng(17).standard_normal((9, 3)) * 2
    counts = [4, 5, 0]
    a = impl.aux(G, np.array(counts), 0.01)
    P, frac, mp, loss, dG = brute.aux(G.tolist(), counts, 0.01)
    _close(a.probs, P, what="brute p")
    _close(a.mean_prob, mp, what="brute mean_prob")
    assert abs(a.loss - loss) < 1e-15
    _close(a.d_gate_logits, dG, rtol=1e-10, atol=1e-17, what="brute dG")


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
