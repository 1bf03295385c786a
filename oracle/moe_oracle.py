"""fp64 CPU oracle for the top-1 Mixture-of-Experts gate.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The HIP library never calls it and
shares no code with it; the only thing both sides use is the seeded input
generator, which holds none of the gate's arithmetic.

What is computed, and where the pages define it (the commit page
"11b96dac6a  Top-1 Mixture-of-Experts gate per Switch Transformer" unless noted):

* route      -- summary block and PERFORMANCE block: one expert per (b, h) token,
                the top-1 of gate_logits, picked by a single serial scan.
                Ties: the lowest expert index (strict ">" while scanning upward).
* group      -- counts, exclusive offsets and the stable permutation that lists
                the tokens of expert 0, then expert 1, ... each in ascending token
                order.  The pages have no such step; it is the plain definition of
                a stable counting sort by expert.
* forward    -- summary block: routed_ctx = W[e*] @ fused_ctx + b[e*], with W laid
                out [N_E, H_out, H_in] (PERFORMANCE block: one output channel is a
                dot product over the input dimension).  No scaling by the gate
                probability: the STE statement in ARCHITECTURE gives the gate no
                gradient through this path.
* backward   -- summary block: gradients flow only through the selected expert;
                inactive experts get exactly zero; d_fused_ctx = W[e*]^T @ d_out
                (optionally added to a previous d_fused_ctx: the page calls it an
                accumulator).  The gate logits get no gradient from this path.
* backward_entries -- the same sums as backward's d_W[e] and d_b[e], restricted to chosen
                output and input features (for sampled checks of very large inputs).
* aux        -- summary block: softmax of gate_logits and the load-balancing loss
                lambda * N_E * sum_e frac_e * mean_prob_e.  The softmax follows the
                stable form of the softmax/cross-entropy page ("6cfd7e6691"): shift
                by the row max, exponentiate, divide by the row sum.  frac is the
                share of tokens routed to each expert (a count, so it is held
                constant when differentiating); mean_prob is the mean softmax
                probability over all B*N_H tokens.

Every array is taken in fp64 from the stored values (fp32, or bf16 widened
exactly).  Pins that tie these functions to the mathematics live in
tests/test_oracle.py.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def _tokens(a: np.ndarray, last: int) -> np.ndarray:
    return np.asarray(a, dtype=np.float64).reshape(-1, last)


def route(gate_logits: np.ndarray, NE: int) -> np.ndarray:
    """Top-1 expert per token by an upward strict-'>' scan (lowest index wins ties)."""
    G = _tokens(gate_logits, NE)
    best = G[:, 0].copy()
    idx = np.zeros(G.shape[0], dtype=np.int32)
    for e in range(1, NE):
        better = G[:, e] > best
        best = np.where(better, G[:, e], best)
        idx = np.where(better, np.int32(e), idx)
    return idx


def group(expert_idx: np.ndarray, NE: int):
    """Counts, exclusive offsets [N_E+1] and the stable by-expert permutation."""
    idx = np.asarray(expert_idx).reshape(-1)
    counts = np.bincount(idx, minlength=NE).astype(np.int32)
    offsets = np.zeros(NE + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    perm = np.argsort(idx, kind="stable").astype(np.int32)
    return counts, offsets, perm


@dataclass
class FwdResult:
    expert_idx: np.ndarray
    counts: np.ndarray
    offsets: np.ndarray
    perm: np.ndarray
    routed_ctx: np.ndarray  # [T, H] fp64


def forward(fused_ctx, gate_logits, W, b) -> FwdResult:
    NE, H, _ = np.shape(W)
    X = _tokens(fused_ctx, H)
    Wd = np.asarray(W, dtype=np.float64)
    bd = np.asarray(b, dtype=np.float64)
    idx = route(gate_logits, NE)
    counts, offsets, perm = group(idx, NE)
    Y = np.empty_like(X)
    for e in range(NE):
        rows = idx == e
        Y[rows] = X[rows] @ Wd[e].T + bd[e]
    return FwdResult(idx, counts, offsets, perm, Y)


@dataclass
class BwdResult:
    d_fused_ctx: np.ndarray  # [T, H]
    d_W: np.ndarray          # [N_E, H, H]
    d_b: np.ndarray          # [N_E, H]


def backward(d_out, fused_ctx, W, expert_idx, d_fused_ctx_prev=None) -> BwdResult:
    NE, H, _ = np.shape(W)
    dY = _tokens(d_out, H)
    X = _tokens(fused_ctx, H)
    Wd = np.asarray(W, dtype=np.float64)
    idx = np.asarray(expert_idx).reshape(-1)
    dX = np.zeros_like(X) if d_fused_ctx_prev is None else _tokens(d_fused_ctx_prev, H).copy()
    dW = np.zeros((NE, H, H))
    db = np.zeros((NE, H))
    for e in range(NE):
        rows = idx == e
        if not rows.any():
            continue  # inactive expert: exactly zero gradient
        dX[rows] += dY[rows] @ Wd[e]
        dW[e] = dY[rows].T @ X[rows]
        db[e] = dY[rows].sum(axis=0)
    return BwdResult(dX, dW, db)


def backward_entries(d_out_cols, fused_ctx_cols, expert_idx, e: int):
    """Selected entries of d_W[e] and d_b[e], from the same definition as `backward` (summary
    block: expert e's gradient sums over its own tokens only), for inputs too large to
    differentiate whole.  d_out_cols [T, k_o] holds the wanted columns o of d_out for every
    token, fused_ctx_cols [T, k_i] the wanted columns i of fused_ctx; returns
        d_W[e][o, i] = sum over tokens t routed to e of d_out[t, o] * fused_ctx[t, i]   [k_o, k_i]
        d_b[e][o]    = sum over tokens t routed to e of d_out[t, o]                     [k_o]
    both exactly zero when expert e has no tokens."""
    dY = np.asarray(d_out_cols, dtype=np.float64)
    X = np.asarray(fused_ctx_cols, dtype=np.float64)
    rows = np.asarray(expert_idx).reshape(-1) == e
    if not rows.any():
        return np.zeros((dY.shape[1], X.shape[1])), np.zeros(dY.shape[1])
    return dY[rows].T @ X[rows], dY[rows].sum(axis=0)


@dataclass
class AuxResult:
    probs: np.ndarray       # [T, N_E]
    frac: np.ndarray        # [N_E]
    mean_prob: np.ndarray   # [N_E]
    loss: float
    d_gate_logits: np.ndarray  # [T, N_E]


def softmax(gate_logits, NE: int) -> np.ndarray:
    G = _tokens(gate_logits, NE)
    z = np.exp(G - G.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def aux(gate_logits, counts, lam: float) -> AuxResult:
    counts = np.asarray(counts, dtype=np.float64)
    NE = counts.shape[0]
    p = softmax(gate_logits, NE)
    T = p.shape[0]
    frac = counts / T
    mean_prob = p.mean(axis=0)
    loss = float(lam * NE * np.dot(frac, mean_prob))
    # d loss / d G[t, j] with frac constant: (lam*NE/T) * sum_e frac_e * dp_e/dG_j,
    # and dp_e/dG_j = p_e (delta_ej - p_j) for a softmax row.
    s = p @ frac
    dG = (lam * NE / T) * p * (frac[None, :] - s[:, None])
    return AuxResult(p, frac, mean_prob, loss, dG)


def run_all(inp, lam=None, d_fused_ctx_prev=None):
    """fwd -> bwd -> aux on one set of inputs (from workloads.make_inputs)."""
    f = forward(inp.fused_ctx, inp.gate_logits, inp.W, inp.b)
    bw = backward(inp.d_out, inp.fused_ctx, inp.W, f.expert_idx, d_fused_ctx_prev)
    a = aux(inp.gate_logits, f.counts, inp.wl.lam if lam is None else lam)
    return f, bw, a
