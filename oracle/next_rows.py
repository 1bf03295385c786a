"""fp64 CPU oracles for three operations adjacent to the gate (test infrastructure only).

* reduce_axis0 -- perf-pass page ("b23f8f2efa"), reduce_axis0 entry; MHA page ("9170d24fe3"),
  trainer and BUG blocks: out[j] = sum_r in[r, j] over an [n_batch, n_tail] array (the MoE
  uses n_batch = B*N_H, n_tail = N_E*H*H).
* horizon mean collapse -- MHA page, new-kernel block: [B, N_H, H] -> [B, H] by averaging over
  the horizon axis; its backward spreads d_out[b] / N_H to every horizon.
* softmax + cross-entropy gradient head -- softmax/cross-entropy page ("6cfd7e6691"), kernel
  block: per (b, h) row of A logits, p = softmax (max-shifted), CE = -log(max(p[label], 1e-30)),
  grad = (p - onehot(label)) / B (mean over the batch), and a label of -1 (sentinel) gives a
  zero loss and a zero gradient row.
"""
from __future__ import annotations

import numpy as np


def reduce_axis0(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).sum(axis=0)


def horizon_mean_fwd(x) -> np.ndarray:
    """x [B, N_H, H] -> [B, H]."""
    return np.asarray(x, dtype=np.float64).mean(axis=1)


def horizon_mean_bwd(d_out, NH: int) -> np.ndarray:
    """d_out [B, H] -> [B, N_H, H]."""
    d = np.asarray(d_out, dtype=np.float64)
    return np.repeat(d[:, None, :] / NH, NH, axis=1)


def softmax_ce(logits, labels):
    """logits [B, N_H, A], labels [B, N_H] int (-1 = sentinel) -> (ce [B, N_H], grad [B, N_H, A])."""
    z = np.asarray(logits, dtype=np.float64)
    lab = np.asarray(labels)
    B = z.shape[0]
    A = z.shape[-1]
    e = np.exp(z - z.max(axis=-1, keepdims=True))
    p = e / e.sum(axis=-1, keepdims=True)
    valid = (lab >= 0) & (lab < A)
    safe = np.where(valid, lab, 0)
    p_lab = np.take_along_axis(p, safe[..., None], axis=-1)[..., 0]
    ce = np.where(valid, -np.log(np.maximum(p_lab, 1e-30)), 0.0)
    onehot = np.zeros_like(p)
    np.put_along_axis(onehot, safe[..., None], 1.0, axis=-1)
    grad = np.where(valid[..., None], (p - onehot) / B, 0.0)
    return ce, grad
