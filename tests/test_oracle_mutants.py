"""Plant plausible mistakes in copies of the CPU oracle and check that the pins catch each.

Mistakes are planted only in the oracle, on the CPU.  A mutant passes the suite
only if no pin notices it, which fails the test.
"""
import types

import numpy as np
import pytest

from oracle import moe_oracle as O
from tests import oracle_pins


def _copy(**repl):
    ns = types.SimpleNamespace(route=O.route, group=O.group, forward=O.forward,
                               backward=O.backward, backward_entries=O.backward_entries, aux=O.aux,
                               softmax=O.softmax)
    for k, v in repl.items():
        setattr(ns, k, v)
    return ns


def _route_last_tie(G, NE):
    G = np.asarray(G, dtype=np.float64).reshape(-1, NE)
    return (NE - 1 - np.argmax(G[:, ::-1], axis=1)).astype(np.int32)


def _group_unstable(idx, NE):
    counts, offsets, perm = O.group(idx, NE)
    out = perm.copy()
    for e in range(NE):
        out[offsets[e]:offsets[e + 1]] = perm[offsets[e]:offsets[e + 1]][::-1]
    return counts, offsets, out


def _fwd_variant(kind):
    def fwd(X, G, W, b):
        NE, H, _ = np.shape(W)
        Xf = np.asarray(X, dtype=np.float64).reshape(-1, H)
        idx = O.route(G, NE)
        counts, offsets, perm = O.group(idx, NE)
        Y = np.empty_like(Xf)
        for e in range(NE):
            r = idx == e
            if kind == "w_not_transposed":
                Y[r] = Xf[r] @ W[e] + b[e]
            elif kind == "no_bias":
                Y[r] = Xf[r] @ W[e].T
            elif kind == "wrong_bias_expert":
                Y[r] = Xf[r] @ W[e].T + b[(e + 1) % NE]
            elif kind == "prob_scaled":
                p = O.softmax(G, NE)[r, e][:, None]
                Y[r] = p * (Xf[r] @ W[e].T + b[e])
        return O.FwdResult(idx, counts, offsets, perm, Y)
    return fwd


def _bwd_variant(kind):
    def bwd(dY, X, W, idx, prev=None):
        r = O.backward(dY, X, W, idx, prev)
        NE, H, _ = np.shape(W)
        dYf = np.asarray(dY, dtype=np.float64).reshape(-1, H)
        Xf = np.asarray(X, dtype=np.float64).reshape(-1, H)
        idx = np.asarray(idx).reshape(-1)
        for e in range(NE):
            m = idx == e
            if not m.any():
                if kind == "inactive_negzero":
                    r.d_W[e] = -0.0
                continue
            if kind == "dx_transposed":
                r.d_fused_ctx[m] = dYf[m] @ W[e].T
            elif kind == "dw_transposed":
                r.d_W[e] = Xf[m].T @ dYf[m]
            elif kind == "db_all_tokens":
                r.d_b[e] = dYf.sum(axis=0)
            elif kind == "dw_mean":
                r.d_W[e] /= m.sum()
        if kind == "no_accumulate" and prev is not None:
            r = O.backward(dY, X, W, idx, None)
        return r
    return bwd


def _entries_variant(kind):
    def entries(dYc, Xc, idx, e):
        dYc = np.asarray(dYc, dtype=np.float64)
        Xc = np.asarray(Xc, dtype=np.float64)
        m = np.asarray(idx).reshape(-1) == e
        if kind == "all_tokens":
            return dYc.T @ Xc, dYc.sum(axis=0)
        if kind == "next_expert":
            m = np.asarray(idx).reshape(-1) == (e + 1) % 4
        return dYc[m].T @ Xc[m], dYc[m].sum(axis=0)
    return entries


def _aux_variant(kind):
    def aux(G, counts, lam):
        a = O.aux(G, counts, lam)
        counts = np.asarray(counts, dtype=np.float64)
        NE = counts.size
        T = a.probs.shape[0]
        if kind == "no_ne_factor":
            a.loss /= NE
            a.d_gate_logits /= NE
        elif kind == "grad_sign":
            a.d_gate_logits = -a.d_gate_logits
        elif kind == "grad_uses_mean_prob":
            p = a.probs
            s = p @ a.mean_prob
            a.d_gate_logits = (lam * NE / T) * p * (a.mean_prob[None, :] - s[:, None])
        elif kind == "grad_missing_jacobian_term":
            a.d_gate_logits = (lam * NE / T) * a.probs * a.frac[None, :]
        elif kind == "frac_per_expert_mean":
            a.frac = counts / max(counts.max(), 1)
            a.loss = float(lam * NE * np.dot(a.frac, a.mean_prob))
        return a
    return aux


def _softmax_no_shift(G, NE):
    G = np.asarray(G, dtype=np.float64).reshape(-1, NE)
    with np.errstate(over="ignore", invalid="ignore"):
        z = np.exp(G)
        return z / z.sum(axis=1, keepdims=True)


MUTANTS = {
    "route_last_index_on_tie": _copy(route=_route_last_tie),
    "group_unstable_perm": _copy(group=_group_unstable),
    "fwd_w_not_transposed": _copy(forward=_fwd_variant("w_not_transposed")),
    "fwd_no_bias": _copy(forward=_fwd_variant("no_bias")),
    "fwd_wrong_bias_expert": _copy(forward=_fwd_variant("wrong_bias_expert")),
    "fwd_scaled_by_gate_prob": _copy(forward=_fwd_variant("prob_scaled")),
    "bwd_dx_transposed": _copy(backward=_bwd_variant("dx_transposed")),
    "bwd_dw_transposed": _copy(backward=_bwd_variant("dw_transposed")),
    "bwd_db_over_all_tokens": _copy(backward=_bwd_variant("db_all_tokens")),
    "bwd_dw_mean_not_sum": _copy(backward=_bwd_variant("dw_mean")),
    "bwd_inactive_negative_zero": _copy(backward=_bwd_variant("inactive_negzero")),
    "bwd_ignores_accumulate": _copy(backward=_bwd_variant("no_accumulate")),
    "bwd_entries_over_all_tokens": _copy(backward_entries=_entries_variant("all_tokens")),
    "bwd_entries_of_next_expert": _copy(backward_entries=_entries_variant("next_expert")),
    "aux_missing_ne_factor": _copy(aux=_aux_variant("no_ne_factor")),
    "aux_grad_sign": _copy(aux=_aux_variant("grad_sign")),
    "aux_grad_uses_mean_prob": _copy(aux=_aux_variant("grad_uses_mean_prob")),
    "aux_grad_missing_jacobian_term": _copy(aux=_aux_variant("grad_missing_jacobian_term")),
    "aux_frac_normalised_by_max": _copy(aux=_aux_variant("frac_per_expert_mean")),
    "softmax_without_shift": _copy(softmax=_softmax_no_shift),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_some_pin_catches_mutant(name):
    impl = MUTANTS[name]
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(impl)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught mutant {name}"
