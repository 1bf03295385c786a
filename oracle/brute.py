"""Brute-force, loop-only second oracle for tiny inputs.

TEST INFRASTRUCTURE ONLY (see oracle/moe_oracle.py for who may import it).
Every quantity is written element by element with Python floats (IEEE double)
and the ``math`` module, with no array library, so it shares no formulation with
the vectorised oracle: the tests compare the two.  It follows the same passages
of the MoE-gate commit page (summary, ARCHITECTURE and PERFORMANCE blocks) and the
stable softmax of the softmax/cross-entropy page.
"""
from __future__ import annotations

import math


def route(G):
    out = []
    for row in G:
        best_e, best_v = 0, row[0]
        for e in range(1, len(row)):
            if row[e] > best_v:
                best_e, best_v = e, row[e]
        out.append(best_e)
    return out


def group(idx, NE):
    counts = [0] * NE
    for e in idx:
        counts[e] += 1
    offsets = [0] * (NE + 1)
    for e in range(NE):
        offsets[e + 1] = offsets[e] + counts[e]
    perm = []
    for e in range(NE):
        for t, et in enumerate(idx):
            if et == e:
                perm.append(t)
    return counts, offsets, perm


def forward(X, G, W, b):
    """X [T][H], G [T][NE], W [NE][H_out][H_in], b [NE][H]."""
    idx = route(G)
    Y = []
    for t, x in enumerate(X):
        e = idx[t]
        Y.append([sum(W[e][o][i] * x[i] for i in range(len(x))) + b[e][o] for o in range(len(W[e]))])
    return idx, Y


def backward(dY, X, W, idx):
    NE, H = len(W), len(W[0])
    T = len(X)
    dX = [[sum(W[idx[t]][o][i] * dY[t][o] for o in range(H)) for i in range(H)] for t in range(T)]
    dW = [[[0.0] * H for _ in range(H)] for _ in range(NE)]
    db = [[0.0] * H for _ in range(NE)]
    for t in range(T):
        e = idx[t]
        for o in range(H):
            db[e][o] += dY[t][o]
            for i in range(H):
                dW[e][o][i] += dY[t][o] * X[t][i]
    return dX, dW, db


def aux(G, counts, lam):
    T, NE = len(G), len(counts)
    P = []
    for row in G:
        m = max(row)
        z = [math.exp(v - m) for v in row]
        s = sum(z)
        P.append([v / s for v in z])
    frac = [c / T for c in counts]
    mean_prob = [sum(P[t][e] for t in range(T)) / T for e in range(NE)]
    loss = lam * NE * sum(frac[e] * mean_prob[e] for e in range(NE))
    # dL/dG[t][j] = (lam*NE/T) * sum_e frac_e * P[t][e] * (delta_ej - P[t][j])
    dG = []
    for t in range(T):
        row = []
        for j in range(NE):
            acc = 0.0
            for e in range(NE):
                acc += frac[e] * P[t][e] * ((1.0 if e == j else 0.0) - P[t][j])
            row.append(lam * NE / T * acc)
        dG.append(row)
    return P, frac, mean_prob, loss, dG
