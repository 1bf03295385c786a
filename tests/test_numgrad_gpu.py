"""Numerical-gradient check of the HIP path, after the MoE-gate commit page ("11b96dac6a"),
NUMGRAD VERIFICATION block: central differences of the forward against the analytic backward,
11 checks (4 of d_W, 3 of d_b, 4 of d_fused_ctx) at 5e-2 relative / 5e-3 absolute.

Here both sides are the library's own kernels: the scalar loss is L = sum_t <Y[t], R[t]> with
R = d_out, so dL/dX, dL/dW and dL/db are what moe_top1_bwd returns for dY = R, and each central
difference re-runs moe_top1_fwd on a perturbed copy of one input.  L is linear in X, W and b for
fixed routing (X, W and b do not move the argmax), so the differences are exact up to rounding.
Three checks of dG (the aux loss's logit gradient, frac held constant) are added on a workload
with continuous logits, at tokens whose top-two logit gap exceeds the step."""
import dataclasses

import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu

RTOL, ATOL = 5e-2, 5e-3  # the page's tolerances


def _loss(d, R):
    from tests import gpu_run
    o = gpu_run.Buffers(d)
    gpu_run.fwd(d, o)
    y = gpu_run.to_host(o.y).astype(np.float64).reshape(R.shape)
    return float((y * R).sum())


def _central(d, R, name, flat_index, eps):
    """Central difference of L along one element of input `name`; the step is the one the fp32
    values actually take."""
    base = getattr(d, name)
    plus, minus = base.clone(), base.clone()
    v = float(base.reshape(-1)[flat_index])
    hi = np.float32(v + eps)
    lo = np.float32(v - eps)
    plus.view(-1)[flat_index] = float(hi)
    minus.view(-1)[flat_index] = float(lo)
    lp = _loss(dataclasses.replace(d, **{name: plus}), R)
    lm = _loss(dataclasses.replace(d, **{name: minus}), R)
    return (lp - lm) / (float(hi) - float(lo))


def _close(fd, an):
    return abs(fd - an) <= ATOL + RTOL * abs(an)


def test_numgrad_dx_dw_db(gpu_lib):
    import torch  # noqa: F401  (device buffers)
    from tests import gpu_run
    inp = workloads.make_inputs(workloads.workload(1))  # B=64, N_H=5, H=128, N_E=4, fp32
    print(f"[numgrad] {inp.wl}", flush=True)
    T, H, NE = inp.wl.T, inp.wl.H, inp.wl.NE
    d = gpu_run.upload(inp)
    o = gpu_run.Buffers(d)
    gpu_run.fwd(d, o)
    gpu_run.bwd(d, o)
    s = gpu_run.snapshot(o)
    R = inp.d_out.astype(np.float64).reshape(T, H)
    rng = np.random.default_rng(11)
    active = [e for e in range(NE) if s["counts"][e] > 0]
    assert active, "no expert received tokens"
    eps = 1e-2
    failures = []
    for _ in range(4):  # d_fused_ctx
        t, i = int(rng.integers(T)), int(rng.integers(H))
        fd, an = _central(d, R, "x", t * H + i, eps), float(s["dx"].reshape(T, H)[t, i])
        if not _close(fd, an):
            failures.append(("dX", t, i, fd, an))
    for _ in range(4):  # d_W
        e, r, c = int(rng.choice(active)), int(rng.integers(H)), int(rng.integers(H))
        fd, an = _central(d, R, "W", (e * H + r) * H + c, eps), float(s["dW"][e, r, c])
        if not _close(fd, an):
            failures.append(("dW", e, r, c, fd, an))
    for _ in range(3):  # d_b
        e, r = int(rng.choice(active)), int(rng.integers(H))
        fd, an = _central(d, R, "b", e * H + r, eps), float(s["db"][e, r])
        if not _close(fd, an):
            failures.append(("db", e, r, fd, an))
    assert not failures, failures


def test_numgrad_aux_logits(gpu_lib):
    import torch
    from tests import gpu_run
    wl = workloads.custom(64, 5, 128, 4)  # continuous N(0, 1) logits
    inp = workloads.make_inputs(wl)
    print(f"[numgrad aux] {wl}", flush=True)
    T, NE, lam = wl.T, wl.NE, wl.lam
    d = gpu_run.upload(inp)
    o = gpu_run.Buffers(d)
    gpu_run.fwd(d, o)
    gpu_run.aux(d, o)
    s = gpu_run.snapshot(o)
    G = inp.gate_logits.reshape(T, NE).astype(np.float64)
    top2 = np.sort(G, axis=1)[:, -2:]
    eps = 1e-2
    ok_tokens = np.nonzero(top2[:, 1] - top2[:, 0] > 4 * eps)[0]
    rng = np.random.default_rng(5)
    scale = T / (lam * NE)  # dG is O(lam N_E / T): compare it on the unit scale

    def aux_loss(g):
        o2 = gpu_run.Buffers(d)
        d2 = dataclasses.replace(d, g=g)
        gpu_run.fwd(d2, o2)
        gpu_run.aux(d2, o2)
        torch.cuda.synchronize()
        return float(gpu_run.to_host(o2.loss)[0])

    failures = []
    for _ in range(3):
        t, j = int(rng.choice(ok_tokens)), int(rng.integers(NE))
        plus, minus = d.g.clone(), d.g.clone()
        v = float(G[t, j])
        hi, lo = np.float32(v + eps), np.float32(v - eps)
        plus.view(-1)[t * NE + j] = float(hi)
        minus.view(-1)[t * NE + j] = float(lo)
        fd = (aux_loss(plus) - aux_loss(minus)) / (float(hi) - float(lo))
        an = float(s["dg"].reshape(T, NE)[t, j])
        if not _close(fd * scale, an * scale):
            failures.append((t, j, fd, an))
    assert not failures, failures
