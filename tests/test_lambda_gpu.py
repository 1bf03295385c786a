"""Adaptive lambda on the device: the controller kernel against the oracle, and the aux pass
reading lambda from device memory (adaptive-lambda page, formula and validation blocks)."""
import json
import math
import os

import numpy as np
import pytest

import workloads
from oracle import lambda_controller as L
from oracle import moe_oracle as O
from tests import compare as C

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "lambda_controller_worked.json")


def _run_controller(ent, K, **kw):
    import torch
    import mixture_experts_top_amd as moe
    e = torch.tensor([ent], dtype=torch.float32, device="cuda")
    out = torch.full((1,), float("nan"), dtype=torch.float32, device="cuda")
    moe.moe_lambda_eff_update(e, out, K, **kw)
    return float(out.cpu()[0])


def test_controller_regimes_and_page_values(gpu_lib):
    g = json.load(open(GOLDEN))
    K = g["K"]
    tgt = L.entropy_target(K)
    cases = [math.log(K), tgt + 0.1, tgt, tgt / 2, 0.0] + [r["ent_ema"] for r in g["printed"]]
    for ent in cases:
        ent32 = float(np.float32(ent))
        got = _run_controller(ent32, K)
        ref = L.lambda_eff(ent32, K)
        assert abs(got - ref) <= 1e-5, (ent, got, ref)           # the page's unit-test bound
        # the kernel gets the knobs as fp32: with the same fp32 inputs it rounds the fp64 result once
        ref32 = L.lambda_eff(ent32, K, *(float(np.float32(v)) for v in (L.FLOOR, L.MAX_EXTRA, L.TARGET_FRAC)))
        assert got == float(np.float32(ref32)), (ent, got, ref32)
    for r in g["printed"]:
        assert abs(_run_controller(r["ent_ema"], K) - r["lambda_eff"]) <= 0.5e-4


@pytest.mark.parametrize("K", [2, 4, 16, 64])
def test_controller_other_expert_counts(gpu_lib, K):
    for ent in (0.0, 0.3, 0.5 * L.entropy_target(K), math.log(K)):
        ent32 = float(np.float32(ent))
        knobs = [float(np.float32(v)) for v in (0.02, 0.2, 0.6)]
        assert _run_controller(ent32, K, lambda_floor=0.02, lambda_max_extra=0.2, entropy_target_frac=0.6) == \
            float(np.float32(L.lambda_eff(ent32, K, *knobs)))


@pytest.mark.parametrize("B", [300, 9000], ids=["small", "multiblock"])
def test_aux_with_device_lambda_matches_host_lambda(gpu_lib, B):
    import torch
    import mixture_experts_top_amd as moe
    from tests import gpu_run
    inp = workloads.make_inputs(workloads.custom(B, 5, 64, 8, lam=0.0))
    d = gpu_run.upload(inp)
    o = gpu_run.Buffers(d)
    gpu_run.fwd(d, o)
    ent = torch.tensor([np.float32(0.9)], device="cuda")
    lam_dev = torch.empty(1, dtype=torch.float32, device="cuda")
    moe.moe_lambda_eff_update(ent, lam_dev, 8)
    lam = float(lam_dev.cpu()[0])
    gpu_run.aux(d, o, lam=lam)
    host = gpu_run.snapshot(o)
    o2 = gpu_run.Buffers(d)
    o2.counts.copy_(o.counts)
    moe.moe_aux_loss_lambda_dev(d.g, o2.counts, lam_dev, o2.loss, o2.dg, frac=o2.frac, mean_prob=o2.mean_prob,
                                probs=o2.probs, workspace=o2.ws)
    dev = gpu_run.snapshot(o2)
    for k in ("loss", "dg", "frac", "mean_prob", "probs"):
        assert np.array_equal(host[k].view(np.uint32), dev[k].view(np.uint32)), k
    # and the chain matches the oracles
    f = O.forward(inp.fused_ctx, inp.gate_logits, inp.W, inp.b)
    a = O.aux(inp.gate_logits, f.counts, L.lambda_eff(float(np.float32(0.9)), 8))
    C.elementwise("loss", dev["loss"][0], a.loss)
