"""moe_top1_fwd_aux against the calls it stands for: moe_top1_fwd followed by moe_aux_loss
(or moe_aux_loss_lambda_dev) must give the same bits on every output, on the shapes where
the loss rides on the routing and forward launches (fp32, N_E <= 8, small T), on the routing
and scatter launches (N_E <= 16 otherwise), and on those where the library makes the calls
one by one (N_E > 16).  Parity of the one-call path with the oracle
is checked by test_parity (its step uses this call)."""
import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu

CASES = {
    "pages_shape": workloads.workload(2),
    "tiny_ref_ties": workloads.workload(1),
    "ragged_H128_NE3": workloads.custom(173, 7, 128, 3),
    "ragged_H64_NE5": workloads.custom(97, 5, 64, 5),
    "H256_NE8": workloads.custom(61, 9, 256, 8),
    "H512_NE4": workloads.custom(40, 6, 512, 4),
    "dense_NE1": workloads.custom(300, 5, 128, 1),
    "single_token": workloads.custom(1, 1, 128, 4),
    "empty_expert": workloads.custom(64, 5, 128, 4, gate_bias={2: -1.0e4}),
    "multiblock_H64_NE8": workloads.custom(8191, 5, 64, 8),
    "NE7_int_ties": workloads.custom(80, 5, 256, 7, gate="int"),
    # shapes where the loss rides on the routing launches (N_E <= 8): scatter with the scan
    # folded in, and separate scan + scatter (n_blk x N_E > 4096), fp32 and bf16
    "large_T": workloads.workload(3),
    "scan_scatter_NE8": workloads.custom(28000, 5, 128, 8),
    "scan_scatter_NE3_ragged": workloads.custom(70001, 5, 64, 3, gate_bias={1: -1.0e4}),
    "bf16": workloads.custom(200, 5, 128, 4, act="bf16"),
    "bf16_H256_NE5": workloads.custom(3001, 5, 256, 5, act="bf16"),
    "bf16_single_token": workloads.custom(1, 1, 128, 4, act="bf16"),
    "bf16_NE1": workloads.custom(300, 5, 128, 1, act="bf16"),
    "bf16_empty_expert_ties": workloads.custom(64, 5, 64, 4, act="bf16", gate="int", gate_bias={2: -1.0e4}),
    "NE16": workloads.custom(200, 5, 128, 16),
    "NE13_scan_scatter": workloads.custom(20000, 5, 64, 13, gate="int"),
    # shapes where the calls run one by one
    "NE17": workloads.custom(200, 5, 128, 17),
}
KEYS = ("y", "idx", "counts", "offsets", "perm", "loss", "dg", "frac", "mean_prob", "probs")


def _same_bits(name, a, b):
    a, b = np.ascontiguousarray(a), np.ascontiguousarray(b)
    assert a.shape == b.shape, name
    assert a.tobytes() == b.tobytes(), f"{name}: {int((a.view(np.uint8) != b.view(np.uint8)).sum())} bytes differ"


def _snap(o, keys=KEYS):
    from tests import gpu_run
    s = gpu_run.snapshot(o)
    return {k: s[k] for k in keys}


@pytest.mark.parametrize("name", sorted(CASES))
def test_fwd_aux_equals_separate_calls(gpu_lib, name):
    from tests import gpu_run
    print(f"[fwd_aux] {name} {CASES[name]}", flush=True)
    inp = workloads.make_inputs(CASES[name])
    d = gpu_run.upload(inp)
    sep = gpu_run.Buffers(d)
    gpu_run.fwd(d, sep)
    gpu_run.aux(d, sep)
    one = gpu_run.Buffers(d)
    gpu_run.fwd_aux(d, one)
    a, b = _snap(sep), _snap(one)
    for k in KEYS:
        _same_bits(k, a[k], b[k])
    assert np.isfinite(b["loss"]).all() and np.isfinite(b["dg"]).all()


@pytest.mark.parametrize("name", ["pages_shape", "ragged_H128_NE3", "large_T", "scan_scatter_NE8", "bf16"])
def test_fwd_aux_lambda_dev(gpu_lib, name):
    import torch
    import mixture_experts_top_amd as moe
    from tests import gpu_run
    inp = workloads.make_inputs(CASES[name])
    d = gpu_run.upload(inp)
    lam = torch.tensor([0.037], dtype=torch.float32, device="cuda")
    sep = gpu_run.Buffers(d)
    gpu_run.fwd(d, sep)
    moe.moe_aux_loss_lambda_dev(d.g, sep.counts, lam, sep.loss, sep.dg, frac=sep.frac, mean_prob=sep.mean_prob,
                                probs=sep.probs, workspace=sep.ws)
    one = gpu_run.Buffers(d)
    gpu_run.fwd_aux(d, one, lam=float("nan"), lambda_dev=lam)  # the host value is ignored
    a, b = _snap(sep), _snap(one)
    for k in KEYS:
        _same_bits(k, a[k], b[k])


def test_fwd_aux_optional_outputs(gpu_lib):
    import mixture_experts_top_amd as moe
    from tests import gpu_run
    inp = workloads.make_inputs(CASES["pages_shape"])
    d = gpu_run.upload(inp)
    full = gpu_run.Buffers(d)
    gpu_run.fwd_aux(d, full)
    part = gpu_run.Buffers(d)
    moe.moe_top1_fwd_aux(d.x, d.g, d.W, d.b, part.y, part.idx, part.counts, part.offsets, part.perm, d.lam,
                         part.loss, part.dg, workspace=part.ws)
    a, b = _snap(full), _snap(part, ("y", "perm", "loss", "dg"))
    for k in ("y", "perm", "loss", "dg"):
        _same_bits(k, a[k], b[k])
    assert np.isnan(gpu_run.to_host(part.probs)).all(), "probs written although not requested"


def test_fwd_aux_repeat_same_buffers(gpu_lib):
    """A second call on the same buffers and workspace (stale contents) gives the same bits."""
    from tests import gpu_run
    inp = workloads.make_inputs(CASES["multiblock_H64_NE8"])
    d = gpu_run.upload(inp)
    o = gpu_run.Buffers(d)
    gpu_run.fwd_aux(d, o)
    first = _snap(o)
    gpu_run.fwd_aux(d, o)
    again = _snap(o)
    for k in KEYS:
        _same_bits(k, first[k], again[k])
