"""Bitwise reproducibility: no atomics, fixed reduction orders."""
import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wl", [workloads.workload(2), workloads.custom(173, 7, 256, 5),
                                workloads.custom(1000, 5, 128, 8, gate_bias={4: 2.5}, lam=0.05),
                                workloads.custom(300, 5, 512, 8, act="bf16"), workloads.workload(4),
                                workloads.workload(3)],
                         ids=["pages_shape", "ragged_H256_NE5", "skewed", "bf16_H512", "wider_bf16", "imbalanced"])
def test_repeats_are_bitwise_identical(gpu_lib, wl):
    from tests import gpu_run
    inp = workloads.make_inputs(wl)
    other = workloads.make_inputs(workloads.custom(37, 3, 64, 3))
    d = gpu_run.upload(inp)
    d2 = gpu_run.upload(other)
    o = gpu_run.Buffers(d)
    o2 = gpu_run.Buffers(d2)
    gpu_run.step(d, o)
    ref = gpu_run.snapshot(o)
    for rep in range(10):
        gpu_run.step(d2, o2)  # interleave another shape
        o_new = gpu_run.Buffers(d)
        gpu_run.step(d, o_new)
        got = gpu_run.snapshot(o_new)
        for k, v in ref.items():
            assert np.array_equal(v.view(np.uint8), got[k].view(np.uint8)), f"repeat {rep}: {k} differs"


@pytest.mark.parametrize("wl", [workloads.workload(2), workloads.custom(20000, 5, 256, 8, gate_bias={4: 1.5}),
                                workloads.custom(300, 5, 512, 8, act="bf16")],
                         ids=["pages_shape", "persistent_H256", "bf16_H512"])
def test_aux_on_second_stream_matches_serial(gpu_lib, wl):
    """The auxiliary loss on its own stream, overlapping the backward, gives the serial
    step's bits: the two passes share the workspace but not its regions."""
    import torch
    from tests import gpu_run
    inp = workloads.make_inputs(wl)
    d = gpu_run.upload(inp)
    o = gpu_run.Buffers(d)
    gpu_run.step(d, o)
    ref = gpu_run.snapshot(o)
    side = torch.cuda.Stream()
    o2 = gpu_run.Buffers(d)
    for rep in range(3):
        gpu_run.step(d, o2, aux_stream=side)
        got = gpu_run.snapshot(o2)
        for k, v in ref.items():
            assert np.array_equal(v.view(np.uint8), got[k].view(np.uint8)), f"repeat {rep}: {k} differs"


@pytest.mark.slow
def test_large_stress_repeats_are_bitwise_identical(gpu_lib):
    """Large stress (1,048,576 tokens, H = 256, N_E = 16): the persistent forward and d_X
    tiles and the 128 x 128 d_W chunk tiles, ten repeats with another shape between them,
    every output compared bit for bit on the device (the perf page's Discipline block)."""
    import torch
    from tests import gpu_run
    wl = workloads.workload(5)
    print(f"[determinism] workload 5 {wl}", flush=True)
    d = gpu_run.upload(workloads.make_inputs(wl))
    d2 = gpu_run.upload(workloads.make_inputs(workloads.custom(37, 3, 64, 3)))
    o = gpu_run.Buffers(d)
    o2 = gpu_run.Buffers(d2)
    names = ("y", "idx", "counts", "offsets", "perm", "dx", "dW", "db", "loss", "dg", "frac", "mean_prob", "probs")
    gpu_run.step(d, o)
    ref = {k: getattr(o, k).clone() for k in names}
    for rep in range(10):
        gpu_run.step(d2, o2)  # interleave another shape
        for k in names:  # every output must be written again
            t = getattr(o, k)
            t.fill_(-1) if t.dtype == torch.int32 else t.fill_(float("nan"))
        gpu_run.step(d, o)
        torch.cuda.synchronize()
        for k in names:
            a, b = ref[k], getattr(o, k)
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"repeat {rep}: {k} differs"
