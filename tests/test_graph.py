"""The three calls are capture-safe: a HIP graph of fwd -> bwd -> aux replays to the
eager results (several replays, with eager work and synchronisation in between)."""
import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu


GRAPH_CASES = {
    # the aux loss on the forward launch (fp32, small T), on the scatter with the scan folded in
    # (bf16), and on a separate scan + scatter (n_blk x N_E > 4096)
    "gather_f32": workloads.custom(300, 5, 128, 4),
    "scatter_scan_bf16": workloads.custom(300, 5, 256, 4, act="bf16"),
    "scan_scatter_f32": workloads.custom(28000, 5, 128, 8),
}


@pytest.mark.parametrize("name", sorted(GRAPH_CASES))
def test_graph_replay_matches_eager(gpu_lib, name):
    import torch
    from tests import gpu_run
    print(f"[graph] {name} {GRAPH_CASES[name]}", flush=True)
    inp = workloads.make_inputs(GRAPH_CASES[name])
    d = gpu_run.upload(inp)
    eager = gpu_run.Buffers(d)
    gpu_run.step(d, eager)
    ref = gpu_run.snapshot(eager)

    o = gpu_run.Buffers(d)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        gpu_run.step(d, o)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gpu_run.step(d, o)
    for rep in range(4):
        for t in (o.y, o.dx, o.dW, o.db, o.dg, o.loss):
            t.fill_(float("nan"))
        o.perm.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = gpu_run.snapshot(o)
        for k, v in ref.items():
            assert np.array_equal(v.view(np.uint8), got[k].view(np.uint8)), f"replay {rep}: {k} differs"
        gpu_run.step(d, eager)  # eager work between replays
        torch.cuda.synchronize()


def test_graph_with_aux_stream_matches_eager(gpu_lib):
    """Fork/join capture: the auxiliary loss on a second stream inside the graph."""
    import torch
    from tests import gpu_run
    inp = workloads.make_inputs(workloads.custom(4096, 5, 128, 4))
    d = gpu_run.upload(inp)
    eager = gpu_run.Buffers(d)
    gpu_run.step(d, eager)
    ref = gpu_run.snapshot(eager)

    o = gpu_run.Buffers(d)
    s, side = torch.cuda.Stream(), torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        gpu_run.step(d, o, aux_stream=side)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gpu_run.step(d, o, aux_stream=side)
    for rep in range(4):
        for t in (o.y, o.dx, o.dW, o.db, o.dg, o.loss):
            t.fill_(float("nan"))
        o.perm.fill_(-1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = gpu_run.snapshot(o)
        for k, v in ref.items():
            assert np.array_equal(v.view(np.uint8), got[k].view(np.uint8)), f"replay {rep}: {k} differs"
        gpu_run.step(d, eager)
        torch.cuda.synchronize()
