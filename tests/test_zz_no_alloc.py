"""moe_top1_fwd_noalloc (scratch in the library's per-device array, no workspace argument)
against moe_top1_fwd with a caller's workspace, through the C ABI: two calls in a row, the
second with a smaller input, each compared bit for bit (same kernels) on every output.
The first shape takes the multi-launch routing (scan + scatter), the second the one-launch
small-token forward that forms perm itself; a bf16 pair covers the other forward kernels."""
import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu


def _outputs(d, T, NE):
    import torch
    dev = d.x.device
    return {"y": torch.full_like(d.x, float("nan")),
            "idx": torch.full((T,), -1, dtype=torch.int32, device=dev),
            "counts": torch.full((NE,), -1, dtype=torch.int32, device=dev),
            "offsets": torch.full((NE + 1,), -1, dtype=torch.int32, device=dev),
            "perm": torch.full((T,), -1, dtype=torch.int32, device=dev)}


def _bits(t):
    import torch
    t = t.detach()
    if t.dtype in (torch.float32, torch.bfloat16):
        t = t.view(torch.int32 if t.dtype == torch.float32 else torch.int16)
    return t.cpu().numpy()


def _run_pair(wl):
    import torch
    import mixture_experts_top_amd as moe
    from mixture_experts_top_amd import runner
    inp = workloads.make_inputs(wl)
    d = runner.upload(inp)
    T, NE = wl.T, wl.NE
    ref, got = _outputs(d, T, NE), _outputs(d, T, NE)
    ws = torch.empty(moe.moe_workspace_bytes(wl.B, wl.NH, wl.H, NE, runner.act_code(d.x)), dtype=torch.uint8,
                     device=d.x.device)
    moe.moe_top1_fwd(d.x, d.g, d.W, d.b, ref["y"], ref["idx"], ref["counts"], ref["offsets"], ref["perm"],
                     workspace=ws)
    moe.moe_top1_fwd_noalloc(d.x, d.g, d.W, d.b, got["y"], got["idx"], got["counts"], got["offsets"], got["perm"])
    torch.cuda.synchronize()
    for k in ref:
        a, b = _bits(ref[k]), _bits(got[k])
        assert np.array_equal(a, b), f"{wl.name}: {k} differs from moe_top1_fwd ({int((a != b).sum())} entries)"


@pytest.mark.parametrize("pair", [
    (workloads.workload(3), workloads.workload(2)),
    (workloads.custom(4096, 5, 512, 8, act="bf16"), workloads.custom(200, 5, 128, 4, act="bf16")),
], ids=["f32_imbalanced_then_pages_shape", "bf16_H512_then_H128"])
def test_noalloc_forward_matches_workspace_forward(gpu_lib, pair):
    big, small = pair
    assert small.T < big.T
    print(f"[no-alloc] {big.name} then {small.name}", flush=True)
    _run_pair(big)
    _run_pair(small)


def test_noalloc_rejects_scratch_beyond_the_array(gpu_lib):
    import torch
    import mixture_experts_top_amd as moe
    # ceil(T / 256) * N_E = 32768 * 64 histogram entries: 16 MiB of scratch, above the 8 MiB array
    B, NH, H, NE = 1 << 20, 8, 64, 64
    x = torch.empty(16, device="cuda")  # never read: the call fails before any launch
    with pytest.raises(moe.MoeError) as ei:
        lib = moe.load_library()
        moe._check(lib.moe_top1_fwd_noalloc(x.data_ptr(), x.data_ptr(), x.data_ptr(), x.data_ptr(), x.data_ptr(),
                                            x.data_ptr(), x.data_ptr(), x.data_ptr(), x.data_ptr(), B, NH, H, NE, 0,
                                            None))
    assert ei.value.status == 3 and "device array" in str(ei.value)
