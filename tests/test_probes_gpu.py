"""The calibration probes behind the benchmark's `peaks` record: the MFMA loop runs and
reports positive tick counts with finite checksums, and the copy reproduces its input bit
for bit (sizes with a ragged tail of the grid-stride loop)."""
import pytest

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("act", [0, 1], ids=["f32", "bf16"])
def test_mfma_probe_runs(gpu_lib, act):
    import torch
    m = gpu_lib
    wgs, iters = 16, 50
    sink = torch.full((wgs * 256,), float("nan"), dtype=torch.float32, device="cuda")
    ticks = torch.full((wgs, 2), -1, dtype=torch.int64, device="cuda")
    m.moe_probe_mfma(act, wgs, iters, sink, ticks)
    torch.cuda.synchronize()
    assert torch.isfinite(sink).all()
    assert (ticks > 0).all()


@pytest.mark.parametrize("nbytes", [16, 4096 * 16 + 48, (8 << 20) + 256])
def test_copy_probe_is_exact(gpu_lib, nbytes):
    import torch
    g = torch.Generator(device="cuda").manual_seed(nbytes)
    src = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, device="cuda", generator=g)
    dst = torch.zeros_like(src)
    gpu_lib.moe_probe_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
