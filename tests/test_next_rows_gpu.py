"""GPU parity for reduce_axis0, the horizon mean collapse (and the backward that folds it in)
and the softmax-CE gradient head, against the fp64 oracles."""
import math

import numpy as np
import pytest

import workloads
from oracle import moe_oracle as O
from oracle import next_rows as N
from tests import compare as C

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------- reduce_axis0
@pytest.mark.parametrize("shape", [(1, 1), (7, 5), (64, 4), (1000, 1003), (3001, 4096), (129, 40000), (20, 65536)])
def test_reduce_axis0_parity_and_repeatability(gpu_lib, shape):
    import torch
    import mixture_experts_top_amd as moe
    rng = np.random.default_rng(sum(shape))
    x = rng.standard_normal(shape).astype(np.float32)
    xd = torch.from_numpy(x).cuda()
    out = torch.full((shape[1],), float("nan"), device="cuda")
    moe.moe_reduce_axis0(xd, out)
    got = out.cpu().numpy()
    C.per_expert_scaled("reduce_axis0", got[None], N.reduce_axis0(x)[None])
    out2 = torch.full((shape[1],), float("nan"), device="cuda")
    moe.moe_reduce_axis0(xd, out2)
    assert np.array_equal(got.view(np.uint32), out2.cpu().numpy().view(np.uint32))


@pytest.mark.slow
def test_reduce_axis0_pages_moe_shape_sampled(gpu_lib):
    """n_batch = B*N_H = 20480, n_tail = N_E*H*H = 65536 (the MoE scratch shape the MHA page
    sizes reduce_axis0 for); sampled columns against the oracle."""
    import torch
    import mixture_experts_top_amd as moe
    n_batch, n_tail = 20480, 65536
    g = torch.Generator(device="cuda").manual_seed(2024)
    xd = torch.randn(n_batch, n_tail, device="cuda", generator=g)
    out = torch.empty(n_tail, device="cuda")
    moe.moe_reduce_axis0(xd, out)
    cols = np.sort(np.random.default_rng(0).choice(n_tail, 256, replace=False))
    ref = N.reduce_axis0(xd[:, torch.from_numpy(cols).cuda()].cpu().numpy())
    C.per_expert_scaled("reduce_axis0[sampled]", out.cpu().numpy()[cols][None], ref[None])


# ---------------------------------------------------------------- horizon mean collapse
@pytest.mark.parametrize("act", ["f32", "bf16"])
@pytest.mark.parametrize("B,NH,H", [(1, 1, 64), (37, 5, 128), (300, 8, 256), (17, 3, 512)])
def test_horizon_mean_collapse(gpu_lib, act, B, NH, H):
    import torch
    import mixture_experts_top_amd as moe
    from tests import gpu_run
    rng = np.random.default_rng(B * NH + H)
    x = rng.standard_normal((B, NH, H)).astype(np.float32)
    d = rng.standard_normal((B, H)).astype(np.float32)
    xb = db = None
    if act == "bf16":
        xb, db = workloads.f32_to_bf16_bits(x), workloads.f32_to_bf16_bits(d)
        x, d = workloads.bf16_bits_to_f32(xb), workloads.bf16_bits_to_f32(db)
    xd, dd = gpu_run.dev_act(x, xb), gpu_run.dev_act(d, db)
    mean = torch.empty(B, H, dtype=xd.dtype, device="cuda")
    dx = torch.empty(B, NH, H, dtype=xd.dtype, device="cuda")
    moe.moe_horizon_mean_collapse_fwd(xd, mean)
    moe.moe_horizon_mean_collapse_bwd(dd, dx)
    gm, gdx = gpu_run.to_host(mean), gpu_run.to_host(dx)
    if act == "bf16":
        C.bf16_scaled("mean", gm, N.horizon_mean_fwd(x))
        C.bf16_scaled("d_x", gdx, N.horizon_mean_bwd(d, NH))
    else:
        C.elementwise("mean", gm, N.horizon_mean_fwd(x))
        C.elementwise("d_x", gdx, N.horizon_mean_bwd(d, NH))


@pytest.mark.parametrize("wl", [workloads.custom(173, 7, 128, 3), workloads.custom(61, 5, 256, 8),
                                workloads.custom(3001, 5, 64, 4),
                                pytest.param(workloads.custom(14000, 5, 128, 4), marks=pytest.mark.slow),
                                pytest.param(workloads.custom(9000, 5, 256, 6), marks=pytest.mark.slow),
                                pytest.param(workloads.custom(14000, 5, 256, 6), marks=pytest.mark.slow),
                                workloads.custom(97, 5, 128, 3, act="bf16"),
                                workloads.custom(150, 7, 256, 5, act="bf16"),
                                workloads.custom(600, 5, 512, 8, act="bf16", gate_bias={2: 1.0}),
                                pytest.param(workloads.custom(16500, 8, 256, 5, act="bf16"), marks=pytest.mark.slow),
                                pytest.param(workloads.custom(7000, 5, 512, 8, act="bf16", seed=33),
                                             marks=pytest.mark.slow)],
                         ids=["H128", "H256", "H64_multiblock", "H128_large_T_tiling", "H256_big_dw_tiles",
                              "H256_w_stationary",
                              "bf16_H128", "bf16_H256", "bf16_H512", "bf16_H256_large_T", "bf16_H512_w_stationary"])
def test_bwd_from_mean_equals_collapse_then_bwd(gpu_lib, wl):
    import torch
    import mixture_experts_top_amd as moe
    from tests import gpu_run
    inp = workloads.make_inputs(wl)
    B, NH, H = inp.fused_ctx.shape
    d_mean = np.random.default_rng(9).standard_normal((B, H)).astype(np.float32)
    d_bits = None
    if wl.act == "bf16":
        d_bits = workloads.f32_to_bf16_bits(d_mean)
        d_mean = workloads.bf16_bits_to_f32(d_bits)
    dv = gpu_run.upload(inp)
    o = gpu_run.Buffers(dv)
    gpu_run.fwd(dv, o)
    dm = gpu_run.dev_act(d_mean, d_bits)
    # unfused: collapse backward, then the gate backward
    dY = torch.empty(B, NH, H, dtype=dv.x.dtype, device="cuda")
    moe.moe_horizon_mean_collapse_bwd(dm, dY)
    dv2 = gpu_run.DevInputs(dv.x, dv.g, dv.W, dv.b, dY, dv.lam)
    gpu_run.bwd(dv2, o)
    ref = gpu_run.snapshot(o)
    # fused
    o2 = gpu_run.Buffers(dv)
    o2.offsets.copy_(o.offsets)
    o2.perm.copy_(o.perm)
    moe.moe_top1_bwd_from_mean(dm, dv.x, dv.W, o2.offsets, o2.perm, o2.dx, o2.dW, o2.db, workspace=o2.ws)
    got = gpu_run.snapshot(o2)
    for k in ("dx", "dW", "db"):
        assert np.array_equal(got[k].view(np.uint32), ref[k].view(np.uint32)), k
    # and against the oracle
    f = O.forward(inp.fused_ctx, inp.gate_logits, inp.W, inp.b)
    bw = O.backward(N.horizon_mean_bwd(d_mean, NH), inp.fused_ctx, inp.W, f.expert_idx)
    if wl.act == "bf16":
        C.bf16_scaled("d_fused_ctx", got["dx"].reshape(B * NH, H), bw.d_fused_ctx)
        C.bf16_scaled("d_W", got["dW"], bw.d_W, per_expert=True)
        C.bf16_scaled("d_b", got["db"], bw.d_b, per_expert=True)
    else:
        C.elementwise("d_fused_ctx", got["dx"].reshape(B * NH, H), bw.d_fused_ctx)
        C.per_expert_scaled("d_W", got["dW"], bw.d_W)
        C.per_expert_scaled("d_b", got["db"], bw.d_b)


# ---------------------------------------------------------------- softmax-CE head
@pytest.mark.parametrize("B,NH,A", [(64, 5, 21), (1, 1, 21), (1000, 3, 21), (33, 2, 1), (40, 7, 8), (70, 3, 33),
                                    (50, 4, 64)])
def test_softmax_ce_parity(gpu_lib, B, NH, A):
    import torch
    import mixture_experts_top_amd as moe
    rng = np.random.default_rng(B + NH + A)
    z = (rng.standard_normal((B, NH, A)) * 3).astype(np.float32)
    lab = rng.integers(0, A, size=(B, NH)).astype(np.int32)
    lab.reshape(-1)[::7] = -1          # sentinel rows
    if B * NH > 5:
        lab.reshape(-1)[3] = A + 5     # out of range: treated as a sentinel
    grad = torch.full((B, NH, A), float("nan"), device="cuda")
    ce = torch.full((B, NH), float("nan"), device="cuda")
    moe.moe_softmax_ce_grad(torch.from_numpy(z).cuda(), torch.from_numpy(lab).cuda(), grad, ce)
    g, c = grad.cpu().numpy(), ce.cpu().numpy()
    rce, rgrad = N.softmax_ce(z, lab)
    C.elementwise("ce", c, rce)
    C.elementwise("grad * B", g * B, rgrad * B)
    sentinel = (lab < 0) | (lab >= A)
    assert np.all(g[sentinel] == 0) and np.all(c[sentinel] == 0)
    if (~sentinel).any():
        assert np.abs(g[~sentinel].sum(axis=-1)).max() * B < 1e-5


@pytest.mark.parametrize("shift", [1, 2, 3])
def test_softmax_ce_parity_unaligned(gpu_lib, shift):
    """logits and grad 4-byte but not 16-byte aligned: the element-wise sweeps."""
    import torch
    import mixture_experts_top_amd as moe
    B, NH, A = 300, 3, 21
    rng = np.random.default_rng(shift)
    z = (rng.standard_normal((B, NH, A)) * 3).astype(np.float32)
    lab = rng.integers(0, A, size=(B, NH)).astype(np.int32)
    lab.reshape(-1)[::5] = -1
    zbuf = torch.zeros(B * NH * A + 4, device="cuda")
    zbuf[shift:shift + B * NH * A] = torch.from_numpy(z.reshape(-1)).cuda()
    gbuf = torch.full((B * NH * A + 4,), float("nan"), device="cuda")
    zv = zbuf[shift:shift + B * NH * A].view(B, NH, A)
    gv = gbuf[shift:shift + B * NH * A].view(B, NH, A)
    assert zv.data_ptr() % 16 != 0 and gv.data_ptr() % 16 != 0
    ce = torch.full((B, NH), float("nan"), device="cuda")
    moe.moe_softmax_ce_grad(zv, torch.from_numpy(lab).cuda(), gv, ce)
    rce, rgrad = N.softmax_ce(z, lab)
    C.elementwise("ce", ce.cpu().numpy(), rce)
    C.elementwise("grad * B", gv.cpu().numpy() * B, rgrad * B)
    assert torch.isnan(gbuf[:shift]).all() and torch.isnan(gbuf[shift + B * NH * A:]).all(), "wrote outside grad"


def test_softmax_ce_uniform_logits_give_log_21(gpu_lib):
    import torch
    import mixture_experts_top_amd as moe
    B, NH, A = 16, 5, 21
    z = torch.full((B, NH, A), 0.25, device="cuda")
    lab = torch.arange(B * NH, dtype=torch.int32, device="cuda").reshape(B, NH) % A
    grad = torch.empty(B, NH, A, device="cuda")
    ce = torch.empty(B, NH, device="cuda")
    moe.moe_softmax_ce_grad(z, lab, grad, ce)
    assert np.allclose(ce.cpu().numpy(), math.log(21), rtol=0, atol=1e-6)
    assert abs(round(float(ce[0, 0]), 4) - 3.0445) < 1e-12


def test_softmax_ce_log_floor(gpu_lib):
    import torch
    import mixture_experts_top_amd as moe
    z = torch.zeros(1, 1, 21, device="cuda")
    z[0, 0, 3] = -2000.0
    grad = torch.empty(1, 1, 21, device="cuda")
    ce = torch.empty(1, 1, device="cuda")
    moe.moe_softmax_ce_grad(z, torch.tensor([[3]], dtype=torch.int32, device="cuda"), grad, ce)
    assert abs(float(ce[0, 0]) - 30 * math.log(10)) < 1e-4
