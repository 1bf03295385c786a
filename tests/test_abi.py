"""The C-ABI library on the host: it loads, exports every declared entry point, and
rejects bad arguments before touching a device (no compute calls, no GPU needed)."""
import ctypes
import os
import re

import pytest

import mixture_experts_top_amd as m

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_top1.h")

INVALID, UNSUPPORTED, WORKSPACE = 1, 2, 3
FAKE = 0x10000  # aligned, never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return m.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"moe_top1_fwd", "moe_top1_bwd", "moe_aux_loss", "moe_top1_route", "moe_workspace_bytes"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"library does not export {n}"


def test_version_and_strings(lib):
    assert m.moe_abi_version() == 1
    assert lib.moe_status_string(0) == b"ok"
    assert [m.moe_kernel_name(i) for i in range(len(m.KERNELS))] == m.KERNELS
    assert m.moe_kernel_name(99) is None


def test_workspace_bytes_grows_with_tokens():
    a = m.moe_workspace_bytes(64, 5, 128, 4)
    b = m.moe_workspace_bytes(4096, 5, 128, 4)
    c = m.moe_workspace_bytes(131072, 8, 256, 16)
    assert 0 < a < b < c
    assert c < 2 * 2 ** 30  # partials stay far below the 1 GiB activations of this shape
    assert all(x % 256 == 0 for x in (a, b, c))


@pytest.mark.parametrize("H,NE,code", [(96, 4, UNSUPPORTED), (128, 0, INVALID), (128, 65, UNSUPPORTED),
                                       (1024, 4, UNSUPPORTED), (0, 4, INVALID)])
def test_workspace_bytes_rejects_shapes(lib, H, NE, code):
    out = ctypes.c_size_t(0)
    assert lib.moe_workspace_bytes(8, 5, H, NE, 0, ctypes.byref(out)) == code
    assert lib.moe_last_error()


def test_workspace_bytes_rejects_overflow_and_dtype(lib):
    out = ctypes.c_size_t(0)
    assert lib.moe_workspace_bytes(1 << 22, 8, 512, 4, 0, ctypes.byref(out)) == INVALID  # T*H >= 2^31
    assert lib.moe_workspace_bytes(8, 5, 128, 4, 7, ctypes.byref(out)) == UNSUPPORTED
    assert lib.moe_workspace_bytes(8, 5, 128, 4, 0, None) == INVALID


def _fwd(lib, **kw):
    a = dict(x=FAKE, g=FAKE, w=FAKE, b=FAKE, y=FAKE, idx=FAKE, cnt=FAKE, off=FAKE, perm=FAKE,
             B=8, NH=5, H=128, NE=4, act=0, ws=FAKE, wsb=1 << 40)
    a.update(kw)
    return lib.moe_top1_fwd(a["x"], a["g"], a["w"], a["b"], a["y"], a["idx"], a["cnt"], a["off"], a["perm"],
                            a["B"], a["NH"], a["H"], a["NE"], a["act"], a["ws"], a["wsb"], None)


def test_fwd_validation(lib):
    assert _fwd(lib, x=None) == INVALID
    assert b"fused_ctx" in lib.moe_last_error()
    assert _fwd(lib, perm=None) == INVALID
    assert _fwd(lib, w=FAKE + 4) == INVALID  # misaligned
    assert b"aligned" in lib.moe_last_error()
    assert _fwd(lib, B=0) == INVALID
    assert _fwd(lib, NH=-1) == INVALID
    assert _fwd(lib, H=100) == UNSUPPORTED
    assert _fwd(lib, NE=100) == UNSUPPORTED
    assert _fwd(lib, act=3) == UNSUPPORTED
    assert _fwd(lib, ws=None) == WORKSPACE
    assert _fwd(lib, wsb=16) == WORKSPACE
    assert b"needed" in lib.moe_last_error()


def test_bwd_validation(lib):
    def bwd(**kw):
        a = dict(dy=FAKE, x=FAKE, w=FAKE, off=FAKE, perm=FAKE, dx=FAKE, dw=FAKE, db=FAKE, ws=FAKE, wsb=1 << 40,
                 H=128, NE=4)
        a.update(kw)
        return lib.moe_top1_bwd(a["dy"], a["x"], a["w"], a["off"], a["perm"], a["dx"], a["dw"], a["db"], 0,
                                8, 5, a["H"], a["NE"], 0, a["ws"], a["wsb"], None)
    assert bwd(dy=None) == INVALID
    assert bwd(db=None) == INVALID
    assert bwd(off=FAKE + 8) == INVALID
    assert bwd(H=32) == UNSUPPORTED
    assert bwd(wsb=0) == WORKSPACE


def test_fwd_aux_validation(lib):
    def fa(**kw):
        a = dict(x=FAKE, g=FAKE, w=FAKE, b=FAKE, y=FAKE, idx=FAKE, cnt=FAKE, off=FAKE, perm=FAKE, lam=0.01,
                 lam_dev=None, loss=FAKE, dg=FAKE, probs=None, H=128, NE=4, act=0, ws=FAKE, wsb=1 << 40)
        a.update(kw)
        return lib.moe_top1_fwd_aux(a["x"], a["g"], a["w"], a["b"], a["y"], a["idx"], a["cnt"], a["off"],
                                    a["perm"], a["lam"], a["lam_dev"], a["loss"], a["dg"], None, None, a["probs"],
                                    8, 5, a["H"], a["NE"], a["act"], a["ws"], a["wsb"], None)
    assert fa(x=None) == INVALID
    assert b"fused_ctx" in lib.moe_last_error()
    assert fa(perm=None) == INVALID
    assert fa(loss=None) == INVALID
    assert fa(dg=None) == INVALID
    assert fa(probs=FAKE + 4) == INVALID
    assert fa(lam=float("nan")) == INVALID
    assert b"lambda" in lib.moe_last_error()
    assert fa(lam=float("nan"), lam_dev=FAKE + 2, loss=None) == INVALID  # loss checked first
    assert fa(lam=float("nan"), lam_dev=FAKE + 2) == INVALID
    assert b"lambda_dev" in lib.moe_last_error()
    assert fa(H=96) == UNSUPPORTED
    assert fa(NE=65) == UNSUPPORTED
    assert fa(act=5) == UNSUPPORTED
    assert fa(ws=None) == WORKSPACE
    assert fa(wsb=16) == WORKSPACE


def test_aux_validation(lib):
    def aux(**kw):
        a = dict(g=FAKE, cnt=FAKE, lam=0.01, loss=FAKE, dg=FAKE, ws=FAKE, wsb=1 << 40, NE=4)
        a.update(kw)
        return lib.moe_aux_loss(a["g"], a["cnt"], a["lam"], a["loss"], a["dg"], None, None, None,
                                8, 5, a["NE"], a["ws"], a["wsb"], None)
    assert aux(g=None) == INVALID
    assert aux(loss=None) == INVALID
    assert aux(dg=None) == INVALID
    assert aux(lam=float("nan")) == INVALID
    assert aux(lam=float("inf")) == INVALID
    assert aux(NE=0) == INVALID
    assert aux(NE=65) == UNSUPPORTED
    assert aux(ws=None) == WORKSPACE
    assert aux(cnt=FAKE + 2) == INVALID


def test_route_validation(lib):
    assert lib.moe_top1_route(None, FAKE, FAKE, FAKE, FAKE, 8, 5, 4, FAKE, 1 << 40, None) == INVALID
    assert lib.moe_top1_route(FAKE, FAKE, FAKE, FAKE, FAKE, 8, 5, 4, FAKE, 4, None) == WORKSPACE


def test_launch_timer_validation(lib):
    assert lib.moe_set_launch_timer(99, FAKE, FAKE) == INVALID
    assert lib.moe_set_launch_timer(3, None, FAKE) == INVALID
    assert lib.moe_set_launch_timer(-1, None, None) == 0


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(2, 5, 64)
    with pytest.raises(ValueError):
        m.moe_top1_fwd(x, torch.zeros(2, 5, 4), torch.zeros(4, 64, 64), torch.zeros(4, 64), x,
                       torch.zeros(10, dtype=torch.int32), torch.zeros(4, dtype=torch.int32),
                       torch.zeros(5, dtype=torch.int32), torch.zeros(10, dtype=torch.int32),
                       workspace=torch.zeros(1 << 20, dtype=torch.uint8))


def test_lambda_entry_points_validation(lib):
    assert lib.moe_lambda_eff_update(None, 0.01, 0.09, 0.7, 8, FAKE, None) == INVALID
    assert lib.moe_lambda_eff_update(FAKE, 0.01, 0.09, 0.7, 8, None, None) == INVALID
    assert lib.moe_lambda_eff_update(FAKE + 2, 0.01, 0.09, 0.7, 8, FAKE, None) == INVALID
    assert lib.moe_lambda_eff_update(FAKE, 0.01, 0.09, 0.7, 1, FAKE, None) == UNSUPPORTED
    assert lib.moe_lambda_eff_update(FAKE, 0.01, 0.09, 0.0, 8, FAKE, None) == INVALID
    assert lib.moe_lambda_eff_update(FAKE, float("nan"), 0.09, 0.7, 8, FAKE, None) == INVALID
    assert lib.moe_aux_loss_lambda_dev(FAKE, FAKE, None, FAKE, FAKE, None, None, None, 8, 5, 4, FAKE, 1 << 40,
                                       None) == INVALID
    assert lib.moe_aux_loss_lambda_dev(None, FAKE, FAKE, FAKE, FAKE, None, None, None, 8, 5, 4, FAKE, 1 << 40,
                                       None) == INVALID


def test_next_rows_validation(lib):
    out = ctypes.c_size_t(0)
    assert lib.moe_reduce_axis0_workspace_bytes(0, 5, ctypes.byref(out)) == INVALID
    assert lib.moe_reduce_axis0_workspace_bytes(20480, 65536, ctypes.byref(out)) == 0 and out.value > 0
    assert lib.moe_reduce_axis0_workspace_bytes(10, 64, ctypes.byref(out)) == 0 and out.value == 0
    assert lib.moe_reduce_axis0(None, 4, 4, FAKE, None, 0, None) == INVALID
    assert lib.moe_reduce_axis0(FAKE + 4, 4, 4, FAKE, None, 0, None) == INVALID       # float4 path needs 16 B
    assert lib.moe_reduce_axis0(FAKE, 20480, 65536, FAKE, None, 0, None) == WORKSPACE
    assert lib.moe_horizon_mean_collapse_fwd(FAKE, FAKE, 4, 5, 6, 0, None) == UNSUPPORTED   # H % 4
    assert lib.moe_horizon_mean_collapse_bwd(FAKE, FAKE, 4, 5, 12, 1, None) == UNSUPPORTED  # H % 8 for bf16
    assert lib.moe_horizon_mean_collapse_fwd(None, FAKE, 4, 5, 64, 0, None) == INVALID
    assert lib.moe_top1_bwd_from_mean(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 8, 5, 128, 4, 1, FAKE,
                                      0, None) == WORKSPACE                              # bf16, no room
    assert lib.moe_top1_bwd_from_mean(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 8, 5, 128, 4, 2, FAKE,
                                      1 << 40, None) == UNSUPPORTED                      # unknown dtype
    assert lib.moe_softmax_ce_grad(FAKE, FAKE, FAKE, FAKE, 4, 5, 65, None) == UNSUPPORTED
    assert lib.moe_softmax_ce_grad(FAKE, None, FAKE, FAKE, 4, 5, 21, None) == INVALID
    assert lib.moe_softmax_ce_grad(FAKE, FAKE, FAKE, FAKE, 0, 5, 21, None) == INVALID


def test_probe_validation(lib):
    assert lib.moe_probe_mfma(2, 8, 10, FAKE, FAKE, None) == UNSUPPORTED               # unknown dtype
    assert lib.moe_probe_mfma(0, 0, 10, FAKE, FAKE, None) == INVALID                   # no workgroups
    assert lib.moe_probe_mfma(0, (1 << 20) + 1, 10, FAKE, FAKE, None) == INVALID
    assert lib.moe_probe_mfma(1, 8, 0, FAKE, FAKE, None) == INVALID                    # no iterations
    assert lib.moe_probe_mfma(0, 8, 10, None, FAKE, None) == INVALID
    assert lib.moe_probe_mfma(0, 8, 10, FAKE, FAKE + 4, None) == INVALID               # ticks need 8 B
    assert lib.moe_probe_copy(FAKE, FAKE + 8, 1024, None) == INVALID                   # 16-byte alignment
    assert lib.moe_probe_copy(FAKE, FAKE, 1000, None) == INVALID                       # multiple of 16
    assert lib.moe_probe_copy(None, FAKE, 1024, None) == INVALID
