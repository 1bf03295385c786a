"""Top-1 Mixture-of-Experts gate on MI355X (gfx950): Python binding of libmoe_top1.so.

The functions here carry the names of the C entry points in include/moe_top1.h and do
argument marshalling only: shapes are read from the tensors, device pointers and the
current HIP stream are passed through, and every step of the computation runs in the
library's HIP kernels.  There is no fallback: if the library or a GPU is missing, the
calls raise.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = [
    "load_library", "library_path", "moe_abi_version", "moe_workspace_bytes", "moe_top1_route",
    "moe_top1_fwd", "moe_top1_fwd_noalloc", "moe_top1_bwd", "moe_aux_loss", "moe_set_launch_timer", "moe_kernel_name",
    "moe_lambda_eff_update", "moe_aux_loss_lambda_dev", "moe_reduce_axis0", "moe_reduce_axis0_workspace_bytes",
    "moe_horizon_mean_collapse_fwd", "moe_horizon_mean_collapse_bwd", "moe_top1_bwd_from_mean",
    "moe_softmax_ce_grad", "moe_probe_mfma", "moe_probe_copy", "MoeError", "KERNELS", "DTYPE_F32", "DTYPE_BF16",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
DTYPE_F32, DTYPE_BF16 = 0, 1
KERNELS = ["route", "scan", "scatter", "fwd_gemm", "bwd_gemm", "reduce", "aux", "aux_final", "w_transpose",
           "lambda_update", "reduce_axis0", "collapse", "softmax_ce"]

_lib: Optional[ctypes.CDLL] = None


class MoeError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"[status {status}] {msg}")
        self.status = status


def library_path() -> str:
    return os.path.join(_PKG, "libmoe_top1.so")


def load_library() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m mixture_experts_top_amd.build` "
                          "or __graft_entry__.build()")
    # torch first: its HIP runtime (same soname) is then the one the library binds to,
    # so the process holds a single runtime and torch's device pointers are valid here.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    P, I64, I32, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    sig = {
        "moe_abi_version": ([], I32),
        "moe_status_string": ([I32], ctypes.c_char_p),
        "moe_last_error": ([], ctypes.c_char_p),
        "moe_kernel_name": ([I32], ctypes.c_char_p),
        "moe_workspace_bytes": ([I64, I64, I64, I64, I32, ctypes.POINTER(SZ)], I32),
        "moe_top1_route": ([P, P, P, P, P, I64, I64, I64, P, SZ, P], I32),
        "moe_top1_fwd": ([P, P, P, P, P, P, P, P, P, I64, I64, I64, I64, I32, P, SZ, P], I32),
        "moe_top1_fwd_noalloc": ([P, P, P, P, P, P, P, P, P, I64, I64, I64, I64, I32, P], I32),
        "moe_top1_bwd": ([P, P, P, P, P, P, P, P, I32, I64, I64, I64, I64, I32, P, SZ, P], I32),
        "moe_aux_loss": ([P, P, ctypes.c_float, P, P, P, P, P, I64, I64, I64, P, SZ, P], I32),
        "moe_set_launch_timer": ([I32, P, P], I32),
        "moe_lambda_eff_update": ([P, ctypes.c_float, ctypes.c_float, ctypes.c_float, I64, P, P], I32),
        "moe_aux_loss_lambda_dev": ([P, P, P, P, P, P, P, P, I64, I64, I64, P, SZ, P], I32),
        "moe_reduce_axis0_workspace_bytes": ([I64, I64, ctypes.POINTER(SZ)], I32),
        "moe_reduce_axis0": ([P, I64, I64, P, P, SZ, P], I32),
        "moe_horizon_mean_collapse_fwd": ([P, P, I64, I64, I64, I32, P], I32),
        "moe_horizon_mean_collapse_bwd": ([P, P, I64, I64, I64, I32, P], I32),
        "moe_top1_bwd_from_mean": ([P, P, P, P, P, P, P, P, I32, I64, I64, I64, I64, I32, P, SZ, P], I32),
        "moe_softmax_ce_grad": ([P, P, P, P, I64, I64, I64, P], I32),
        "moe_probe_mfma": ([I32, I64, I64, P, P, P], I32),
        "moe_probe_copy": ([P, P, I64, P], I32),
        "moe_top1_fwd_aux": ([P, P, P, P, P, P, P, P, P, ctypes.c_float, P, P, P, P, P, P,
                              I64, I64, I64, I64, I32, P, SZ, P], I32),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _lib = lib
    return lib


def _check(st: int):
    if st != 0:
        lib = load_library()
        raise MoeError(st, f"{lib.moe_status_string(st).decode()}: {lib.moe_last_error().decode()}")


def moe_abi_version() -> int:
    return load_library().moe_abi_version()


def moe_kernel_name(k: int) -> Optional[str]:
    r = load_library().moe_kernel_name(k)
    return r.decode() if r else None


def moe_workspace_bytes(B: int, NH: int, H: int, NE: int, act: int = DTYPE_F32) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().moe_workspace_bytes(B, NH, H, NE, act, ctypes.byref(out)))
    return out.value


# ------------------------------------------------------------------ tensor helpers

def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("all tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("all tensors must be contiguous")
    return t.data_ptr()


_raw_stream = None


def _stream(stream) -> Optional[int]:
    """The given stream's handle, else the current stream of the current device.  The raw
    lookup avoids building a Stream object on every call (a few microseconds each)."""
    global _raw_stream
    if stream is not None:
        return stream.cuda_stream
    import torch
    if _raw_stream is None:
        get = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        _raw_stream = (lambda: get(torch.cuda.current_device())) if get is not None else \
            (lambda: torch.cuda.current_stream().cuda_stream)
    return _raw_stream()


def _act(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return DTYPE_F32
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    raise ValueError(f"activation dtype must be float32 or bfloat16, got {t.dtype}")


def _scratch(nbytes, device, stream):
    """A temporary device buffer for one call.  torch's caching allocator ties a block to the
    stream it was allocated on; when the kernels run on another stream, record_stream keeps
    the block from being handed out again before that stream has run them."""
    import torch
    buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
    if stream is not None and stream != torch.cuda.current_stream(buf.device):
        buf.record_stream(stream)
    return buf


def _workspace(ws, B, NH, H, NE, act, device, stream=None):
    """A caller's workspace is passed with its size (the library rejects one too small);
    without one, a workspace of the required size is allocated for this call."""
    if ws is None:
        ws = _scratch(moe_workspace_bytes(B, NH, H, NE, act), device, stream)
    return ws, ws.numel() * ws.element_size()


def _shape3(t, name):
    sh = t.shape
    if len(sh) != 3:
        raise ValueError(f"{name} must be [B, N_H, *], got {tuple(sh)}")
    return sh[0], sh[1], sh[2]


def _expect(t, name, shape, dtype):
    """Host-side check that a buffer has exactly the shape and dtype the kernels assume."""
    if t is None:
        return
    if t.shape != shape:
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


# ------------------------------------------------------------------ entry points

def moe_top1_route(gate_logits, expert_idx, expert_counts, expert_offsets, perm, workspace=None, stream=None):
    import torch
    B, NH, NE = _shape3(gate_logits, "gate_logits")
    T = B * NH
    _expect(gate_logits, "gate_logits", (B, NH, NE), torch.float32)
    _expect(expert_idx, "expert_idx", (T,), torch.int32)
    _expect(expert_counts, "expert_counts", (NE,), torch.int32)
    _expect(expert_offsets, "expert_offsets", (NE + 1,), torch.int32)
    _expect(perm, "perm", (T,), torch.int32)
    ws, wsb = _workspace(workspace, B, NH, 64, NE, DTYPE_F32, gate_logits.device, stream)
    _check(load_library().moe_top1_route(_ptr(gate_logits), _ptr(expert_idx), _ptr(expert_counts),
                                         _ptr(expert_offsets), _ptr(perm), B, NH, NE, _ptr(ws), wsb,
                                         _stream(stream)))


def moe_top1_fwd(fused_ctx, gate_logits, W, b, routed_ctx, expert_idx, expert_counts, expert_offsets, perm,
                 workspace=None, stream=None):
    import torch
    B, NH, H = _shape3(fused_ctx, "fused_ctx")
    NE = int(gate_logits.shape[-1])
    T = B * NH
    act = _act(fused_ctx)
    _expect(gate_logits, "gate_logits", (B, NH, NE), torch.float32)
    _expect(W, "W", (NE, H, H), fused_ctx.dtype)
    _expect(b, "b", (NE, H), torch.float32)
    _expect(routed_ctx, "routed_ctx", (B, NH, H), fused_ctx.dtype)
    _expect(expert_idx, "expert_idx", (T,), torch.int32)
    _expect(expert_counts, "expert_counts", (NE,), torch.int32)
    _expect(expert_offsets, "expert_offsets", (NE + 1,), torch.int32)
    _expect(perm, "perm", (T,), torch.int32)
    ws, wsb = _workspace(workspace, B, NH, H, NE, act, fused_ctx.device, stream)
    _check(load_library().moe_top1_fwd(_ptr(fused_ctx), _ptr(gate_logits), _ptr(W), _ptr(b), _ptr(routed_ctx),
                                       _ptr(expert_idx), _ptr(expert_counts), _ptr(expert_offsets), _ptr(perm),
                                       B, NH, H, NE, act, _ptr(ws), wsb, _stream(stream)))


def moe_top1_fwd_noalloc(fused_ctx, gate_logits, W, b, routed_ctx, expert_idx, expert_counts, expert_offsets, perm,
                         stream=None):
    """moe_top1_fwd with its scratch in the library's per-device array: no workspace argument,
    nothing allocated (calls that overlap on one device race)."""
    import torch
    B, NH, H = _shape3(fused_ctx, "fused_ctx")
    NE = int(gate_logits.shape[-1])
    T = B * NH
    act = _act(fused_ctx)
    _expect(gate_logits, "gate_logits", (B, NH, NE), torch.float32)
    _expect(W, "W", (NE, H, H), fused_ctx.dtype)
    _expect(b, "b", (NE, H), torch.float32)
    _expect(routed_ctx, "routed_ctx", (B, NH, H), fused_ctx.dtype)
    _expect(expert_idx, "expert_idx", (T,), torch.int32)
    _expect(expert_counts, "expert_counts", (NE,), torch.int32)
    _expect(expert_offsets, "expert_offsets", (NE + 1,), torch.int32)
    _expect(perm, "perm", (T,), torch.int32)
    _check(load_library().moe_top1_fwd_noalloc(_ptr(fused_ctx), _ptr(gate_logits), _ptr(W), _ptr(b),
                                               _ptr(routed_ctx), _ptr(expert_idx), _ptr(expert_counts),
                                               _ptr(expert_offsets), _ptr(perm), B, NH, H, NE, act,
                                               _stream(stream)))


def moe_top1_fwd_aux(fused_ctx, gate_logits, W, b, routed_ctx, expert_idx, expert_counts, expert_offsets, perm,
                     lam, loss, d_gate_logits, frac=None, mean_prob=None, probs=None, lambda_dev=None,
                     workspace=None, stream=None):
    """moe_top1_fwd followed by the aux loss on the counts it wrote, in one call (lambda from
    `lambda_dev` on the device when given, else `lam`)."""
    import torch
    B, NH, H = _shape3(fused_ctx, "fused_ctx")
    NE = int(gate_logits.shape[-1])
    T = B * NH
    act = _act(fused_ctx)
    _expect(gate_logits, "gate_logits", (B, NH, NE), torch.float32)
    _expect(W, "W", (NE, H, H), fused_ctx.dtype)
    _expect(b, "b", (NE, H), torch.float32)
    _expect(routed_ctx, "routed_ctx", (B, NH, H), fused_ctx.dtype)
    _expect(expert_idx, "expert_idx", (T,), torch.int32)
    _expect(expert_counts, "expert_counts", (NE,), torch.int32)
    _expect(expert_offsets, "expert_offsets", (NE + 1,), torch.int32)
    _expect(perm, "perm", (T,), torch.int32)
    _expect(loss, "loss", (1,), torch.float32)
    _expect(d_gate_logits, "d_gate_logits", (B, NH, NE), torch.float32)
    _expect(frac, "frac", (NE,), torch.float32)
    _expect(mean_prob, "mean_prob", (NE,), torch.float32)
    _expect(probs, "probs", (B, NH, NE), torch.float32)
    _expect(lambda_dev, "lambda_dev", (1,), torch.float32)
    ws, wsb = _workspace(workspace, B, NH, H, NE, act, fused_ctx.device, stream)
    _check(load_library().moe_top1_fwd_aux(_ptr(fused_ctx), _ptr(gate_logits), _ptr(W), _ptr(b), _ptr(routed_ctx),
                                           _ptr(expert_idx), _ptr(expert_counts), _ptr(expert_offsets), _ptr(perm),
                                           float(lam), _ptr(lambda_dev), _ptr(loss), _ptr(d_gate_logits),
                                           _ptr(frac), _ptr(mean_prob), _ptr(probs), B, NH, H, NE, act, _ptr(ws),
                                           wsb, _stream(stream)))


def moe_top1_bwd(d_routed_ctx, fused_ctx, W, expert_offsets, perm, d_fused_ctx, d_W, d_b, accumulate_dx=False,
                 workspace=None, stream=None):
    import torch
    B, NH, H = _shape3(fused_ctx, "fused_ctx")
    NE = int(W.shape[0])
    T = B * NH
    act = _act(fused_ctx)
    _expect(d_routed_ctx, "d_routed_ctx", (B, NH, H), fused_ctx.dtype)
    _expect(W, "W", (NE, H, H), fused_ctx.dtype)
    _expect(expert_offsets, "expert_offsets", (NE + 1,), torch.int32)
    _expect(perm, "perm", (T,), torch.int32)
    _expect(d_fused_ctx, "d_fused_ctx", (B, NH, H), fused_ctx.dtype)
    _expect(d_W, "d_W", (NE, H, H), torch.float32)
    _expect(d_b, "d_b", (NE, H), torch.float32)
    ws, wsb = _workspace(workspace, B, NH, H, NE, act, fused_ctx.device, stream)
    _check(load_library().moe_top1_bwd(_ptr(d_routed_ctx), _ptr(fused_ctx), _ptr(W), _ptr(expert_offsets),
                                       _ptr(perm), _ptr(d_fused_ctx), _ptr(d_W), _ptr(d_b), int(bool(accumulate_dx)),
                                       B, NH, H, NE, act, _ptr(ws), wsb, _stream(stream)))


def moe_aux_loss(gate_logits, expert_counts, lam, loss, d_gate_logits, frac=None, mean_prob=None, probs=None,
                 workspace=None, stream=None):
    import torch
    B, NH, NE = _shape3(gate_logits, "gate_logits")
    _expect(gate_logits, "gate_logits", (B, NH, NE), torch.float32)
    _expect(expert_counts, "expert_counts", (NE,), torch.int32)
    _expect(loss, "loss", (1,), torch.float32)
    _expect(d_gate_logits, "d_gate_logits", (B, NH, NE), torch.float32)
    _expect(frac, "frac", (NE,), torch.float32)
    _expect(mean_prob, "mean_prob", (NE,), torch.float32)
    _expect(probs, "probs", (B, NH, NE), torch.float32)
    ws, wsb = _workspace(workspace, B, NH, 64, NE, DTYPE_F32, gate_logits.device, stream)
    _check(load_library().moe_aux_loss(_ptr(gate_logits), _ptr(expert_counts), float(lam), _ptr(loss),
                                       _ptr(d_gate_logits), _ptr(frac), _ptr(mean_prob), _ptr(probs),
                                       B, NH, NE, _ptr(ws), wsb, _stream(stream)))


def moe_lambda_eff_update(ent_ema, lambda_eff, NE, lambda_floor=0.01, lambda_max_extra=0.09,
                          entropy_target_frac=0.7, stream=None):
    import torch
    _expect(ent_ema, "ent_ema", (1,), torch.float32)
    _expect(lambda_eff, "lambda_eff", (1,), torch.float32)
    _check(load_library().moe_lambda_eff_update(_ptr(ent_ema), float(lambda_floor), float(lambda_max_extra),
                                                float(entropy_target_frac), int(NE), _ptr(lambda_eff),
                                                _stream(stream)))


def moe_aux_loss_lambda_dev(gate_logits, expert_counts, lambda_dev, loss, d_gate_logits, frac=None, mean_prob=None,
                            probs=None, workspace=None, stream=None):
    import torch
    B, NH, NE = _shape3(gate_logits, "gate_logits")
    _expect(gate_logits, "gate_logits", (B, NH, NE), torch.float32)
    _expect(expert_counts, "expert_counts", (NE,), torch.int32)
    _expect(lambda_dev, "lambda_dev", (1,), torch.float32)
    _expect(loss, "loss", (1,), torch.float32)
    _expect(d_gate_logits, "d_gate_logits", (B, NH, NE), torch.float32)
    _expect(frac, "frac", (NE,), torch.float32)
    _expect(mean_prob, "mean_prob", (NE,), torch.float32)
    _expect(probs, "probs", (B, NH, NE), torch.float32)
    ws, wsb = _workspace(workspace, B, NH, 64, NE, DTYPE_F32, gate_logits.device, stream)
    _check(load_library().moe_aux_loss_lambda_dev(_ptr(gate_logits), _ptr(expert_counts), _ptr(lambda_dev),
                                                  _ptr(loss), _ptr(d_gate_logits), _ptr(frac), _ptr(mean_prob),
                                                  _ptr(probs), B, NH, NE, _ptr(ws), wsb, _stream(stream)))


def moe_reduce_axis0_workspace_bytes(n_batch: int, n_tail: int) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().moe_reduce_axis0_workspace_bytes(n_batch, n_tail, ctypes.byref(out)))
    return out.value


def moe_reduce_axis0(inp, out, workspace=None, stream=None):
    """inp [n_batch, n_tail] fp32 -> out [n_tail]."""
    import torch
    if inp.dim() != 2:
        raise ValueError("inp must be [n_batch, n_tail]")
    n_batch, n_tail = (int(x) for x in inp.shape)
    _expect(inp, "inp", (n_batch, n_tail), torch.float32)
    _expect(out, "out", (n_tail,), torch.float32)
    need = moe_reduce_axis0_workspace_bytes(n_batch, n_tail)
    if workspace is None and need:
        workspace = _scratch(need, inp.device, stream)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().moe_reduce_axis0(_ptr(inp), n_batch, n_tail, _ptr(out), _ptr(workspace), wsb,
                                           _stream(stream)))


def moe_horizon_mean_collapse_fwd(x, ctx_mean, stream=None):
    B, NH, H = _shape3(x, "x")
    _expect(ctx_mean, "ctx_mean", (B, H), x.dtype)
    _check(load_library().moe_horizon_mean_collapse_fwd(_ptr(x), _ptr(ctx_mean), B, NH, H, _act(x), _stream(stream)))


def moe_horizon_mean_collapse_bwd(d_ctx_mean, d_x, stream=None):
    B, NH, H = _shape3(d_x, "d_x")
    _expect(d_ctx_mean, "d_ctx_mean", (B, H), d_x.dtype)
    _check(load_library().moe_horizon_mean_collapse_bwd(_ptr(d_ctx_mean), _ptr(d_x), B, NH, H, _act(d_x),
                                                        _stream(stream)))


def moe_top1_bwd_from_mean(d_ctx_mean, fused_ctx, W, expert_offsets, perm, d_fused_ctx, d_W, d_b,
                           accumulate_dx=False, workspace=None, stream=None):
    import torch
    B, NH, H = _shape3(fused_ctx, "fused_ctx")
    NE = int(W.shape[0])
    T = B * NH
    act = _act(fused_ctx)
    _expect(d_ctx_mean, "d_ctx_mean", (B, H), fused_ctx.dtype)
    _expect(W, "W", (NE, H, H), fused_ctx.dtype)
    _expect(expert_offsets, "expert_offsets", (NE + 1,), torch.int32)
    _expect(perm, "perm", (T,), torch.int32)
    _expect(d_fused_ctx, "d_fused_ctx", (B, NH, H), fused_ctx.dtype)
    _expect(d_W, "d_W", (NE, H, H), torch.float32)
    _expect(d_b, "d_b", (NE, H), torch.float32)
    ws, wsb = _workspace(workspace, B, NH, H, NE, act, fused_ctx.device, stream)
    _check(load_library().moe_top1_bwd_from_mean(_ptr(d_ctx_mean), _ptr(fused_ctx), _ptr(W), _ptr(expert_offsets),
                                                 _ptr(perm), _ptr(d_fused_ctx), _ptr(d_W), _ptr(d_b),
                                                 int(bool(accumulate_dx)), B, NH, H, NE, act, _ptr(ws), wsb,
                                                 _stream(stream)))


def moe_softmax_ce_grad(logits, labels, grad, ce, stream=None):
    import torch
    B, NH, A = _shape3(logits, "logits")
    _expect(logits, "logits", (B, NH, A), torch.float32)
    _expect(labels, "labels", (B, NH), torch.int32)
    _expect(grad, "grad", (B, NH, A), torch.float32)
    _expect(ce, "ce", (B, NH), torch.float32)
    _check(load_library().moe_softmax_ce_grad(_ptr(logits), _ptr(labels), _ptr(grad), _ptr(ce), B, NH, A,
                                              _stream(stream)))


def moe_probe_mfma(act, workgroups, iters, sink, ticks, stream=None):
    """Calibration MFMA loop (see moe_top1.h): sink [workgroups * 256] fp32, ticks
    [workgroups, 2] int64 on the GPU."""
    import torch
    _expect(sink, "sink", (workgroups * 256,), torch.float32)
    _expect(ticks, "ticks", (workgroups, 2), torch.int64)
    _check(load_library().moe_probe_mfma(act, workgroups, iters, _ptr(sink), _ptr(ticks), _stream(stream)))


def moe_probe_copy(src, dst, stream=None):
    """Calibration copy dst = src (same number of bytes, a multiple of 16)."""
    nb = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nb:
        raise ValueError("src and dst must hold the same number of bytes")
    _check(load_library().moe_probe_copy(_ptr(src), _ptr(dst), nb, _stream(stream)))


def moe_set_launch_timer(kernel, ev_start=None, ev_stop=None):
    """Bracket every launch of one kernel (name or MOE_KERNEL_* id) with two torch.cuda.Events;
    kernel=None clears."""
    lib = load_library()
    if kernel is None:
        _check(lib.moe_set_launch_timer(-1, None, None))
        return
    kid = KERNELS.index(kernel) if isinstance(kernel, str) else int(kernel)
    _check(lib.moe_set_launch_timer(kid, ev_start.cuda_event, ev_stop.cuda_event))
