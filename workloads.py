"""Seeded synthetic inputs for the top-1 MoE gate.

This module only draws random numbers and rounds them to the storage dtype.
It contains none of the gate's arithmetic, so both the CPU oracle and the HIP
path can take their inputs from it without sharing any of the method.

Shapes follow the pages' tensors (page "11b96dac6a", summary and ARCHITECTURE):
  fused_ctx   [B, N_H, H]        activations
  gate_logits [B, N_H, N_E]      fp32
  W           [N_E, H_out, H_in] one [H, H] linear per expert
  b           [N_E, H]           fp32 bias
  d_out       [B, N_H, H]        upstream gradient of routed_ctx

Recipe (fixed, so every run and both sides see the same arrays):
  * rng = numpy.random.default_rng(seed), seed = 1000 + k for workload k.
  * Draw order: fused_ctx, gate_logits (base), per-expert logit offsets
    (large-stress workload only), W, b, d_out.
  * Normal and uniform variates are drawn in float64, in blocks of 2**24
    values, then rounded to fp32 (round to nearest even).  bf16 tensors are
    then rounded once more, fp32 -> bf16 with round to nearest even, and kept
    as uint16 bit patterns together with their exact fp32 widening.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Dict, Optional

import numpy as np

_BLOCK = 1 << 24


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    NH: int
    H: int
    NE: int
    act: str = "f32"              # "f32" or "bf16": dtype of fused_ctx, W, d_out, routed_ctx, d_fused_ctx
    lam: float = 0.01
    gate: str = "normal"          # "int" (uniform integers in [-2, 2]) or "normal"
    gate_std: float = 1.0
    gate_bias: Dict[int, float] = field(default_factory=dict)  # fixed per-expert logit offsets
    gate_offset_range: float = 0.0  # >0: per-expert offsets ~ U(-r, r), drawn after the base logits
    seed: int = 0

    @property
    def T(self) -> int:
        return self.B * self.NH


# The five workloads, numbered 1..5 (seed 1000 + k).
WORKLOADS: Dict[int, Workload] = {
    1: Workload("tiny_ref", B=64, NH=5, H=128, NE=4, gate="int", lam=0.01, seed=1001),
    2: Workload("pages_shape", B=4096, NH=5, H=128, NE=4, lam=0.01, seed=1002),
    3: Workload("imbalanced", B=16384, NH=5, H=128, NE=8, gate_bias={4: 2.5}, lam=0.05, seed=1003),
    4: Workload("wider_bf16", B=32768, NH=5, H=512, NE=8, act="bf16", lam=0.01, seed=1004),
    5: Workload("large_stress", B=131072, NH=8, H=256, NE=16, gate_std=1.5,
                gate_offset_range=1.0, lam=0.01, seed=1005),
}


def workload(k: int, **overrides) -> Workload:
    w = WORKLOADS[k]
    return replace(w, **overrides) if overrides else w


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest even) and return the uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _normal(rng, n: int, std: float = 1.0) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, _BLOCK):
        m = min(_BLOCK, n - s)
        out[s:s + m] = (rng.standard_normal(m) * std).astype(np.float32)
    return out


def _uniform(rng, n: int, lo: float, hi: float) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, _BLOCK):
        m = min(_BLOCK, n - s)
        out[s:s + m] = rng.uniform(lo, hi, m).astype(np.float32)
    return out


@dataclass
class Inputs:
    """Host arrays for one workload.

    Float tensors are fp32 arrays holding the stored values.  For bf16
    workloads the ``*_bits`` fields hold the uint16 patterns that go to the
    device, and the fp32 arrays hold their exact widening.
    """
    wl: Workload
    fused_ctx: np.ndarray
    gate_logits: np.ndarray
    W: np.ndarray
    b: np.ndarray
    d_out: np.ndarray
    fused_ctx_bits: Optional[np.ndarray] = None
    W_bits: Optional[np.ndarray] = None
    d_out_bits: Optional[np.ndarray] = None


def make_inputs(wl: Workload, seed: Optional[int] = None) -> Inputs:
    rng = np.random.default_rng(wl.seed if seed is None else seed)
    B, NH, H, NE, T = wl.B, wl.NH, wl.H, wl.NE, wl.T
    bound = 1.0 / np.sqrt(H)

    x = _normal(rng, T * H).reshape(B, NH, H)
    if wl.gate == "int":
        g = rng.integers(-2, 3, size=T * NE).astype(np.float32).reshape(B, NH, NE)
    else:
        g = _normal(rng, T * NE, wl.gate_std).reshape(B, NH, NE)
    if wl.gate_offset_range > 0.0:
        off = rng.uniform(-wl.gate_offset_range, wl.gate_offset_range, NE)
        g = (g.astype(np.float64) + off).astype(np.float32)
    for e, v in wl.gate_bias.items():
        g[..., e] = (g[..., e].astype(np.float64) + v).astype(np.float32)
    w = _uniform(rng, NE * H * H, -bound, bound).reshape(NE, H, H)
    bias = _uniform(rng, NE * H, -bound, bound).reshape(NE, H)
    dy = _normal(rng, T * H).reshape(B, NH, H)

    inp = Inputs(wl, x, np.ascontiguousarray(g), w, bias, dy)
    if wl.act == "bf16":
        inp.fused_ctx_bits = f32_to_bf16_bits(x)
        inp.W_bits = f32_to_bf16_bits(w)
        inp.d_out_bits = f32_to_bf16_bits(dy)
        inp.fused_ctx = bf16_bits_to_f32(inp.fused_ctx_bits)
        inp.W = bf16_bits_to_f32(inp.W_bits)
        inp.d_out = bf16_bits_to_f32(inp.d_out_bits)
    return inp


def custom(B: int, NH: int, H: int, NE: int, *, act: str = "f32", gate: str = "normal",
           lam: float = 0.01, seed: int = 7, **kw) -> Workload:
    """A small workload with the same distributions, for edge cases and tests."""
    return Workload(f"custom_{B}x{NH}x{H}x{NE}_{act}", B=B, NH=NH, H=H, NE=NE, act=act,
                    gate=gate, lam=lam, seed=seed, **kw)


@dataclass
class DeviceInputs:
    """Inputs drawn on the GPU (torch tensors), for sizes too large to draw on the host in the
    time a test has: same shapes, distributions and draw order as make_inputs, from torch's
    counter-based device generator instead of numpy's; bf16 tensors are rounded from fp32
    with round to nearest even (torch's conversion)."""
    wl: Workload
    fused_ctx: "object"
    gate_logits: "object"
    W: "object"
    b: "object"
    d_out: "object"


def make_inputs_device(wl: Workload, device="cuda", seed: Optional[int] = None) -> DeviceInputs:
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(wl.seed if seed is None else seed)
    B, NH, H, NE = wl.B, wl.NH, wl.H, wl.NE
    bound = 1.0 / float(np.sqrt(H))
    act = torch.bfloat16 if wl.act == "bf16" else torch.float32

    def normal(shape, std=1.0):
        t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        return t.mul_(std) if std != 1.0 else t

    def uniform(shape):
        return torch.rand(shape, generator=g, device=device, dtype=torch.float32).mul_(2 * bound).sub_(bound)

    x = normal((B, NH, H)).to(act)
    if wl.gate == "int":
        gl = torch.randint(-2, 3, (B, NH, NE), generator=g, device=device).to(torch.float32)
    else:
        gl = normal((B, NH, NE), wl.gate_std)
    if wl.gate_offset_range > 0.0:
        r = wl.gate_offset_range
        gl += torch.rand(NE, generator=g, device=device, dtype=torch.float32) * (2 * r) - r
    for e, v in wl.gate_bias.items():
        gl[..., e] += v
    w = uniform((NE, H, H)).to(act)
    bias = uniform((NE, H))
    dy = normal((B, NH, H)).to(act)
    return DeviceInputs(wl, x.contiguous(), gl.contiguous(), w.contiguous(), bias.contiguous(), dy.contiguous())
