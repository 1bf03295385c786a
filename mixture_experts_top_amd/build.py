"""Builds libmoe_top1.so for gfx950 with hipcc (no JIT, no hipRTC).

    python -m mixture_experts_top_amd.build [--jobs N]

Each .hip file under csrc/ is compiled to an object in _build/ (in parallel), then
linked into mixture_experts_top_amd/libmoe_top1.so with the gfx950 code objects
embedded.  Packed-fp32 VALU instructions are switched off for all device code.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmoe_top1.so")
# A second library with the bf16 W-stationary and resident-slice kernels switched off, so that
# every bf16 GEMM runs the tiled kernels: at H = 256 / 512 the default dispatch sends every size
# to one of the other two, and the parity tests compare the tiled ones through this build.
LIB_TILED = os.path.join(PKG, "libmoe_top1_tiled.so")
BUILD_TILED = os.path.join(ROOT, "_build_tiled")
TILED_DEFINES = ("MOE_BF16_WST=0", "MOE_BF16_WS_FWD=0")
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
]


def _compile(src: str, build_dir: str = BUILD, defines=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON, *[f"-D{d}" for d in defines], "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 8, verbose: bool = False, defines=(), out: str = LIB, build_dir: str = BUILD) -> str:
    """Compile and link.  `defines` override the kernels' compile-time tuning constants
    (for building variants elsewhere); the default build uses the values in the sources."""
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(lambda f: _compile(f, build_dir, defines), srcs))
    LIB_OUT = out
    tmp = LIB_OUT + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_OUT)
    if verbose:
        print(f"built {LIB_OUT}")
    return LIB_OUT


def build_tiled(jobs: int = 8, verbose: bool = False) -> str:
    """The bf16-tiled test library (see LIB_TILED)."""
    return build(jobs, verbose, defines=TILED_DEFINES, out=LIB_TILED, build_dir=BUILD_TILED)


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=8)
    a = ap.parse_args()
    build(a.jobs, verbose=True)
    sys.exit(0)
