"""Benchmark of the top-1 MoE gate hot path on one MI355X.

One step = moe_top1_fwd_aux (forward + load-balancing loss) + moe_top1_bwd over one batch
of synthetic tokens already resident in HBM (--separate-aux: moe_top1_fwd, moe_top1_bwd and
moe_aux_loss as three calls; same outputs, bit for bit).  Prints one JSON line (last line of stdout):

  value          routed tokens/s of the whole step (T / step time)
  roofline       the dominant kernel's algorithmic flops (or bytes) per launch divided
                 by its average duration, from HIP events that the library records at the
                 start and end of each of its launches inside the timed region, against the
                 MI355X peak
  cpu_baseline   the fp64 CPU oracle timed on this host on a bounded sample

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2|1|3|4|5] [--graph]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PEAK_TFLOPS = {"f32": 157.3, "bf16": 2516.6}
METRIC = "routed tokens/s fwd+bwd+aux (H=128, N_E=4, fp32); % of HBM/MFMA roofline"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(kernel, wl):
    """(amount, unit, bound) per launch: flops for the MFMA GEMMs, HBM bytes otherwise."""
    T, H, NE = wl.T, wl.H, wl.NE
    s = 2 if wl.act == "bf16" else 4
    if kernel == "fwd_gemm":
        return 2.0 * T * H * H, "flop", "mfma"
    if kernel == "bwd_gemm":  # dX and dW in one launch
        return 4.0 * T * H * H, "flop", "mfma"
    if kernel == "route":
        return T * NE * 4 + T * 4, "byte", "hbm"
    if kernel == "scatter":
        return T * 4 * 2, "byte", "hbm"
    if kernel == "aux":
        return 8.0 * T * NE, "byte", "hbm"
    if kernel == "reduce":
        return NE * H * H * 4 + NE * H * 4, "byte", "hbm"
    return 0.0, "byte", "hbm"


def pass_roofline_us(wl):
    """Roofline time (us) of fwd, bwd and aux at the MI355X peaks (algorithmic bytes/flops)."""
    T, H, NE = wl.T, wl.H, wl.NE
    s = 2 if wl.act == "bf16" else 4
    pk = PEAK_TFLOPS[wl.act] * 1e12
    bw = PEAK_HBM_GBS * 1e9
    fb = T * H * s * 2 + T * NE * 4 + NE * H * H * s + NE * H * 4 + T * 4
    ff = 2.0 * T * H * H + T * H
    bb = 3 * T * H * s + T * 4 + NE * H * H * s + NE * H * H * 4 + NE * H * 4
    bf = 4.0 * T * H * H + T * H
    ab = 8.0 * T * NE + NE * 4
    return {"fwd": max(fb / bw, ff / pk) * 1e6, "bwd": max(bb / bw, bf / pk) * 1e6, "aux": ab / bw * 1e6}


KERNEL_SOURCES = {"fwd_gemm": "gemm", "bwd_gemm": "gemm", "route": "route.hip", "scan": "route.hip",
                  "scatter": "route.hip", "reduce": "reduce.hip", "aux": "aux.hip", "aux_final": "aux.hip"}


def _code_only(text):
    """C++ source with comments removed and whitespace runs collapsed (string literals kept)."""
    import re
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c == '"':  # string literal, copied as is
            j = i + 1
            while j < n and text[j] != '"':
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return re.sub(r"\s+", " ", "".join(out)).strip()


def kernel_source_digest(kernel, act):
    """sha256 of the code (comments and whitespace left out) of the HIP source that holds a
    kernel and of the library's headers, which every source includes: matches stored counter
    readings to the code they were taken on."""
    import hashlib
    src = KERNEL_SOURCES[kernel]
    if src == "gemm":
        src = "gemm_bf16.hip" if act == "bf16" else "gemm_f32.hip"
    csrc = os.path.join(ROOT, "mixture_experts_top_amd", "csrc")
    h = hashlib.sha256()
    for name in [src] + sorted(f for f in os.listdir(csrc) if f.endswith(".hpp")):
        with open(os.path.join(csrc, name), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()


def measured_traffic(kernel, wl):
    """HBM bytes per launch from the stored rocprofv3 FETCH_SIZE / WRITE_SIZE readings, scaled
    by a plain copy's readings; None if there is none or the kernel source changed since."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{wl.name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_sha256") != kernel_source_digest(kernel, wl.act):
        return None
    return rec.get("traffic_bytes_per_launch")


def cpu_model():
    """The host CPU's model name (Linux /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(inp, budget_s=12.0, single_budget_s=4.0):
    """The oracle as it stands, on this host's cores, over a bounded sample of the workload;
    then the same sample with the BLAS library held to one thread."""
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        threadpool_limits = None
        cores = 1
    wl = inp.wl
    T = wl.T
    # sample: the first n tokens of the workload (whole batch if it fits the budget)
    n = T
    x, g, dy = inp.fused_ctx.reshape(T, -1), inp.gate_logits.reshape(T, -1), inp.d_out.reshape(T, -1)
    t0 = time.perf_counter()
    O.run_all(inp)
    one = time.perf_counter() - t0
    if one > budget_s:
        n = max(1024, int(T * budget_s / one / 2))

    def run(budget):
        reps, tok, el = 0, 0, 0.0
        while el < budget and reps < 1000:
            t0 = time.perf_counter()
            f = O.forward(x[:n], g[:n], inp.W, inp.b)
            O.backward(dy[:n], x[:n], inp.W, f.expert_idx)
            O.aux(g[:n], f.counts, wl.lam)
            el += time.perf_counter() - t0
            reps += 1
            tok += n
        return tok / el, reps, el

    rate, reps, el = run(budget_s)
    out = {"value": rate, "unit": "routed tokens/s", "cores": int(cores), "kind": "oracle",
           "sample": f"{reps} x fwd+bwd+aux over the first {n} of {T} tokens ({el:.1f} s, fp64 NumPy)",
           "cpu_model": cpu_model(), "host_threads": len(os.sched_getaffinity(0))}
    if threadpool_limits is not None and single_budget_s > 0:
        with threadpool_limits(limits=1, user_api="blas"):
            r1, reps1, el1 = run(single_budget_s)
        out["single_thread"] = {"value": r1, "unit": "routed tokens/s", "cores": 1,
                                "sample": f"{reps1} x the same sample ({el1:.1f} s)"}
    return out


def bench_row(args):
    """One JSON line for a row next to the gate: reduce_axis0, collapse, bwd_from_mean, softmax_ce, lambda."""
    import numpy as np
    import torch

    import mixture_experts_top_amd as moe
    from oracle import next_rows as N
    moe.load_library()
    dev = "cuda"
    g = torch.Generator(device=dev).manual_seed(1234)
    K = args.steps

    def timed(fn, reps=K, warm=args.warmup):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        return a.elapsed_time(b) / reps * 1e3, (t1 - t0) / reps * 1e3

    def cpu_time(fn, budget=args.cpu_budget / 2):
        reps, el = 0, 0.0
        while el < budget and reps < 200:
            t0 = time.perf_counter()
            fn()
            el += time.perf_counter() - t0
            reps += 1
        return el / reps, reps

    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        cores = 1
    row = args.row
    if row == "reduce_axis0":
        nb, nt = 20480, 65536  # n_batch = B*N_H (4096 x 5), n_tail = N_E*H*H (4 x 128 x 128)
        x = torch.randn(nb, nt, device=dev, generator=g)
        out = torch.empty(nt, device=dev)
        ws = torch.empty(max(moe.moe_reduce_axis0_workspace_bytes(nb, nt), 16), dtype=torch.uint8, device=dev)
        us, wall_ms = timed(lambda: moe.moe_reduce_axis0(x, out, workspace=ws))
        nbytes = nb * nt * 4 + nt * 4
        xs = x[:2048].cpu().numpy()
        ct, reps = cpu_time(lambda: N.reduce_axis0(xs))
        cpu = {"value": xs.nbytes / ct / 1e9, "unit": "GB/s", "cores": int(cores), "kind": "oracle",
               "sample": f"{reps} x fp64 column sum of the first 2048 of {nb} rows"}
        cfg = {"workload": "pages_moe_dw_scratch", "n_batch": nb, "n_tail": nt}
    elif row in ("collapse_fwd", "collapse_bwd"):
        B, NH, H = 131072, 8, 256
        x = torch.randn(B, NH, H, device=dev, generator=g)
        m = torch.randn(B, H, device=dev, generator=g)
        if row == "collapse_fwd":
            us, wall_ms = timed(lambda: moe.moe_horizon_mean_collapse_fwd(x, m))
            xs = x[:8192].cpu().numpy()
            ct, reps = cpu_time(lambda: N.horizon_mean_fwd(xs))
        else:
            us, wall_ms = timed(lambda: moe.moe_horizon_mean_collapse_bwd(m, x))
            ms_ = m[:8192].cpu().numpy()
            ct, reps = cpu_time(lambda: N.horizon_mean_bwd(ms_, NH))
        nbytes = B * NH * H * 4 + B * H * 4
        cpu = {"value": (8192 * (NH + 1) * H * 8) / ct / 1e9, "unit": "GB/s (fp64)", "cores": int(cores),
               "kind": "oracle", "sample": f"{reps} x the first 8192 of {B} batch rows"}
        cfg = {"workload": "large_stress_shape", "B": B, "N_H": NH, "H": H, "act": "f32"}
    elif row == "softmax_ce":
        B, NH, A = 131072, 8, 21
        z = torch.randn(B, NH, A, device=dev, generator=g) * 3
        lab = torch.randint(0, A, (B, NH), device=dev, generator=g, dtype=torch.int32)
        lab[:, -1] = -1
        grad = torch.empty_like(z)
        ce = torch.empty(B, NH, device=dev)
        us, wall_ms = timed(lambda: moe.moe_softmax_ce_grad(z, lab, grad, ce))
        nbytes = B * NH * (A * 8 + 8)
        zs, ls = z[:4096].cpu().numpy(), lab[:4096].cpu().numpy()
        ct, reps = cpu_time(lambda: N.softmax_ce(zs, ls))
        cpu = {"value": 4096 * NH / ct, "unit": "rows/s", "cores": int(cores), "kind": "oracle",
               "sample": f"{reps} x the first 4096 of {B} batch rows (x{NH} horizons)"}
        cfg = {"workload": "softmax_ce_21_atoms", "B": B, "N_H": NH, "A": A}
    else:
        raise SystemExit(f"unknown --row {row}")
    achieved = nbytes / (us * 1e-6) / 1e9
    out = {"metric": f"{row} HBM throughput", "value": achieved, "unit": "GB/s", "n_gpus": 1, "steps": K,
           "warmup": args.warmup, "ms_per_step": us / 1e3, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f32", "data": "synthetic (seeded torch generator)", "config": cfg,
           "roofline": {"bound": "hbm", "kernel": row, "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": achieved / PEAK_HBM_GBS, "traffic": None, "avg_launch_us": us,
                        "per_launch": f"{nbytes:.4g} byte"},
           "wall_ms_per_call": wall_ms, "cpu_baseline": cpu}
    print(json.dumps(out), flush=True)


def measure_gate(wl, d, o, args, K, warmup, cold_reps, survey=True, kernel=None):
    """Times K steps of the gate's hot path on the resident inputs d (outputs and workspace o):
    warm-up, a per-kernel survey that finds the dominant kernel (outside the timed region), the
    timed region with that kernel's own start/end events in every `--timer-every`-th step, and
    (cold_reps > 0) steps that each follow a large write evicting L2 and the Infinity Cache,
    with the step and the dominant kernel timed."""
    import numpy as np
    import torch

    import mixture_experts_top_amd as moe
    from mixture_experts_top_amd import runner as gpu_run
    stream = torch.cuda.current_stream()
    aux_stream = torch.cuda.Stream() if args.aux_stream else None  # default priority

    def step():  # the optional probs output is not requested: the aux pass writes dG only
        gpu_run.step(d, o, probs=False, aux_stream=aux_stream, fused=not args.separate_aux)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    def ev():
        return torch.cuda.Event(enable_timing=True)

    # per-kernel averages (outside the timed region) to find the dominant kernel
    nk = 10
    kern_us = {}
    gate_kernels = ["route", "scan", "scatter", "fwd_gemm", "bwd_gemm", "reduce", "aux", "aux_final"]
    for k in (gate_kernels if survey else []):
        evs = [(ev(), ev()) for _ in range(nk)]
        marks = [ev() for _ in range(nk)]
        for a, b in evs:
            a.record(); b.record()
        torch.cuda.synchronize()
        for (a, b), m in zip(evs, marks):
            m.record()
            moe.moe_set_launch_timer(k, a, b)
            step()
            moe.moe_set_launch_timer(None)
            for _ in range(max(1, args.timer_every) - 1):  # the same sampling as the timed region
                step()
        torch.cuda.synchronize()
        # a kernel this shape does not launch leaves its events at their earlier timestamps
        vals = [a.elapsed_time(b) for (a, b), m in zip(evs, marks) if m.elapsed_time(a) >= 0]
        if vals:
            kern_us[k] = float(np.mean(vals) * 1e3)
    if kernel:
        dom = kernel
    elif kern_us:
        dom = max((k for k in kern_us if k in ("fwd_gemm", "bwd_gemm", "aux", "reduce")), key=lambda k: kern_us[k])
    else:
        dom = "fwd_gemm"

    graph = None
    if args.graph:
        s = torch.cuda.Stream()
        s.wait_stream(stream)
        with torch.cuda.stream(s):
            step()
        stream.wait_stream(s)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(warmup):
            graph.replay()
        torch.cuda.synchronize()

    # timed region: K steps; the dominant kernel carries a pair of events in every
    # `--timer-every`-th step (each pair adds its own GPU commands to the step it sits in)
    every = max(1, args.timer_every)
    timed = [i for i in range(K) if i % every == 0]
    evs = {i: (ev(), ev()) for i in timed}
    for a, b in evs.values():
        a.record(); b.record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        if graph is not None:
            graph.replay()
        else:
            if i in evs:
                moe.moe_set_launch_timer(dom, *evs[i])
            elif i - 1 in evs:
                moe.moe_set_launch_timer(None)
            step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    moe.moe_set_launch_timer(None)
    ms = (t1 - t0) / K * 1e3
    if graph is None:
        dom_us = float(np.mean([a.elapsed_time(b) for a, b in evs.values()]) * 1e3)
    else:
        dom_us = kern_us.get(dom, float("nan"))

    # cold caches: the inputs are still in HBM, but a large write before each step evicts them
    # from L2 and the 256 MB Infinity Cache first; the step and its dominant kernel are timed
    cold = None
    if cold_reps > 0 and args.cold_mib > 0 and graph is None:
        flush = torch.empty(args.cold_mib << 18, dtype=torch.float32, device="cuda")
        # the steps alone first (a kernel timer adds work to the step it sits in), then as many
        # again with the dominant kernel's own start / end events
        evc = [(ev(), ev()) for _ in range(cold_reps)]
        evk = [(ev(), ev()) for _ in range(cold_reps)]
        for c, e in evk:
            c.record(); e.record()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(evc):
            flush.fill_(float(i))
            a.record()
            step()
            b.record()
        for i, (c, e) in enumerate(evk):
            flush.fill_(float(i))
            moe.moe_set_launch_timer(dom, c, e)
            step()
            moe.moe_set_launch_timer(None)
        torch.cuda.synchronize()
        cold_us = sorted(a.elapsed_time(b) * 1e3 for a, b in evc)
        cold_k = sorted(c.elapsed_time(e) * 1e3 for c, e in evk)
        cold = {"median_us": cold_us[cold_reps // 2], "min_us": cold_us[0], "flush_mib": args.cold_mib,
                "routed_tokens_per_s": wl.T / (cold_us[cold_reps // 2] * 1e-6), "steps": cold_reps,
                "kernel": dom, "kernel_median_us": cold_k[cold_reps // 2]}
        del flush
    return {"ms": ms, "dom": dom, "dom_us": dom_us, "kern_us": kern_us, "timed_launches": len(evs) if graph is None
            else 0, "graph": graph is not None, "aux_stream": aux_stream is not None, "cold": cold, "step": step}


def kernel_roofline(dom, dom_us, wl):
    amount, unit, bound = algorithmic(dom, wl)
    if bound == "mfma":
        achieved = amount / (dom_us * 1e-6) / 1e12
        return bound, achieved, PEAK_TFLOPS[wl.act], "TFLOP/s", amount, unit
    achieved = amount / (dom_us * 1e-6) / 1e9
    return bound, achieved, PEAK_HBM_GBS, "GB/s", amount, unit


def largest_config(args):
    """The large-stress workload (1,048,576 tokens, H = 256, N_E = 16, fp32), the largest
    configuration the headline target is quoted on: its step, dominant kernel and roofline
    fractions, measured the same way as the headline (a sub-record of the one JSON line)."""
    import torch

    import workloads
    from mixture_experts_top_amd import runner as gpu_run
    wl = workloads.workload(5)
    log(f"[bench] largest config: {wl}")
    d = gpu_run.upload(workloads.make_inputs(wl))
    o = gpu_run.Buffers(d, poison=False)
    m = measure_gate(wl, d, o, args, K=args.largest_steps, warmup=3, cold_reps=5)
    roof = pass_roofline_us(wl)
    bound, achieved, peak, runit, amount, unit = kernel_roofline(m["dom"], m["dom_us"], wl)
    out = {"workload": wl.name, "B": wl.B, "N_H": wl.NH, "H": wl.H, "N_E": wl.NE, "T": wl.T, "act": wl.act,
           "steps": args.largest_steps, "ms_per_step": m["ms"], "routed_tokens_per_s": wl.T / (m["ms"] * 1e-3),
           "step_roofline_us": sum(roof.values()), "step_roofline_frac": sum(roof.values()) / (m["ms"] * 1e3),
           "kernel": m["dom"], "kernel_avg_us": m["dom_us"], "kernel_achieved": achieved, "kernel_peak": peak,
           "kernel_unit": runit, "kernel_frac": achieved / peak, "kernel_timed_launches": m["timed_launches"],
           "kernel_traffic": measured_traffic(m["dom"], wl), "kernels_avg_us": m["kern_us"],
           "cold_cache_step": m["cold"]}
    if m["cold"]:
        kb = kernel_roofline(m["dom"], m["cold"]["kernel_median_us"], wl)
        out["cold_cache_step"]["kernel_frac"] = kb[1] / kb[2]
        out["cold_cache_step"]["step_roofline_frac"] = sum(roof.values()) / m["cold"]["median_us"]
    del d, o
    torch.cuda.empty_cache()
    return out


def measure_peaks(wgs=1024, iters=20000, copy_mib=1024, reps=5):
    """What the chip delivers on this machine, beside the spec-sheet peaks the roofline fractions
    divide by: the library's MFMA loop (four independent chains per wavefront, 4 wavefronts
    per workgroup, 4 workgroups per CU) in fp32 and bf16, the shader clock during it, and the
    STREAM copy.  Best of `reps` timed launches each."""
    import torch

    import mixture_experts_top_amd as moe

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        best = None
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            t = a.elapsed_time(b) * 1e-3
            best = t if best is None else min(best, t)
        return best

    out = {}
    sink = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    ticks = torch.empty(wgs, 2, dtype=torch.int64, device="cuda")
    for act, name, per in ((moe.DTYPE_F32, "f32", 4096), (moe.DTYPE_BF16, "bf16", 32768)):
        it = iters if act == moe.DTYPE_F32 else iters * 4
        t = timed(lambda: moe.moe_probe_mfma(act, wgs, it, sink, ticks))
        flops = wgs * 4 * it * 4 * per
        tk = ticks.cpu().double()
        ratio = float((tk[:, 0] / tk[:, 1]).median())
        out[f"mfma_{name}_tflops"] = flops / t / 1e12
        out[f"mfma_{name}_frac_of_spec"] = flops / t / 1e12 / PEAK_TFLOPS[name]
        # clock64 / wall_clock64 ticks; the constant clock (s_memrealtime) runs at 100 MHz
        out[f"shader_clock_ghz_during_{name}"] = ratio * 0.1
    n = (copy_mib << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    t = timed(lambda: moe.moe_probe_copy(src, dst))
    out["copy_gbs"] = 2 * n * 4 / t / 1e9
    out["copy_frac_of_spec"] = out["copy_gbs"] / PEAK_HBM_GBS
    out["copy_bytes"] = 2 * n * 4
    del src, dst, sink, ticks
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--graph", action="store_true", help="replay the step as one captured HIP graph")
    ap.add_argument("--aux-stream", action="store_true",
                    help="run the auxiliary loss on a second stream, overlapping the backward (default: "
                         "after it, on one stream; the cross-stream join costs more than it hides at the "
                         "pages' shape)")
    ap.add_argument("--separate-aux", action="store_true",
                    help="make the forward, backward and aux-loss calls one by one instead of "
                         "moe_top1_fwd_aux + moe_top1_bwd")
    ap.add_argument("--cold-mib", type=int, default=512,
                    help="also time steps that each follow a write of this many MiB (evicting L2 and the "
                         "256 MB Infinity Cache); 0 skips them")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--cpu-single-budget", type=float, default=4.0,
                    help="seconds of the single-thread oracle timing (0 skips it)")
    ap.add_argument("--largest", choices=["auto", "none"], default="auto",
                    help="auto: also measure the large-stress workload (sub-record largest_config) when the "
                         "headline workload is another one")
    ap.add_argument("--largest-steps", type=int, default=20)
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run a plain device copy of this size first (counter calibration under rocprofv3 --pmc)")
    ap.add_argument("--skip-kernel-survey", action="store_true",
                    help="do not time every kernel first; time --kernel in the timed region")
    ap.add_argument("--kernel", default=None, help="kernel timed live in the timed region (default: the slowest)")
    ap.add_argument("--timer-every", type=int, default=5,
                    help="time the dominant kernel with HIP events in every n-th step of the timed region")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the MFMA-loop / copy calibration (sub-record peaks)")
    ap.add_argument("--row", default="gate",
                    help="gate (default) | reduce_axis0 | collapse_fwd | collapse_bwd | softmax_ce")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import mixture_experts_top_amd as moe
    import workloads
    from mixture_experts_top_amd import runner as gpu_run

    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    if args.row != "gate":
        bench_row(args)
        return
    moe.load_library()
    wl = workloads.workload(args.workload)
    log(f"[bench] workload {args.workload}: {wl}")
    inp = workloads.make_inputs(wl)
    d = gpu_run.upload(inp)
    o = gpu_run.Buffers(d, poison=False)

    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] calibration copy: {args.calib_copy_mib} MiB read + {args.calib_copy_mib} MiB written, 3 launches")
        del src, dst

    m = measure_gate(wl, d, o, args, K=args.steps, warmup=args.warmup, cold_reps=20,
                     survey=not args.skip_kernel_survey, kernel=args.kernel)
    ms, dom, dom_us, kern_us = m["ms"], m["dom"], m["dom_us"], m["kern_us"]
    log("[bench] kernel avg us: " + ", ".join(f"{k}={v:.2f}" for k, v in kern_us.items()) + f"; dominant={dom}")
    bound, achieved, peak, runit, amount, unit = kernel_roofline(dom, dom_us, wl)

    # per-pass times (eager, after the timed region)
    def time_pass(fn, n=20):
        fn()  # the first launch of a kernel in the process loads its code object
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n * 1e3

    pass_us = {"fwd": time_pass(lambda: gpu_run.fwd(d, o)), "bwd": time_pass(lambda: gpu_run.bwd(d, o)),
               "aux": time_pass(lambda: gpu_run.aux(d, o, probs=False)),
               "fwd+aux (one call)": time_pass(lambda: gpu_run.fwd_aux(d, o, probs=False))}
    roof = pass_roofline_us(wl)
    step_roof_frac = sum(roof.values()) / (ms * 1e3)
    cold = m["cold"]
    if cold:
        kb = kernel_roofline(dom, cold["kernel_median_us"], wl)
        cold["kernel_frac"] = kb[1] / kb[2]
        cold["step_roofline_frac"] = sum(roof.values()) / cold["median_us"]
    del d, o
    torch.cuda.empty_cache()

    largest = None
    if args.largest == "auto" and args.workload != 5 and not args.graph:
        largest = largest_config(args)
        log(f"[bench] largest config: {largest['ms_per_step'] * 1e3:.1f} us/step, step frac "
            f"{largest['step_roofline_frac']:.3f}, {largest['kernel']} frac {largest['kernel_frac']:.3f}")

    peaks = None if args.no_peaks else measure_peaks()
    if peaks:
        log("[bench] peaks: " + ", ".join(f"{k}={v:.4g}" for k, v in peaks.items()))
    cpu = None if args.no_cpu_baseline else cpu_baseline(inp, args.cpu_budget, args.cpu_single_budget)
    T = wl.T
    out = {
        "metric": METRIC,
        "value": T / (ms * 1e-3),
        "unit": "routed tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.act,
        "data": "synthetic (seeded; see workloads.py)",
        "config": {"workload": wl.name, "B": wl.B, "N_H": wl.NH, "H": wl.H, "N_E": wl.NE, "T": T,
                   "lambda": wl.lam, "act": wl.act, "launch": "hip-graph" if m["graph"] else "eager",
                   "streams": 2 if m["aux_stream"] else 1,
                   "calls": ("fwd, bwd, aux" if args.separate_aux or m["aux_stream"] else "fwd_aux, bwd"),
                   "parallelism": "single GPU"},
        "roofline": {"bound": bound, "kernel": dom, "achieved": achieved, "peak": peak, "unit": runit,
                     "frac": achieved / peak, "traffic": measured_traffic(dom, wl), "avg_launch_us": dom_us,
                     "timed_launches": m["timed_launches"], "per_launch": f"{amount:.4g} {unit}"},
        "step_roofline_frac": step_roof_frac,
        "pass_us": pass_us,
        "cold_cache_step": cold,
        "pass_roofline_us": roof,
        "kernel_avg_us": kern_us,
        "largest_config": largest,
        "peaks": peaks,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
