"""The guards the kernels put on caller-provided routing (csrc/routing_guard.hpp), checked on
the host: the header's constexpr functions are compiled with g++ into a small driver that
forms every expert's range exactly as the device code does (clamped offsets, a running
maximum over the experts, then the count), and the ranges are checked against what the
kernels rely on: inside [0, T), disjoint, counts summing to at most T, tile and chunk counts
within the host's grid bounds -- and unchanged for routing the forward pass wrote.
(MHA wiring page "9170d24fe3", BUG CAUGHT DURING WIRING block: launches sized from numbers
that do not match the buffers read past their end.)"""
import os
import shutil
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "mixture_experts_top_amd", "csrc")

DRIVER = r"""
#include <cstdio>
#include "routing_guard.hpp"
// stdin: T NE o_0 .. o_NE per case, then K tokens; stdout: lo cnt per expert, then guarded tokens
int main() {
    int T, NE;
    while (std::scanf("%d %d", &T, &NE) == 2) {
        int o[65];
        for (int i = 0; i <= NE; ++i) std::scanf("%d", &o[i]);
        int run = 0;
        for (int e = 0; e < NE; ++e) {
            const int a = moe::guard_offset(o[e], T);
            run = a > run ? a : run;  // the wavefront's inclusive running maximum
            std::printf("%d %d\n", run, moe::guard_count(run, o[e + 1], T));
        }
        int k;
        std::scanf("%d", &k);
        for (int i = 0; i < k; ++i) {
            int v;
            std::scanf("%d", &v);
            std::printf("%d\n", moe::guard_token(v, T));
        }
    }
    return 0;
}
"""


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("g++ not available")
    d = tmp_path_factory.mktemp("guard")
    src = d / "guard.cpp"
    src.write_text(DRIVER)
    exe = d / "guard"
    subprocess.run([gxx, "-std=c++17", "-O1", "-I", HDR, str(src), "-o", str(exe)], check=True)
    return str(exe)


def run_cases(exe, cases):
    lines = []
    for T, off, toks in cases:
        lines.append(f"{T} {len(off) - 1} " + " ".join(str(int(v)) for v in off))
        lines.append(f"{len(toks)} " + " ".join(str(int(v)) for v in toks))
    out = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True, check=True).stdout
    vals = [int(x) for x in out.split()]
    res, p = [], 0
    for T, off, toks in cases:
        NE = len(off) - 1
        rng = np.array(vals[p:p + 2 * NE]).reshape(NE, 2)
        p += 2 * NE
        gt = np.array(vals[p:p + len(toks)])
        p += len(toks)
        res.append((rng, gt))
    return res


def check_invariants(T, rng, P=None, bm=128):
    lo, cnt = rng[:, 0], rng[:, 1]
    assert (lo >= 0).all() and (cnt >= 0).all() and (lo + cnt <= T).all()
    ends = lo + cnt
    assert (lo[1:] >= ends[:-1]).all(), "ranges overlap"
    assert cnt.sum() <= T
    NE = len(lo)
    assert sum((c + bm - 1) // bm for c in cnt) <= (T + bm - 1) // bm + NE  # row tiles within the grid
    if P is not None:  # d_W chunks within the P + N_E partial rows of the workspace
        assert sum(0 if c == 0 else (c * P + T - 1) // T for c in cnt) <= P + NE


def test_valid_routing_is_unchanged(driver):
    r = np.random.default_rng(0)
    cases = []
    for _ in range(200):
        NE = int(r.integers(1, 65))
        T = int(r.integers(1, 100000))
        counts = r.multinomial(T, r.dirichlet(np.ones(NE)))
        off = np.concatenate([[0], np.cumsum(counts)])
        toks = r.integers(0, T, 20)
        cases.append((T, off, toks))
    for (T, off, toks), (rng, gt) in zip(cases, run_cases(driver, cases)):
        np.testing.assert_array_equal(rng[:, 0], off[:-1])
        np.testing.assert_array_equal(rng[:, 1], np.diff(off))
        np.testing.assert_array_equal(gt, toks)


def test_garbage_routing_stays_in_bounds(driver):
    r = np.random.default_rng(1)
    cases = []
    for i in range(400):
        NE = int(r.integers(1, 65))
        T = int(r.integers(1, 50000))
        kind = i % 4
        if kind == 0:  # arbitrary integers, negative and huge included
            off = r.integers(-2 ** 31, 2 ** 31 - 1, NE + 1)
        elif kind == 1:  # offsets of another, larger shape
            counts = r.multinomial(3 * T, r.dirichlet(np.ones(NE)))
            off = np.concatenate([[0], np.cumsum(counts)])
        elif kind == 2:  # decreasing
            off = np.sort(r.integers(-10, T + 10, NE + 1))[::-1]
        else:  # a valid list with a few entries overwritten
            counts = r.multinomial(T, r.dirichlet(np.ones(NE)))
            off = np.concatenate([[0], np.cumsum(counts)])
            for j in r.integers(0, NE + 1, 3):
                off[j] = r.integers(-T, 2 * T + 1)
        toks = np.concatenate([r.integers(-2 ** 31, 2 ** 31 - 1, 10), [-1, T, T - 1, 0, 2 ** 31 - 1, -2 ** 31]])
        cases.append((T, off, toks))
    for (T, off, toks), (rng, gt) in zip(cases, run_cases(driver, cases)):
        check_invariants(T, rng, P=max(1, T // 128))
        assert ((gt >= 0) & (gt < T)).all()
        inside = (toks >= 0) & (toks < T)
        np.testing.assert_array_equal(gt[inside], toks[inside])
