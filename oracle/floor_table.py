"""Regenerates the precision-floor table of the bf16 path's design.

TEST INFRASTRUCTURE ONLY (it runs the oracle and the rounding-point
emulator, ``oracle.emulate``; nothing here is imported by the HIP path).

    python -m oracle.floor_table [--heads 2] [--workloads layer_2k train_4k ...]

For each bf16 workload at its full length it takes the first and the last
(b, h) head of the seeded inputs, runs the float64 oracle, and runs the
emulator at the design's rounding points (fp16 operands with the split-fp16
corner of 128 query rows per started 8192 positions), with no corner, and
with bf16 operands.  It prints, per tensor, reading A (max |err| / rms of the
tensor) and reading B (largest per-row error over the row's RMS) as a
markdown table.

The inputs come from ``bwd_rope_apply_amd/workloads.py``, the seeded input
generator both sides share (it holds none of the method's arithmetic); it is
loaded from its file so that the package's binding is not imported.
"""
from __future__ import annotations

import argparse
import importlib.util
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

from . import emulate as E
from . import ref as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def load_workloads():
    path = os.path.join(ROOT, "bwd_rope_apply_amd", "workloads.py")
    spec = importlib.util.spec_from_file_location("_floor_workloads", path)
    mod = importlib.util.module_from_spec(spec)
    sys.modules[spec.name] = mod
    spec.loader.exec_module(mod)
    return mod


def design_corner(N: int) -> int:
    """The design's exact corner: 128 query rows per started 8192 positions."""
    return 128 * max(1, (N + 8191) // 8192)


VARIANTS = [("fp16 + corner (design)", E.fp16, True), ("fp16, no corner", E.fp16, False),
            ("bf16 + corner", E.bf16, True)]
NAMES = ("O", "dQ", "dK", "dV")


def head_task(inp, wl, b, h, variant):
    """(variant index or -1 for the oracle, outputs) of one head."""
    sl = (slice(b, b + 1), slice(h, h + 1))
    q, k, v, do = (inp.f64(n)[sl] for n in ("q", "k", "v", "do"))
    if variant < 0:
        o, lse = R.ref_fwd(q, k, v, wl.base, inp.alpha, wl.causal)
        dq, dk, dv, da = R.ref_bwd(q, k, v, o, do, lse, wl.base, inp.alpha, wl.causal)
        return dict(O=o, dQ=dq, dK=dk, dV=dv, dalpha=da)
    _, rnd, corner = VARIANTS[variant]
    return E.emulate(q, k, v, do, wl.base, inp.alpha, wl.causal, rnd,
                     corner=design_corner(wl.N) if corner else 0)


def table(names, heads=2, workers=None):
    from threadpoolctl import threadpool_limits
    W = load_workloads()
    workers = workers or max(1, min(16, len(os.sched_getaffinity(0))))
    rows = []
    for name in names:
        wl = W.get(name)
        inp = W.make_inputs(wl)
        picks = [(0, 0), (wl.B - 1, wl.H - 1)][:heads]
        jobs = [(b, h, var) for b, h in picks for var in range(-1, len(VARIANTS))]
        t0 = time.time()
        with threadpool_limits(1):
            with ThreadPoolExecutor(min(workers, len(jobs))) as ex:
                outs = list(ex.map(lambda j: head_task(inp, wl, *j), jobs))
        res = {j: o for j, o in zip(jobs, outs)}
        ref = {n: np.concatenate([res[(b, h, -1)][n] for b, h in picks], axis=1) for n in NAMES}
        ref["dalpha"] = sum(res[(b, h, -1)]["dalpha"] for b, h in picks)
        for vi, (vname, _, _) in enumerate(VARIANTS):
            got = {n: np.concatenate([res[(b, h, vi)][n] for b, h in picks], axis=1) for n in NAMES}
            got["dalpha"] = sum(res[(b, h, vi)]["dalpha"] for b, h in picks)
            rows.append((name, vname, design_corner(wl.N), E.floors(got, ref)))
        print(f"# {name}: {len(picks)} heads, N={wl.N}, D={wl.D}, {time.time() - t0:.0f} s",
              file=sys.stderr, flush=True)
    return rows


def markdown(rows) -> str:
    out = ["| workload | rounding | corner R | O (A / B) | dQ (A / B) | dK (A / B) | dV (A / B) | dalpha (A) |",
           "|---|---|---|---|---|---|---|---|"]
    for name, vname, R_, fl in rows:
        cells = [f"{fl[n][0]:.4f} / {fl[n][1]:.4f}" for n in NAMES]
        r = R_ if "corner" in vname and "no corner" not in vname else 0
        out.append(f"| {name} | {vname} | {r} | " + " | ".join(cells) + f" | {fl['dalpha'][0]:.4f} |")
    return "\n".join(out)


def main():
    ap = argparse.ArgumentParser(description="precision floors of the bf16 path's rounding points")
    ap.add_argument("--heads", type=int, default=2, choices=(1, 2))
    ap.add_argument("--workloads", nargs="*", default=["layer_2k", "train_4k", "long_8k", "vlong_32k"])
    a = ap.parse_args()
    print(markdown(table(a.workloads, a.heads)))


if __name__ == "__main__":
    main()
