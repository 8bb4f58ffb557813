#!/usr/bin/env python3
"""Throughput of exact causal RoPE attention, forward + backward (dQ, dK, dV
and d alpha), on one MI355X, through the library's C ABI.

One step = the forward pass and the backward pass of the whole workload
(default: B=1, H=32, N=8192, D=128, bf16 inputs, causal, base 1e4, alpha ~
U[-1, 0.5]) with inputs resident in device memory.  Prints one JSON line.

Throughput is algorithmic: 6 B H N^2 D flops per step (the two forward
products and the four backward products over the causal half), the standard
count for causal attention training; recomputation of scores in the backward
is not counted (the FlashAttention convention, which adds it, 7 B H N^2 D, is
reported beside it).  The step time is the host's clock around the timed
steps, bracketed by device synchronisations.  The timed step is the forward
in one call and the backward in four (the dK/dV kernel alone in one of
them), so the timed work is exactly the full forward + backward; HIP events
on the stream the library launches on (torch's current stream) bracket the
dK/dV call in every timed step, for the roofline, and nothing else (each
event record costs the GPU a few microseconds).  Untimed steps afterwards
repeat the timed step with an event before every call (calls_ms, events_ms),
and run every kernel in its own call for the per-kernel breakdown
(stages_ms_serial).
One workspace serves both passes: the backward reuses the forward's rotated
fp16 planes and frequency table (saved activations) and prepares only dO
and D.

--gram times Gram-threshold token selection instead (see bench_gram).

--retrieved K times block-list attention instead (each 128-row query block
sees its own block and K seeded key blocks, the exact part of Multipole
Semantic Attention); flops then count the visible pairs only.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_TFLOPS = 2516.6   # fp16 / bf16 dense matrix cores: 256 CU x 2.4 GHz x 4096 flop/clk
HBM_GBS = 8000.0
FP32_MFMA_TFLOPS = 157.3     # fp32 matrix cores: 256 CU x 256 flop/clk x 2.4 GHz (the vector rate too)
METRIC = "causal RoPE-attn fwd+bwd TFLOP/s and % bf16 MFMA peak, n=8192 d_h=128"

# Stage bits of the C ABI (rope_attn_stage)
PREP, EXACT, MAIN, DKDV, DQ, DALPHA, PREP_GRAD = 1, 2, 4, 8, 16, 32, 64
# The timed step: the whole forward in one call, the backward in four calls,
# split where a kernel is timed on its own: prep (PREP_GRAD: only the dO maxima,
# the scaled dO plane and D, reusing the forward's table and operand planes
# from the shared workspace); dK/dV (which also writes the dS panels); dQ (from
# the panels, with the split-operand corner's backward as its last
# workgroups); the d alpha reduction.  EXACT is the float32 path: with bf16
# inputs it does nothing, with fp32 inputs it is the whole pass.
FWD_CALLS = [("fwd", PREP | EXACT | MAIN)]
BWD_CALLS = [("bwd_prep", PREP_GRAD | EXACT), ("bwd_dkdv", DKDV), ("bwd_dq", DQ),
             ("bwd_dalpha", DALPHA)]


def stage_lists(dtype):
    """Every kernel in its own call (serial), timed after the timed step for
    the breakdown; the EXACT stage only where it runs (fp32 inputs)."""
    if dtype == "bf16":
        return ([("fwd_prep", PREP), ("fwd_main", MAIN)],
                [("bwd_prep", PREP_GRAD), ("bwd_dkdv", DKDV), ("bwd_dq", DQ),
                 ("bwd_dalpha", DALPHA)])
    return ([("fwd_prep", PREP), ("fwd_exact", EXACT)],
            [("bwd_prep", PREP_GRAD), ("bwd_exact", EXACT), ("bwd_dalpha", DALPHA)])


# algorithmic products of the dominant matrix-core kernel (units of B H N^2 D
# flops, causal): dV, dP and dK
DOMINANT = ("bwd_dkdv", "dkdv_kernel", 3.0)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long_8k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--unrotated-pairs", type=int, default=0,
                    help="frequency-schedule option: leave the slowest bands unrotated (partial "
                         "RoPE; D/8 is LeRoPE's p-RoPE baseline)")
    ap.add_argument("--scale", type=float, default=0.0,
                    help="frequency-schedule option: softmax scale (0 = 1/sqrt(D))")
    ap.add_argument("--pos-offset", type=int, default=0,
                    help="frequency-schedule option: position of row 0")
    ap.add_argument("--retrieved", type=int, default=-1,
                    help="block-list attention: key blocks retrieved per 128-row query block "
                         "(seeded, uniform among the blocks it may see); -1 = dense")
    ap.add_argument("--min-workspace", action="store_true",
                    help="the smallest backward workspace: no dS panels, dQ recomputes the scores")
    ap.add_argument("--gram", action="store_true",
                    help="time Gram-threshold token selection (and one cascade step) instead")
    ap.add_argument("--gram-workload", default="gram_8k")
    ap.add_argument("--traffic", default=os.path.join(ROOT, "profiles", "traffic_long_8k.json"),
                    help="JSON with measured HBM bytes per launch of the MFMA kernels (used only "
                         "if it was taken on the current kernel source)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 256 MiB device copy 3 times (reference for the "
                         "FETCH_SIZE / WRITE_SIZE counters under rocprofv3 --pmc)")
    return ap.parse_args()


KERNEL_SOURCES = ("mfma.hip", "tile.h", "corner.h", "common.h")


def kernel_source_hash() -> str:
    """sha256 over the sources of the MFMA attention kernels, in order."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "bwd_rope_apply_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(path: str, stage: str, workload: str):
    """HBM bytes per launch of `stage` from a counter summary, or None if the
    summary is missing, covers another workload or was taken on other
    kernel source."""
    if not path or not os.path.exists(path):
        return None
    t = json.load(open(path))
    if t.get("workload") != workload or t.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return t.get("bytes_per_launch", {}).get(stage)


def host_blas():
    """(threads, BLAS library) of numpy's thread pool on this host."""
    import numpy  # noqa: F401  (loads the BLAS that threadpoolctl then reports)
    try:
        from threadpoolctl import threadpool_info
        info = [i for i in threadpool_info() if i.get("user_api") == "blas"] or threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
        lib = ",".join(sorted({str(i.get("internal_api", "?")) for i in info})) or "?"
        return int(threads), lib
    except Exception:  # threadpoolctl is optional
        return len(os.sched_getaffinity(0)), "?"


def device_info():
    """CU count and name of cuda:0, and the dense fp16/bf16 matrix peak
    recomputed from the CU count at the 2.4 GHz the published peak uses."""
    import torch
    props = torch.cuda.get_device_properties(0)
    cus = int(props.multi_processor_count)
    return {"name": props.name, "gcn_arch": getattr(props, "gcnArchName", "?"), "cus": cus,
            "peak_fp16_tflops_at_2p4ghz": round(cus * 4 * 1024 * 2.4e9 / 1e12, 1)}


def clock_sample(run_kernel, wall_ms: float = 0.8):
    """Shader clock (GHz) of one CU: a one-wave probe kernel counts shader
    cycles over a fixed wall-clock interval.  ``run_kernel`` (or None for an
    idle GPU) is launched on the current stream right after the probe is
    queued on a second stream (default priority), so the interval overlaps
    that kernel.  Returns None if the probe library is missing."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "bwd_rope_apply_amd", "libra_clock.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.ra_clock_probe.argtypes = [ctypes.c_void_p, ctypes.c_ulonglong, ctypes.c_void_p]
    lib.ra_clock_probe.restype = ctypes.c_int
    khz = int(lib.ra_wall_clock_khz())
    if khz <= 0:
        return None
    out = torch.zeros(2, dtype=torch.int64, device="cuda")
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    ticks = int(wall_ms * khz)
    if lib.ra_clock_probe(out.data_ptr(), ticks, side.cuda_stream) != 0:
        return None
    if run_kernel is not None:
        run_kernel()
    torch.cuda.synchronize()
    cycles, wall = (int(x) for x in out.cpu().tolist())
    if wall <= 0:
        return None
    return cycles / (wall / (khz * 1e3)) / 1e9


def cpu_baseline(inp, wl):
    """The float64 oracle on one head of the same inputs (a bounded sample),
    timed on the host cores, scaled to TFLOP/s with the same flop count."""
    import numpy as np
    from oracle import ref
    threads, blas = host_blas()
    full = {n: inp.f64(n).reshape(-1, 1, wl.N, wl.D) for n in ("q", "k", "v", "do")}

    def run(heads):
        q, k, v, do = (full[n][:heads].reshape(1, heads, wl.N, wl.D) for n in ("q", "k", "v", "do"))
        t0 = time.perf_counter()
        o, lse = ref.ref_fwd(q, k, v, wl.base, inp.alpha, wl.causal)
        ref.ref_bwd(q, k, v, o, do, lse, wl.base, inp.alpha, wl.causal)
        return time.perf_counter() - t0

    # size the sample to about 10 s of oracle work (at least one head)
    t1 = run(1)
    heads = int(min(wl.B * wl.H, max(1, round(10.0 / max(t1, 1e-3)))))
    dt = run(heads) if heads > 1 else t1
    flops = 6.0 * heads * wl.N * wl.N * wl.D
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{heads} of {wl.B * wl.H} heads (N={wl.N}, D={wl.D}), float64 fwd+bwd incl. "
                      f"dalpha, {dt:.1f} s", "blas": blas,
            "host_cpus": len(os.sched_getaffinity(0))}


def visible_pairs(lists, N: int, causal: bool) -> int:
    """(query, key) pairs that block lists leave visible: per query block
    its own block (the causal triangle under the mask) and each distinct
    listed block in range (earlier blocks only under the mask)."""
    nb = (N + 127) // 128
    size = [min(128, N - 128 * b) for b in range(nb)]
    total = 0
    for per_b in lists:
        for per_h in per_b:
            for qb, sel in enumerate(per_h):
                seen = {qb} | {kb for kb in sel if 0 <= kb < nb and (not causal or kb <= qb)}
                for kb in seen:
                    if causal and kb == qb:
                        total += size[qb] * (size[qb] + 1) // 2
                    else:
                        total += size[qb] * size[kb]
    return total


def gram_cpu_baseline(x, tau, d):
    """The float64 oracle's selection on the first tokens of the sequence (a
    bounded sample of the same workload), timed on the host cores."""
    import numpy as np
    from oracle import gram
    threads, blas = host_blas()
    Ts = min(x.shape[0], 2048)
    xs = np.ascontiguousarray(x[:Ts])
    t0 = time.perf_counter()
    gram.select(xs, tau)
    dt = time.perf_counter() - t0
    return {"value": d * Ts * (Ts - 1) / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "sample": f"first {Ts} of {x.shape[0]} tokens (d={d}), float64 "
                                        f"selection, {dt:.2f} s", "blas": blas}


def bench_gram(args):
    """Gram-threshold selection ("Cascade token selection for transformer
    attention acceleration"): one step = the full selection of one layer's
    tokens (causal T x T Gram product, d T (T - 1) flops); one cascade step
    on the next layer, inheriting that selection, is timed beside it."""
    import numpy as np
    import torch
    from bwd_rope_apply_amd import workloads as W
    from bwd_rope_apply_amd import _lib

    wl = W.get_tokens(args.gram_workload)
    x0s, x1s = (a[0] for a in W.make_tokens(wl, layers=2))
    dev = torch.device("cuda:0")

    def dev_t(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    x0, x1 = dev_t(x0s), dev_t(x1s)
    T, d = wl.T, wl.d
    lib = _lib.load()
    ws = torch.empty(int(lib.gram_select_workspace_bytes(1, T, d)), dtype=torch.uint8, device=dev)
    wsc = torch.empty(int(lib.gram_cascade_workspace_bytes(T, d)), dtype=torch.uint8, device=dev)
    m = torch.empty((1, T), dtype=torch.float32, device=dev)
    rep = torch.empty((1, T), dtype=torch.uint8, device=dev)
    cnt = torch.empty((1,), dtype=torch.int32, device=dev)
    mc, repc = torch.empty((T,), dtype=torch.float32, device=dev), torch.empty((T,), dtype=torch.uint8, device=dev)
    cntc = torch.empty((1,), dtype=torch.int32, device=dev)
    stages = [("prep", _lib.GRAM_STAGE_PREP), ("gram", _lib.GRAM_STAGE_GRAM), ("decide", _lib.GRAM_STAGE_DECIDE)]
    prev = rep[0]

    def step(ev=None):
        for i, (_, bit) in enumerate(stages):
            if ev is not None:
                ev[i].record()
            _lib.gram_select(x0, wl.tau, workspace=ws, out=(m, rep, cnt), stages=bit)
        if ev is not None:
            ev[3].record()
        _lib.gram_cascade(x1, wl.tau, prev, workspace=wsc, out=(mc, repc, cntc))
        if ev is not None:
            ev[4].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    sel = np.array([e[0].elapsed_time(e[3]) for e in evs])
    gram_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    casc = np.array([e[3].elapsed_time(e[4]) for e in evs])
    flops = float(d) * T * (T - 1)
    ms = float(np.median(sel))
    r_prev, r_new = int(rep.sum().item()), int(repc.sum().item())
    kept = int((repc.bool() & rep[0].bool()).sum().item())
    line = {
        "metric": f"Gram-threshold selection TFLOP/s (causal T x T Gram of normalised tokens), T={T} d={d}",
        "value": round(flops / (ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "fp16",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": 1, "T": T, "d": d, "tau": wl.tau, "storage": wl.dtype,
                   "flops_per_step": flops, "wall_ms_per_step_incl_cascade": round(wall * 1e3 / args.steps, 4)},
        "roofline": {"bound": "mfma", "kernel": "gram_max_kernel", "achieved": round(flops / (gram_ms * 1e-3) / 1e12, 2),
                     "peak": PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(flops / (gram_ms * 1e-3) / 1e12 / PEAK_TFLOPS, 4), "traffic": None,
                     "avg_ms": round(gram_ms, 4)},
        "stages_ms": {n: round(float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])), 4)
                      for i, (n, _) in enumerate(stages)},
        "cascade": {"ms_median": round(float(np.median(casc)), 4), "inherited": r_prev, "kept": kept,
                    "added": r_new - kept, "selected": r_new,
                    "gram_ops_vs_full": round((r_prev * r_prev + (T - r_prev) * r_prev) / float(T * T), 4),
                    "speedup_vs_full_selection": round(ms / float(np.median(casc)), 3)},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = gram_cpu_baseline(W.storage_to_f64(x0s), wl.tau, d)
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(heads are independent, a multi-GPU run would shard them and all-reduce dalpha)",
              file=sys.stderr)
        sys.exit(2)
    if args.gram:
        bench_gram(args)
        return

    import numpy as np
    import torch
    from bwd_rope_apply_amd import workloads as W
    from bwd_rope_apply_amd import _lib

    wl = W.get(args.workload)
    inp = W.make_inputs(wl)
    dev = torch.device("cuda:0")

    def dev_t(x):
        if x.dtype == np.uint16:
            return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(x).to(dev)

    q, k, v, do = (dev_t(getattr(inp, n)) for n in ("q", "k", "v", "do"))
    alpha = dev_t(inp.alpha)
    B, H, N, D = wl.B, wl.H, wl.N, wl.D
    f32 = dict(dtype=torch.float32, device=dev)
    o, lse = torch.empty((B, H, N, D), **f32), torch.empty((B, H, N), **f32)
    dq, dk, dv = (torch.empty((B, H, N, D), **f32) for _ in range(3))
    da = torch.empty((D // 2,), **f32)
    dt_code = _lib.BF16 if wl.dtype == "bf16" else _lib.FP32
    # one buffer for both passes (the forward's regions are a prefix of the backward's)
    ws_kind = "bwd_min" if args.min_workspace else "bwd"
    ws_b = torch.empty(_lib.workspace_bytes(ws_kind, B, H, N, D, dt_code, wl.causal), dtype=torch.uint8,
                       device=dev)
    ws_f = ws_b

    fwd_stages, bwd_stages = stage_lists(wl.dtype)
    names = [n for n, _ in fwd_stages] + [n for n, _ in bwd_stages]
    opts = None
    if args.unrotated_pairs or args.scale or args.pos_offset:
        opts = dict(unrotated_pairs=args.unrotated_pairs, scale=args.scale,
                    pos_offset=args.pos_offset)
    opts_config = dict(opts) if opts else None
    # algorithmic flops: 12 D per visible (query, key) pair (forward QK^T and
    # PV, backward dQ, dV, dP, dK); dense causal attention counts N^2 / 2
    # pairs per head
    pairs = B * H * N * N / 2.0
    if args.retrieved >= 0:
        lists = W.block_lists(B, H, N, args.retrieved, wl.causal, wl.seed)
        opts = dict(opts or {}, blocks=_lib.block_csr(lists, dev))
        pairs = float(visible_pairs(lists, N, wl.causal))
        opts_config = dict(opts_config or {}, block_lists={
            "retrieved": args.retrieved, "block": 128,
            "density_vs_causal": round(pairs / (B * H * N * (N + 1) / 2.0), 4)})
    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step(fwd_calls, bwd_calls, events=None, dom_events=None):
        """One fwd + bwd step.  events: one before each call and one at the
        end (the breakdown pass); dom_events: one before and one after the
        dominant call only (the timed steps: each event record costs the GPU
        a few microseconds, so the timed steps carry just these two)."""
        i = 0
        for name, bit in fwd_calls:
            if events is not None:
                events[i].record()
            _lib.fwd(q, k, v, wl.base, alpha, wl.causal, workspace=ws_f, out=(o, lse), stages=bit,
                     opts=opts)
            i += 1
        for name, bit in bwd_calls:
            if events is not None:
                events[i].record()
            if dom_events is not None and name == DOMINANT[0]:
                dom_events[0].record()
            _lib.bwd(q, k, v, o, do, lse, wl.base, alpha, wl.causal, workspace=ws_b,
                     out=(dq, dk, dv, da), stages=bit, opts=opts)
            if dom_events is not None and name == DOMINANT[0]:
                dom_events[1].record()
            i += 1
        if events is not None:
            events[i].record()

    calls = [n for n, _ in FWD_CALLS] + [n for n, _ in BWD_CALLS]
    for _ in range(args.warmup):
        step(FWD_CALLS, BWD_CALLS)
    torch.cuda.synchronize()
    ev_dom = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(FWD_CALLS, BWD_CALLS, dom_events=ev_dom[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if not (torch.isfinite(o).all() and torch.isfinite(dq).all() and torch.isfinite(dk).all()
            and torch.isfinite(dv).all() and torch.isfinite(da).all()):
        print("bench.py: non-finite outputs", file=sys.stderr)
        sys.exit(1)
    # the dominant call's average over the timed steps (the roofline's duration)
    dom_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev_dom]))

    # breakdown pass after the timed steps: the same steps with an event
    # before every call (per-call times, fwd / bwd medians)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)]
          for _ in range(args.steps)]
    for s in range(args.steps):
        step(FWD_CALLS, BWD_CALLS, ev[s])
    torch.cuda.synchronize()
    call_ms = {n: float(np.mean([ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(args.steps)]))
               for i, n in enumerate(calls)}
    nf = len(FWD_CALLS)
    step_ev = np.array([ev[s][0].elapsed_time(ev[s][len(calls)]) for s in range(args.steps)])
    fwd_ev = np.array([ev[s][0].elapsed_time(ev[s][nf]) for s in range(args.steps)])
    bwd_ev = np.array([ev[s][nf].elapsed_time(ev[s][len(calls)]) for s in range(args.steps)])
    # per-kernel breakdown: every kernel in its own call (no overlap), after the timed steps
    nd = min(args.steps, 5)
    evd = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(nd)]
    for s in range(nd):
        step(fwd_stages, bwd_stages, evd[s])
    torch.cuda.synchronize()
    stage_ms = {n: float(np.mean([evd[s][i].elapsed_time(evd[s][i + 1]) for s in range(nd)]))
                for i, n in enumerate(names)}
    ms_step = wall * 1e3 / args.steps
    # shader clock of a CU while the dominant kernel runs, and idle
    clocks = None
    if wl.dtype == "bf16":
        dom_bit = dict(BWD_CALLS)[DOMINANT[0]]
        run_dom = lambda: _lib.bwd(q, k, v, o, do, lse, wl.base, alpha, wl.causal, workspace=ws_b,
                                   out=(dq, dk, dv, da), stages=dom_bit, opts=opts)
        under = [clock_sample(run_dom) for _ in range(3)]
        idle = clock_sample(None)
        if all(c is not None for c in under) and idle is not None:
            clocks = {"sclk_ghz_under_" + DOMINANT[1]: round(float(np.median(under)), 3),
                      "sclk_ghz_idle": round(idle, 3)}
    unit = 2.0 * pairs * D
    flops = 6.0 * unit
    value = flops / (ms_step * 1e-3) / 1e12

    dom, kernel, dom_units = DOMINANT
    if wl.dtype == "bf16":
        achieved = dom_units * unit / (dom_ms * 1e-3) / 1e12
        traffic = measured_traffic(args.traffic, dom, wl.name) if args.retrieved < 0 else None
        roofline = {"bound": "mfma", "kernel": kernel, "achieved": round(achieved, 2),
                    "peak": PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS, 4),
                    "traffic": traffic, "avg_ms": round(dom_ms, 4)}
        if clocks:
            # the same peak at the clock the kernel actually ran at
            ghz = clocks["sclk_ghz_under_" + kernel]
            roofline["observed_sclk_ghz"] = ghz
            roofline["peak_at_observed_sclk"] = round(PEAK_TFLOPS * ghz / 2.4, 1)
            roofline["frac_at_observed_sclk"] = round(achieved / (PEAK_TFLOPS * ghz / 2.4), 4)
        dq_pass = ("recompute" if args.min_workspace or args.retrieved >= 0
                   or _lib.workspace_bytes("bwd", B, H, N, D, dt_code, wl.causal)
                   == _lib.workspace_bytes("bwd_min", B, H, N, D, dt_code, wl.causal) else "ds_panels")
    else:
        # fp32 inputs: the float32 path runs the whole step on the fp32 matrix cores
        roofline = {"bound": "mfma", "kernel": "f32 path (whole step, v_mfma_f32_32x32x2f32)",
                    "achieved": round(value, 4), "peak": FP32_MFMA_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(value / FP32_MFMA_TFLOPS, 5), "traffic": None,
                    "avg_ms": round(ms_step, 4)}
        dq_pass = "fp32_exact"
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16" if wl.dtype == "bf16" else "fp32",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "H": H, "N": N, "D": D, "causal": wl.causal,
                   "base": wl.base, "storage": wl.dtype, "outputs": "fp32",
                   "options": opts_config,
                   "dq_pass": dq_pass,
                   "flops_per_step": flops, "pct_bf16_peak": round(100.0 * value / PEAK_TFLOPS, 2)},
        "roofline": roofline,
        "calls_ms": {n: round(t, 4) for n, t in call_ms.items()},
        "stages_ms_serial": {n: round(t, 4) for n, t in stage_ms.items()},
        "events_ms": {"step_median": round(float(np.median(step_ev)), 4),
                      "step_min": round(float(step_ev.min()), 4),
                      "fwd_median": round(float(np.median(fwd_ev)), 4),
                      "bwd_median": round(float(np.median(bwd_ev)), 4)},
        "tflops_fwd": round(2.0 * unit / (float(np.median(fwd_ev)) * 1e-3) / 1e12, 2),
        "tflops_bwd": round(4.0 * unit / (float(np.median(bwd_ev)) * 1e-3) / 1e12, 2),
        "tflops_fa_convention": round(7.0 * unit / (ms_step * 1e-3) / 1e12, 2),
        "device": dict(device_info(), **(clocks or {})),
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(inp, wl)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
