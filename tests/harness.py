"""Shared helpers of the GPU tests: move seeded inputs to the device, run the
HIP path through the C ABI binding, compare with the float64 oracle."""
from __future__ import annotations

import numpy as np

from bwd_rope_apply_amd import workloads as W


def to_device(x: np.ndarray, device="cuda"):
    import torch
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def device_opts(opts, device="cuda"):
    """The binding's options from the tests' dict: ``block_lists`` (nested
    lists [b][h][query block] of key blocks) become CSR device tensors."""
    if not opts or "block_lists" not in opts:
        return opts
    from bwd_rope_apply_amd import _lib
    d = dict(opts)
    d["blocks"] = _lib.block_csr(d.pop("block_lists"), device)
    return d


def run_gpu(inp: W.Inputs, causal=None, alpha=True, want_dalpha=True, opts=None, ws="bwd"):
    """Forward and backward on the GPU; returns float64 numpy arrays.  opts:
    a dict of options (unrotated_pairs, scale, pos_offset, block_lists).
    ws: the backward workspace size query, "bwd" (with the dS panels where
    they apply) or "bwd_min" (dQ recomputes the scores)."""
    import torch
    from bwd_rope_apply_amd import fwd, bwd, _lib
    wl = inp.wl
    causal = wl.causal if causal is None else causal
    q, k, v, do = (to_device(getattr(inp, n)) for n in ("q", "k", "v", "do"))
    a = to_device(inp.alpha) if alpha else None
    opts = device_opts(opts)
    o, lse = fwd(q, k, v, wl.base, a, causal, opts=opts)
    B, H, N, D = q.shape
    dt = _lib.BF16 if wl.dtype == "bf16" else _lib.FP32
    work = torch.empty(max(1, _lib.workspace_bytes(ws, B, H, N, D, dt, causal)), dtype=torch.uint8,
                       device="cuda")
    dq, dk, dv, da = bwd(q, k, v, o, do, lse, wl.base, a, causal, workspace=work,
                         want_dalpha=want_dalpha, opts=opts)
    torch.cuda.synchronize()
    out = dict(O=o, LSE=lse, dQ=dq, dK=dk, dV=dv, dalpha=da)
    return {n: (None if t is None else t.double().cpu().numpy()) for n, t in out.items()}


def oracle_kwargs(D: int, opts=None) -> dict:
    """The oracle's arguments for the library's frequency-schedule options."""
    opts = opts or {}
    kw = dict(p0=float(opts.get("pos_offset", 0)))
    if opts.get("unrotated_pairs"):
        kw["rot"] = D // 2 - opts["unrotated_pairs"]
    if opts.get("scale"):
        kw["scale"] = float(np.float32(opts["scale"]))
    if opts.get("block_lists") is not None:
        kw["blocks"] = opts["block_lists"]
    return kw


def run_oracle(inp: W.Inputs, causal=None, alpha=True, opts=None):
    from oracle import ref
    wl = inp.wl
    causal = wl.causal if causal is None else causal
    q, k, v, do = (inp.f64(n) for n in ("q", "k", "v", "do"))
    a = inp.alpha if alpha else None
    kw = oracle_kwargs(wl.D, opts)
    o, lse = ref.ref_fwd(q, k, v, wl.base, a, causal, **kw)
    dq, dk, dv, da = ref.ref_bwd(q, k, v, o, do, lse, wl.base, a, causal, **kw)
    return dict(O=o, LSE=lse, dQ=dq, dK=dk, dV=dv, dalpha=da)


def err_rms(got, ref) -> float:
    """Reading A: max |got - ref| / rms(ref)  (bf16 inputs: the bar is 2e-2)."""
    rms = float(np.sqrt(np.mean(np.square(ref))))
    return float(np.max(np.abs(got - ref))) / max(rms, 1e-30)


def err_row(got, ref) -> float:
    """Reading B: the largest per-row max |got - ref| / max(rms(ref_row),
    1e-3 rms(ref)), rows along the last axis (reported beside reading A)."""
    g = np.asarray(got).reshape(-1, np.shape(got)[-1])
    r = np.asarray(ref).reshape(-1, np.shape(ref)[-1])
    rms = float(np.sqrt(np.mean(np.square(r))))
    den = np.maximum(np.sqrt(np.mean(np.square(r), axis=1)), max(1e-3 * rms, 1e-30))
    return float(np.max(np.max(np.abs(g - r), axis=1) / den))


def peak_ratio(ref) -> float:
    """max |ref| / rms(ref): how far reading A's normaliser is below the
    tensor's largest entries."""
    return float(np.max(np.abs(ref))) / max(float(np.sqrt(np.mean(np.square(ref)))), 1e-30)


def err_rel(got, ref) -> float:
    """max |got - ref| / max |ref|  (fp32 inputs: the bar is 1e-4)."""
    return float(np.max(np.abs(got - ref))) / max(float(np.max(np.abs(ref))), 1e-30)


def report(got, ref, names=("O", "dQ", "dK", "dV", "dalpha")):
    return {n: (err_rms(got[n], ref[n]), err_rel(got[n], ref[n])) for n in names
            if got.get(n) is not None}


def readings(got, ref, names=("O", "dQ", "dK", "dV")):
    """{name: (reading A, reading B, peak / rms of the reference)}."""
    return {n: (err_rms(got[n], ref[n]), err_row(got[n], ref[n]), peak_ratio(ref[n]))
            for n in names if got.get(n) is not None}


def oracle_workers() -> int:
    """Threads for running the oracle head by head (numpy releases the GIL in
    its array loops); at most 16, the CPU share of one GPU."""
    import os
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def compare_all_heads(inp: W.Inputs, got: dict, causal=None, workers=None):
    """Runs the oracle on every (b, h) of ``inp`` (one head per task, tasks
    in threads) and compares the GPU's outputs ``got`` with it element by
    element.  Returns {name: (reading A, reading B)} over all heads for O,
    dQ, dK, dV, the largest |LSE| difference, and dalpha's reading A against
    the oracle's dalpha (the sum of every head's part)."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    from oracle import ref
    wl = inp.wl
    causal = wl.causal if causal is None else causal
    q, k, v, do = (inp.f64(n) for n in ("q", "k", "v", "do"))
    th = ref.theta_hat(wl.base, inp.alpha, wl.D)
    names = ("O", "dQ", "dK", "dV")

    def one(bh):
        b, h = divmod(bh, wl.H)
        sl = (slice(b, b + 1), slice(h, h + 1))
        o, lse = ref.ref_fwd(q[sl], k[sl], v[sl], wl.base, inp.alpha, causal)
        dq, dk, dv, _ = ref.ref_bwd(q[sl], k[sl], v[sl], o, do[sl], lse, wl.base, inp.alpha, causal)
        r = dict(O=o[0, 0], dQ=dq[0, 0], dK=dk[0, 0], dV=dv[0, 0])
        st = {}
        for n in names:
            d = np.abs(got[n][b, h] - r[n])
            st[n] = (d.max(axis=1), np.sqrt(np.mean(np.square(r[n]), axis=1)),
                     float(np.sum(np.square(r[n]))))
        st["LSE"] = float(np.abs(got["LSE"][b, h] - lse[0, 0]).max())
        st["dalpha"] = ref.dalpha_chain(q[sl], k[sl], dq, dk, th)
        return st

    n_bh = wl.B * wl.H
    workers = workers or oracle_workers()
    # one BLAS thread per task whenever tasks run concurrently (a threaded
    # OpenBLAS called from several threads at once is not safe); a single
    # head gets every core through BLAS instead
    with threadpool_limits(workers if n_bh == 1 else 1):
        with ThreadPoolExecutor(min(workers, n_bh)) as ex:
            parts = list(ex.map(one, range(n_bh)))
    out = {}
    count = wl.N * wl.D * n_bh
    for n in names:
        rowmax = np.concatenate([p[n][0] for p in parts])
        rowrms = np.concatenate([p[n][1] for p in parts])
        rms = np.sqrt(sum(p[n][2] for p in parts) / count)
        a = float(rowmax.max()) / max(rms, 1e-30)
        b = float(np.max(rowmax / np.maximum(rowrms, max(1e-3 * rms, 1e-30))))
        out[n] = (a, b)
    out["LSE_abs"] = max(p["LSE"] for p in parts)
    want = np.sum([p["dalpha"] for p in parts], axis=0)
    out["dalpha"] = (err_rms(got["dalpha"], want), float("nan"))
    return out
