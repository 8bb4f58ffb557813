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
    """max |got - ref| / rms(ref)  (bf16 inputs: the bar is 2e-2)."""
    rms = float(np.sqrt(np.mean(np.square(ref))))
    return float(np.max(np.abs(got - ref))) / max(rms, 1e-30)


def err_rel(got, ref) -> float:
    """max |got - ref| / max |ref|  (fp32 inputs: the bar is 1e-4)."""
    return float(np.max(np.abs(got - ref))) / max(float(np.max(np.abs(ref))), 1e-30)


def report(got, ref, names=("O", "dQ", "dK", "dV", "dalpha")):
    return {n: (err_rms(got[n], ref[n]), err_rel(got[n], ref[n])) for n in names
            if got.get(n) is not None}
