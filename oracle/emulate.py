"""Rounding-point emulation of the bf16 path's numerical design, in float64.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
baseline leg of the benchmark may import this module.  It shares no code with
the HIP path and imports nothing from it; it re-uses the oracle's own
rotation and frequency definitions (``oracle.ref``).

It answers one question before and beside the kernels: with operands rounded
where the design rounds them, how far from the exact result can a correct
implementation of that design land?  It computes the same function as
``oracle.ref`` (exact causal softmax attention with RoPE and learnable
log-frequencies, forward and backward; "RoPE attention can be trained in
almost-linear time", Methodology 1 and 2; LeRoPE, Central mechanism and Key
design choices), with every other step in float64, and rounds the values at
these points only:

  q~      rotated query times log2(e) * scale, once per row (the forward's
          and the backward's operand)
  k~      rotated key, once per row
  v, dO   the value rows; the upstream gradient after its per-head
          power-of-two scale s = 2^(2 - floor(log2 max|dO|))
  P       the softmax weights that multiply V (forward) and dO (dV)
  dS      P o (dP - D_i), the operand of dQ~ and dK~

``rnd`` is the rounding applied at those points: ``fp16`` (the design),
``bf16`` (the alternative the design rejects) or ``exact`` (none: then the
result equals ``oracle.ref`` up to float64 summation order, which is pinned
by a test).  Query rows below ``corner`` use split operands at every point
(x = hi + lo with hi = rnd(x), lo = rnd(x - hi)), and so do the keys those
rows see, as the design's exact corner does.

The forward's weights are taken relative to a running reference that lags
each row's maximum by a spread offset of up to LAZY_SLACK (log2 units), so
that the largest weight is a generic value with its own rounding error, as
under the design's lazily moved reference (relative to the exact maximum it
would be exactly 1, which hides that error).  ``norm_rounded``: O's
normaliser is the sum of the rounded weights the numerator uses (the
design), else the unrounded sum; ``lse_rounded``: the LSE takes the same
rounded sum (the design), else the unrounded one.  D_i is formed from the
emulated O (float32 in the design).

Errors are reported under two readings of "max abs error <= 2e-2 on outputs
normalised by their RMS":
  A (graded)   per tensor: max |x - ref| / rms(ref)
  B            per row: max |x_row - ref_row| / max(rms(ref_row), 1e-3 rms(ref)),
               the largest over rows
"""
from __future__ import annotations

import numpy as np

from . import ref as R

LOG2E = 1.4426950408889634
LN2 = 0.6931471805599453


# ------------------------------------------------------------------ rounding
def fp16(x):
    """Round to IEEE binary16, nearest-even (overflow to +-inf, subnormals
    as the format has them)."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def bf16(x):
    """Round to bfloat16, nearest-even, through float32 (as a float32 value
    is rounded to bfloat16: add 0x7fff plus the kept LSB, truncate)."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def exact(x):
    return np.asarray(x, dtype=np.float64)


ROUNDINGS = {"fp16": fp16, "bf16": bf16, "exact": exact}


def split(x, rnd):
    """hi + lo with hi = rnd(x), lo = rnd(x - hi): about twice the bits."""
    hi = rnd(x)
    return hi + rnd(x - hi)


def dO_scale(do_head):
    """The head's power-of-two dO scale: its largest |entry| lands in [4, 8)."""
    mx = float(np.max(np.abs(do_head))) if do_head.size else 0.0
    if not (mx > 0.0) or not np.isfinite(mx):
        return 1.0
    e = int(np.floor(np.log2(mx)))
    return float(2.0 ** min(126, max(-126, 2 - e)))


# ------------------------------------------------------------------ one head
def _rows_rounded(x, r0, corner, rnd):
    """rnd(x) for rows >= corner and split(x) for rows < corner; x holds the
    rows r0, r0 + 1, ... of a head."""
    out = rnd(x)
    n = max(0, min(x.shape[0], corner - r0))
    if n:
        out[:n] = split(x[:n], rnd)
    return out


def _operands(q, k, v, do, th, scale, rnd, corner, p0):
    N, D = q.shape
    phi = R.angles(N, th, p0)
    qt, kt = R.rotate(q, phi), R.rotate(k, phi)
    c = LOG2E * scale
    qh = _rows_rounded(qt * c, 0, corner, rnd)   # log2-unit query operand
    # keys: rounded for the rows past the corner, split for the corner's rows
    kh = {False: rnd(kt), True: _rows_rounded(kt, 0, corner, rnd)}
    s = dO_scale(do) if do is not None else 1.0
    vh = rnd(v)
    doh = rnd(do * s) if do is not None else None
    return phi, qt, kt, qh, kh, vh, doh, s


def _segments(N, block, corner):
    """Query-row ranges [r0, r1) of at most ``block`` rows that do not
    straddle the corner."""
    cuts = sorted(set(list(range(0, N, block)) + ([corner] if 0 < corner < N else []) + [N]))
    return list(zip(cuts[:-1], cuts[1:]))


def _mask(S, r0, causal):
    if causal:
        i = np.arange(r0, r0 + S.shape[0])[:, None]
        j = np.arange(S.shape[1])[None, :]
        S = np.where(j <= i, S, -np.inf)
    return S


LAZY_SLACK = 8.0


def _lazy_offset(r0, r1):
    """A fixed, spread offset in [0, LAZY_SLACK) per row (golden-ratio
    sequence), standing for how far a running reference lags the maximum."""
    i = np.arange(r0, r1, dtype=np.float64)
    return LAZY_SLACK * np.mod(i * 0.6180339887498949, 1.0)


def emulate_head(q, k, v, do, th, causal=True, rnd=fp16, corner=0, scale=None, p0=0.0, block=512,
                 store=True, norm_rounded=True, lse_rounded=True):
    """One head ([N, D] float64 arrays): O, LSE (natural log), dQ, dK, dV
    (un-rotated frame) with the design's rounding points.  ``do`` None skips
    the backward.  ``store``: O and LSE are float32 outputs (the backward
    reads them back), else kept in float64."""
    N, D = q.shape
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    phi, qt, kt, qh, kh, vh, doh, s = _operands(q, k, v, do, th, scale, rnd, corner, p0)

    def S2(r0, r1, ke):   # scores in log2 units, masked
        return _mask(qh[r0:r1] @ kh[r0 < corner][:ke].T, r0, causal)

    o = np.empty((N, D))
    lse2 = np.empty(N)
    for r0, r1 in _segments(N, block, corner):
        ke = r1 if causal else N
        S = S2(r0, r1, ke)
        # the running reference: below the row maximum by up to LAZY_SLACK
        # (log2 units), so the largest weight is a generic value, not 1
        m = S.max(axis=1, keepdims=True) - _lazy_offset(r0, r1)[:, None]
        P = np.exp2(S - m)
        Pr = _rows_rounded(P, r0, corner, rnd)
        lsum = P.sum(axis=1)                 # unrounded weights
        lr = Pr.sum(axis=1)                  # the weights PV uses
        o[r0:r1] = (Pr @ vh[:ke]) / (lr if norm_rounded else lsum)[:, None]
        lse2[r0:r1] = m[:, 0] + np.log2(lr if lse_rounded else lsum)
    lse = lse2 * LN2
    if store:   # the stored outputs
        o = o.astype(np.float32).astype(np.float64)
        lse = lse.astype(np.float32).astype(np.float64)
    if do is None:
        return o, lse, None, None, None

    Drow = (doh * o).sum(axis=1)                     # from the scaled dO
    l2 = lse * LOG2E
    dqt = np.zeros((N, D))
    dkt = np.zeros((N, D))
    dv = np.zeros((N, D))
    for r0, r1 in _segments(N, block, corner):
        ke = r1 if causal else N
        P = np.exp2(S2(r0, r1, ke) - l2[r0:r1, None])
        dP = doh[r0:r1] @ vh[:ke].T
        dS = P * (dP - Drow[r0:r1, None])
        Pr = _rows_rounded(P, r0, corner, rnd)
        dSr = _rows_rounded(dS, r0, corner, rnd)
        dv[:ke] += Pr.T @ doh[r0:r1]
        dqt[r0:r1] = scale * (dSr @ kh[r0 < corner][:ke])
        dkt[:ke] += LN2 * (dSr.T @ qh[r0:r1])
    dq = R.unrotate(dqt / s, phi)
    dk = R.unrotate(dkt / s, phi)
    return o, lse, dq, dk, dv / s


def emulate(q, k, v, do, base, alpha=None, causal=True, rnd=fp16, corner=0, scale=None,
            p0=0.0, rot=None, block=512, store=True, norm_rounded=True, lse_rounded=True):
    """All heads of [B, H, N, D] inputs: dict O, LSE, dQ, dK, dV, dalpha."""
    q, k, v = R._f64(q), R._f64(k), R._f64(v)
    do = None if do is None else R._f64(do)
    B, H, N, D = q.shape
    th = R.theta_hat(base, alpha, D, rot)
    out = {n: np.empty((B, H, N, D)) for n in ("O", "dQ", "dK", "dV")}
    out["LSE"] = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):
            o, lse, dq, dk, dv = emulate_head(q[b, h], k[b, h], v[b, h],
                                              None if do is None else do[b, h], th, causal, rnd,
                                              corner, scale, p0, block, store, norm_rounded,
                                              lse_rounded)
            out["O"][b, h], out["LSE"][b, h] = o, lse
            if do is not None:
                out["dQ"][b, h], out["dK"][b, h], out["dV"][b, h] = dq, dk, dv
    out["dalpha"] = (R.dalpha_chain(q, k, out["dQ"], out["dK"], th, p0)
                     if do is not None else None)
    return out


# ------------------------------------------------------------------ readings
def reading_a(got, ref):
    """max |got - ref| / rms(ref) over the whole tensor."""
    rms = float(np.sqrt(np.mean(np.square(ref))))
    return float(np.max(np.abs(got - ref))) / max(rms, 1e-300)


def reading_b(got, ref):
    """The largest per-row max |got - ref| / max(rms(ref_row), 1e-3 rms(ref));
    rows run along the last axis."""
    rms = float(np.sqrt(np.mean(np.square(ref))))
    g = np.asarray(got).reshape(-1, got.shape[-1])
    r = np.asarray(ref).reshape(-1, ref.shape[-1])
    row_rms = np.sqrt(np.mean(np.square(r), axis=1))
    den = np.maximum(row_rms, 1e-3 * rms)
    return float(np.max(np.max(np.abs(g - r), axis=1) / np.maximum(den, 1e-300)))


def floors(got, ref, names=("O", "dQ", "dK", "dV")):
    """{name: (reading A, reading B)}, plus dalpha under reading A."""
    res = {n: (reading_a(got[n], ref[n]), reading_b(got[n], ref[n])) for n in names}
    if got.get("dalpha") is not None and ref.get("dalpha") is not None:
        res["dalpha"] = (reading_a(got["dalpha"], ref["dalpha"]), float("nan"))
    return res
