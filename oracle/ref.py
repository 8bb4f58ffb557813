"""Float64 CPU oracle for exact softmax attention with rotary position
embedding (RoPE) and learnable log-frequencies, forward and backward.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
baseline leg of the benchmark may import this module.  It shares no code with
the HIP path and imports nothing from it.

What it computes, written out from the definitions (no tiling, fusion or
reordering beyond a loop over query-row blocks, which leaves every sum's
terms unchanged):

  frequencies   theta_m = b^(-2m/D), m = 0..D/2-1, and the effective
                frequency theta_hat_m = exp(alpha_m) * theta_m
                (LeRoPE, "Central mechanism"; alpha = 0 gives standard RoPE,
                "Key design choices", initialisation).
  rotation      each (x_2m, x_2m+1) pair of a query or key row at position p
                is turned by the angle (p + p0) * theta_hat_m, counter-
                clockwise (LeRoPE, "Problem statement": queries and keys are
                rotated in two-dimensional frequency bands; values are not).
  forward       S = Q~ K~^T / sqrt(D), causal mask j <= i, normalised
                softmax s(x) per row, O = P V, and the row log-sum-exp
                ("RoPE attention can be trained in almost-linear time",
                Problem definition and Methodology 1, s(x)).
  backward      with the upstream gradient dO standing for the error term
                l(x) (output minus target), beta = dO V^T, and
                gamma = diag(s) beta - s s^T beta, i.e. dS = P o (dP - D) with
                D_i = sum_c dO_ic O_ic (same page, Methodology 1 and 2,
                gamma_1 and gamma_2); dQ~ = dS K~ / sqrt(D),
                dK~ = dS^T Q~ / sqrt(D), dV = P^T dO, then back to the
                un-rotated frame by the transpose rotation.
  d alpha       the gradient of the per-band log-frequency, summed over
                every batch entry and head because one alpha vector is shared
                by all heads and layers (LeRoPE, "Key design choices",
                parameter sharing).  Chain rule through the angle:
                d phi / d alpha_m = (p + p0) theta_hat_m and
                d x~ / d phi = J x~ with J the quarter turn, which gives
                dalpha_m = theta_hat_m * sum_p (p + p0) (x_2m g_2m+1 - x_2m+1 g_2m)
                over query rows (x = q, g = dQ) and key rows (x = k, g = dK),
                in either frame because J commutes with the rotation.
                ``oracle.dtft`` derives the same number from the surrogate
                of LeRoPE, "Theoretical analysis".

Readings where the pages are silent (each is a stated convention): theta_m =
b^(-2m/D); interleaved pairs (2m, 2m+1); counter-clockwise rotation; softmax
scale 1/sqrt(D); positions 0..N-1 for both queries and keys; causal keeps
j <= i; the scalar loss whose vector-Jacobian product is returned is
L = sum(O * dO).

Frequency-schedule variants (optional arguments, defaults = the above):
  rot     partial RoPE: only pairs m < rot are rotated and the slower bands
          m >= rot pass through (theta_hat_m = 0 there, so their alpha has
          no effect and a zero gradient); LeRoPE's p-RoPE baseline, which
          leaves the slowest 25% of bands unrotated ("Experimental setup",
          baselines), is rot = 0.75 * D/2.
  scale   the softmax scale on q.k (default 1/sqrt(D)); context-extension
          schemes that LeRoPE combines with (named under "Extrapolation")
          act through per-band alpha offsets and such a scale.
  p0      the position of the first row, shared by queries and keys.

Block-list attention (optional ``blocks``): exact attention restricted, for
each query block of BLOCK = 128 rows, to its own (diagonal) key block plus a
given set of other key blocks -- the exact part of Multipole Semantic
Attention ("Retrieval-augmented approximation": exact attention only for the
retrieved pairs and the local block diagonal).  ``blocks[b][h][qb]`` is an
iterable of key-block indices; out-of-range entries are ignored, and under
the causal mask blocks after the diagonal contribute nothing.  O and LSE are
over exactly the visible keys, so results over disjoint key sets merge
through their LSEs.

Inputs are numpy arrays [B, H, N, D] of any float type (upcast exactly to
float64); alpha is [D/2].
"""
from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------- frequencies
def thetas(base: float, D: int) -> np.ndarray:
    """Standard RoPE band rates theta_m = base^(-2m/D) (LeRoPE, Problem
    statement: a fixed geometric sequence set by the base b)."""
    m = np.arange(D // 2, dtype=np.float64)
    return np.float64(base) ** (-2.0 * m / D)


def theta_hat(base: float, alpha, D: int, rot=None) -> np.ndarray:
    """Effective frequency exp(alpha_m) * theta_m (LeRoPE, Central mechanism);
    zero for the unrotated bands m >= rot (partial RoPE)."""
    a = np.zeros(D // 2) if alpha is None else np.asarray(alpha, dtype=np.float64)
    th = np.exp(a) * thetas(base, D)
    if rot is not None:
        th = np.where(np.arange(D // 2) < rot, th, 0.0)
    return th


def angles(N: int, th: np.ndarray, p0: float = 0.0) -> np.ndarray:
    """phi[p, m] = (p + p0) * theta_hat_m for p = 0..N-1."""
    pos = np.arange(N, dtype=np.float64) + p0
    return pos[:, None] * th[None, :]


# ------------------------------------------------------------------ rotation
def rotate(x: np.ndarray, phi: np.ndarray) -> np.ndarray:
    """Turn every (x_2m, x_2m+1) pair of row p by +phi[p, m]."""
    c, s = np.cos(phi), np.sin(phi)
    xe, xo = x[..., 0::2], x[..., 1::2]
    out = np.empty(np.broadcast_shapes(x.shape), dtype=np.float64)
    out[..., 0::2] = xe * c - xo * s
    out[..., 1::2] = xe * s + xo * c
    return out


def unrotate(g: np.ndarray, phi: np.ndarray) -> np.ndarray:
    """Apply the transpose rotation R(phi)^T = R(-phi) (the chain rule of
    ``rotate`` for a gradient)."""
    return rotate(g, -phi)


def wedge(x: np.ndarray, g: np.ndarray) -> np.ndarray:
    """Per pair: x_2m g_2m+1 - x_2m+1 g_2m, i.e. <g, J x> with J the quarter
    turn [[0,-1],[1,0]] acting on the pair."""
    return x[..., 0::2] * g[..., 1::2] - x[..., 1::2] * g[..., 0::2]


# -------------------------------------------------------------- attention
BLOCK = 128


def block_visible(N: int, sel) -> np.ndarray:
    """[N, N] bool: key j visible to query i when block(j) is block(i) or in
    sel[block(i)] (no causal mask applied here)."""
    nb = (N + BLOCK - 1) // BLOCK
    vis = np.zeros((nb, nb), dtype=bool)
    for qb in range(nb):
        vis[qb, qb] = True
        for kb in (sel[qb] if qb < len(sel) else ()):
            if 0 <= kb < nb:
                vis[qb, kb] = True
    blk = np.arange(N) // BLOCK
    return vis[blk[:, None], blk[None, :]]


def _key_end(r1: int, N: int, causal: bool) -> int:
    """Keys j < key_end can be unmasked for query rows < r1."""
    return r1 if causal else N


def _scores(qt_blk, kt, scale, r0, causal, vis=None):
    """S = scale * Q~ K~^T for query rows r0.., masked to -inf where j > i
    (and, with a block-visibility matrix, where the key's block is not
    visible to the query's)."""
    S = scale * (qt_blk @ kt.T)
    if causal:
        i = np.arange(r0, r0 + qt_blk.shape[0])[:, None]
        j = np.arange(kt.shape[0])[None, :]
        S = np.where(j <= i, S, -np.inf)
    if vis is not None:
        S = np.where(vis[r0:r0 + qt_blk.shape[0], :kt.shape[0]], S, -np.inf)
    return S


def _logsumexp(S):
    m = S.max(axis=1, keepdims=True)
    return (m + np.log(np.exp(S - m).sum(axis=1, keepdims=True)))[:, 0]


def _softmax_grad(P, dP, Drow):
    """gamma = diag(s) beta - s s^T beta per row, i.e. P o (dP - D) with
    D_i = s_i^T beta_i (the gamma_2 scalar)."""
    return P * (dP - Drow[:, None])


def _scale(D, scale):
    return 1.0 / np.sqrt(D) if scale is None else float(scale)


def _head_fwd(q, k, v, th, causal, p0, block, scale=None, vis=None):
    N, D = q.shape
    scale = _scale(D, scale)
    phi = angles(N, th, p0)
    qt, kt = rotate(q, phi), rotate(k, phi)
    o = np.empty((N, D))
    lse = np.empty(N)
    for r0 in range(0, N, block):
        r1 = min(N, r0 + block)
        ke = _key_end(r1, N, causal)
        S = _scores(qt[r0:r1], kt[:ke], scale, r0, causal, vis)
        L = _logsumexp(S)
        P = np.exp(S - L[:, None])
        o[r0:r1] = P @ v[:ke]
        lse[r0:r1] = L
    return o, lse


def _head_bwd(q, k, v, o, do, lse, th, causal, p0, block, scale=None, vis=None):
    N, D = q.shape
    scale = _scale(D, scale)
    phi = angles(N, th, p0)
    qt, kt = rotate(q, phi), rotate(k, phi)
    Drow = (do * o).sum(axis=1)
    dqt = np.zeros((N, D))
    dkt = np.zeros((N, D))
    dv = np.zeros((N, D))
    for r0 in range(0, N, block):
        r1 = min(N, r0 + block)
        ke = _key_end(r1, N, causal)
        S = _scores(qt[r0:r1], kt[:ke], scale, r0, causal, vis)
        P = np.exp(S - lse[r0:r1, None])
        dv[:ke] += P.T @ do[r0:r1]
        dP = do[r0:r1] @ v[:ke].T
        dS = _softmax_grad(P, dP, Drow[r0:r1])
        dqt[r0:r1] = scale * (dS @ kt[:ke])
        dkt[:ke] += scale * (dS.T @ qt[r0:r1])
    dq, dk = unrotate(dqt, phi), unrotate(dkt, phi)
    return dq, dk, dv


def dalpha_chain(q, k, dq, dk, th, p0=0.0) -> np.ndarray:
    """dalpha_m = theta_hat_m * sum_{b,h} [sum_i (i+p0) wedge(q_i, dQ_i)_m
    + sum_j (j+p0) wedge(k_j, dK_j)_m], all in the un-rotated frame."""
    N = q.shape[-2]
    pos = np.arange(N, dtype=np.float64) + p0
    tq = (pos[:, None] * wedge(q, dq)).reshape(-1, N, th.size).sum(axis=(0, 1))
    tk = (pos[:, None] * wedge(k, dk)).reshape(-1, N, th.size).sum(axis=(0, 1))
    return th * (tq + tk)


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def _vis(blocks, b, h, N):
    return None if blocks is None else block_visible(N, blocks[b][h])


def ref_fwd(q, k, v, base, alpha=None, causal=True, p0=0.0, block=512, scale=None, rot=None,
            blocks=None):
    """Returns (O [B,H,N,D], LSE [B,H,N]), float64; LSE is the natural-log
    log-sum-exp of the scaled, masked scores of each row."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, N, D = q.shape
    th = theta_hat(base, alpha, D, rot)
    o = np.empty((B, H, N, D))
    lse = np.empty((B, H, N))
    for b in range(B):
        for h in range(H):  # heads are independent work units
            o[b, h], lse[b, h] = _head_fwd(q[b, h], k[b, h], v[b, h], th, causal, p0, block, scale,
                                           _vis(blocks, b, h, N))
    return o, lse


def ref_bwd(q, k, v, o, do, lse, base, alpha=None, causal=True, p0=0.0, block=512, scale=None,
            rot=None, blocks=None):
    """Returns (dQ, dK, dV [B,H,N,D] in the un-rotated frame, dalpha [D/2]):
    the vector-Jacobian product of (Q, K, V, alpha) -> O for the upstream
    gradient dO, given the forward's O and LSE."""
    q, k, v, o, do, lse = map(_f64, (q, k, v, o, do, lse))
    B, H, N, D = q.shape
    th = theta_hat(base, alpha, D, rot)
    dq = np.empty((B, H, N, D))
    dk = np.empty((B, H, N, D))
    dv = np.empty((B, H, N, D))
    for b in range(B):
        for h in range(H):
            dq[b, h], dk[b, h], dv[b, h] = _head_bwd(
                q[b, h], k[b, h], v[b, h], o[b, h], do[b, h], lse[b, h], th, causal, p0, block,
                scale, _vis(blocks, b, h, N))
    return dq, dk, dv, dalpha_chain(q, k, dq, dk, th, p0)


def ref_dense(q, k, v, do, base, alpha=None, causal=True, p0=0.0, scale=None, rot=None):
    """Every intermediate of one call as full matrices, for tiny inputs:
    dict with S, P, O, LSE, D, dP, dS, dQ, dK, dV, dalpha, qt, kt, theta_hat."""
    q, k, v, do = map(_f64, (q, k, v, do))
    B, H, N, D = q.shape
    th = theta_hat(base, alpha, D, rot)
    phi = angles(N, th, p0)
    qt, kt = rotate(q, phi), rotate(k, phi)
    scale = _scale(D, scale)
    S = scale * np.einsum("bhid,bhjd->bhij", qt, kt)
    if causal:
        S = np.where(np.tril(np.ones((N, N), dtype=bool)), S, -np.inf)
    m = S.max(axis=-1, keepdims=True)
    LSE = (m + np.log(np.exp(S - m).sum(axis=-1, keepdims=True)))[..., 0]
    P = np.exp(S - LSE[..., None])
    O = P @ v
    Drow = (do * O).sum(axis=-1)
    dP = do @ np.swapaxes(v, -1, -2)
    dS = P * (dP - Drow[..., None])
    dqt = scale * (dS @ kt)
    dkt = scale * (np.swapaxes(dS, -1, -2) @ qt)
    dq, dk = unrotate(dqt, phi), unrotate(dkt, phi)
    dv = np.swapaxes(P, -1, -2) @ do
    return dict(S=S, P=P, O=O, LSE=LSE, D=Drow, dP=dP, dS=dS, dQ=dq, dK=dk, dV=dv,
                dalpha=dalpha_chain(q, k, dq, dk, th, p0), qt=qt, kt=kt, theta_hat=th)


def ref_head_rows(q, k, v, do, base, alpha=None, causal=True, rows=(), cols=(),
                  p0=0.0, block=512, scale=None, rot=None):
    """One head ([N, D] arrays) at full length, outputs at sampled positions.

    Runs the forward of the whole head (O and LSE of every row are needed by
    the key-side gradients), then evaluates from the definitions:
    dQ at query rows ``rows`` and dK, dV at key rows ``cols``.
    Returns dict with O, LSE (all rows), dQ[rows], dK[cols], dV[cols]
    (un-rotated frame)."""
    q, k, v, do = map(_f64, (q, k, v, do))
    N, D = q.shape
    th = theta_hat(base, alpha, D, rot)
    o, lse = _head_fwd(q, k, v, th, causal, p0, block, scale)
    scale = _scale(D, scale)
    phi = angles(N, th, p0)
    qt, kt = rotate(q, phi), rotate(k, phi)
    Drow = (do * o).sum(axis=1)
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    dq = np.zeros((rows.size, D))
    for n_, i in enumerate(rows):
        ke = i + 1 if causal else N
        s = scale * (kt[:ke] @ qt[i])
        p = np.exp(s - lse[i])
        dp = v[:ke] @ do[i]
        ds = p * (dp - Drow[i])
        dq[n_] = unrotate(scale * (ds @ kt[:ke])[None, :], phi[i:i + 1])[0]
    dk = np.zeros((cols.size, D))
    dv = np.zeros((cols.size, D))
    for n_, j in enumerate(cols):
        r0 = j if causal else 0
        s = scale * (qt[r0:] @ kt[j])
        p = np.exp(s - lse[r0:])
        dv[n_] = p @ do[r0:]
        dp = do[r0:] @ v[j]
        ds = p * (dp - Drow[r0:])
        dk[n_] = unrotate(scale * (ds @ qt[r0:])[None, :], phi[j:j + 1])[0]
    return dict(O=o, LSE=lse, dQ=dq, dK=dk, dV=dv)
