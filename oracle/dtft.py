"""Frequency gradient from the surrogate of LeRoPE, "Theoretical analysis".

TEST INFRASTRUCTURE ONLY (see ``oracle.ref``).

The page states that the gradient for the frequency of band m is the
derivative of a surrogate P_m(theta): the real part of the discrete-time
Fourier transform of the offset-aggregated gradient signal.  Written out:
with z = x_2m + i x_2m+1 for the un-rotated query and key pairs, a score is
S_ij = (1/sqrt D) sum_m Re(z_q,i conj(z_k,j) e^{i (i-j) theta_hat_m}), so with
the score gradient dS frozen,

    G_m(Delta) = sum_{b,h} sum_{i-j=Delta} (1/sqrt D) dS_ij z_q,i conj(z_k,j)
    P_m(theta) = Re sum_Delta G_m(Delta) e^{i Delta theta}
    dL/dtheta_hat_m = P_m'(theta_hat_m)
    dalpha_m = theta_hat_m * P_m'(theta_hat_m)   (theta_hat = e^alpha theta)

Reading: the sign convention of the transform (e^{+i Delta theta}) follows
from the counter-clockwise rotation; the page gives no formula.
"""
from __future__ import annotations

import numpy as np

from . import ref


def offset_signal(q, k, dS) -> np.ndarray:
    """G[m, Delta + N - 1] for Delta = -(N-1)..N-1, summed over b, h."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, H, N, D = q.shape
    zq = q[..., 0::2] + 1j * q[..., 1::2]          # [B,H,N,D/2]
    zk = k[..., 0::2] + 1j * k[..., 1::2]
    scale = 1.0 / np.sqrt(D)
    G = np.zeros((D // 2, 2 * N - 1), dtype=np.complex128)
    for b in range(B):
        for h in range(H):
            for m in range(D // 2):
                M = scale * dS[b, h] * np.outer(zq[b, h, :, m], np.conj(zk[b, h, :, m]))
                for delta in range(-(N - 1), N):
                    # entries with i - j = delta lie on diagonal offset j - i = -delta
                    G[m, delta + N - 1] += np.trace(M, offset=-delta)
    return G


def surrogate(G: np.ndarray, theta: np.ndarray) -> np.ndarray:
    """P_m(theta_m) = Re sum_Delta G_m(Delta) e^{i Delta theta_m}."""
    N = (G.shape[1] + 1) // 2
    delta = np.arange(-(N - 1), N, dtype=np.float64)
    return np.real((G * np.exp(1j * delta[None, :] * np.asarray(theta)[:, None])).sum(axis=1))


def surrogate_slope(G: np.ndarray, theta: np.ndarray) -> np.ndarray:
    """P_m'(theta_m) = Re sum_Delta i Delta G_m(Delta) e^{i Delta theta_m}."""
    N = (G.shape[1] + 1) // 2
    delta = np.arange(-(N - 1), N, dtype=np.float64)
    e = np.exp(1j * delta[None, :] * np.asarray(theta)[:, None])
    return np.real((1j * delta[None, :] * G * e).sum(axis=1))


def dalpha_dtft(q, k, v, do, base, alpha=None, causal=True, p0=0.0) -> np.ndarray:
    """dalpha through the surrogate; tiny inputs only (full score matrices)."""
    d = ref.ref_dense(q, k, v, do, base, alpha, causal, p0)
    th = d["theta_hat"]
    G = offset_signal(q, k, d["dS"])
    return th * surrogate_slope(G, th)
