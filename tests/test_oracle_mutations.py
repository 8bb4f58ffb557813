"""Planted mistakes in the oracle (on the CPU) must fail at least one pin.

Each mutant replaces one function of ``oracle.ref`` with a plausible wrong
version (a dropped term, a wrong sign or index, a transposed operand, an
off-by-one mask); the pins of ``test_oracle.py`` are then run against the
mutated oracle and at least one of them must fail.
"""
import numpy as np
import pytest

from oracle import ref
import test_oracle as pins

PIN_SET = [
    ("fd_causal", lambda: pins.test_finite_differences_all_gradients(5, 4, 10.0, True, None, None)),
    ("fd_full", lambda: pins.test_finite_differences_all_gradients(5, 8, 1e4, False, None, None)),
    ("textbook", pins.test_alpha_zero_is_textbook_complex_rope),
    ("alpha_base", pins.test_alpha_trades_against_base),
    ("offset", lambda: pins.test_relative_offset_invariance(True)),
    ("softmax", lambda: pins.test_softmax_rows(True)),
    ("balance", pins.test_rotational_balance),
    ("zero_q", pins.test_zero_queries),
    ("single", pins.test_single_position),
    ("row0", pins.test_causal_row_zero),
    ("sdpa", lambda: pins.test_zero_rotation_is_sdpa(True)),
    ("autograd", lambda: pins.test_autograd_through_complex_rotation(True)),
    ("dalpha3", lambda: pins.test_dalpha_three_derivations(True)),
    ("variants_autograd", lambda: pins.test_autograd_frequency_variants(0.3, 5, 7.0)),
    ("scale_is_query_scaling", pins.test_scale_is_query_scaling),
    ("fd_variant", lambda: pins.test_finite_differences_all_gradients(5, 8, 1e4, True, 0.21, 3)),
    ("blocks_dense", lambda: pins.test_block_list_all_blocks_is_dense(True)),
    ("blocks_brute", lambda: pins.test_block_list_brute_force(True)),
    ("blocks_merge", pins.test_block_list_lse_merge),
    ("blocks_fd", lambda: pins.test_block_list_finite_differences(True)),
]


def _mut_softmax_grad_drop_gamma2(P, dP, Drow):
    return P * dP


def _mut_rotate_clockwise(x, phi):
    c, s = np.cos(phi), np.sin(phi)
    out = np.empty(x.shape)
    out[..., 0::2] = x[..., 0::2] * c + x[..., 1::2] * s
    out[..., 1::2] = -x[..., 0::2] * s + x[..., 1::2] * c
    return out


def _mut_unrotate_wrong_way(g, phi):
    return ref.rotate(g, phi)


def _mut_thetas_exponent(base, D):
    m = np.arange(D // 2, dtype=np.float64)
    return np.float64(base) ** (-1.0 * m / D)


def _mut_dalpha_reversed_positions(q, k, dq, dk, th, p0=0.0):
    # positions counted from the end (a constant shift alone would be
    # harmless: by rotational balance it adds zero)
    return _orig_dalpha(q[..., ::-1, :], k[..., ::-1, :], dq[..., ::-1, :], dk[..., ::-1, :], th, p0)


def _mut_dalpha_theta_not_theta_hat(q, k, dq, dk, th, p0=0.0):
    return _orig_dalpha(q, k, dq, dk, np.ones_like(th), p0) * ref.thetas(1e4, 2 * th.size)


def _mut_dalpha_sign(q, k, dq, dk, th, p0=0.0):
    return -_orig_dalpha(q, k, dq, dk, th, p0)


def _mut_dalpha_keys_only(q, k, dq, dk, th, p0=0.0):
    return _orig_dalpha(q, k, np.zeros_like(dq), dk, th, p0)


def _mut_scores_strict_mask(qt_blk, kt, scale, r0, causal, vis=None):
    S = scale * (qt_blk @ kt.T)
    if causal:
        i = np.arange(r0, r0 + qt_blk.shape[0])[:, None]
        j = np.arange(kt.shape[0])[None, :]
        S = np.where(j < i, S, -np.inf)
    if vis is not None:
        S = np.where(vis[r0:r0 + qt_blk.shape[0], :kt.shape[0]], S, -np.inf)
    return S


def _mut_lse_drops_sum(S):
    return S.max(axis=1)


def _mut_theta_hat_ignores_rot(base, alpha, D, rot=None):
    return _orig_theta_hat(base, alpha, D)


def _mut_theta_hat_rot_off_by_one(base, alpha, D, rot=None):
    return _orig_theta_hat(base, alpha, D, None if rot is None else rot + 1)


def _mut_block_visible_64(N, sel):
    old = ref.BLOCK
    try:
        ref.BLOCK = 64
        return _orig_block_visible(N, sel)
    finally:
        ref.BLOCK = old


def _mut_block_visible_no_diagonal(N, sel):
    nb = (N + ref.BLOCK - 1) // ref.BLOCK
    vis = np.zeros((nb, nb), dtype=bool)
    for qb in range(nb):
        for kb in (sel[qb] if qb < len(sel) else ()):
            if 0 <= kb < nb:
                vis[qb, kb] = True
    blk = np.arange(N) // ref.BLOCK
    return vis[blk[:, None], blk[None, :]]


def _mut_head_bwd_ignores_blocks(q, k, v, o, do, lse, th, causal, p0, block, scale=None, vis=None):
    return _orig_head_bwd(q, k, v, o, do, lse, th, causal, p0, block, scale, None)


_orig_block_visible = ref.block_visible
_orig_theta_hat = ref.theta_hat
_orig_dalpha = ref.dalpha_chain
_orig_head_bwd = ref._head_bwd


def _mut_head_bwd(variant):
    """A copy of the per-head backward with one planted mistake."""
    def f(q, k, v, o, do, lse, th, causal, p0, block, scale=None, vis=None):
        N, D = q.shape
        scale = ref._scale(D, scale)
        if variant == "dk_default_scale":
            dk_scale = 1.0 / np.sqrt(D)
        else:
            dk_scale = scale
        phi = ref.angles(N, th, p0)
        qt, kt = ref.rotate(q, phi), ref.rotate(k, phi)
        Drow = (do * o).sum(axis=1)
        dqt, dkt, dv = np.zeros((N, D)), np.zeros((N, D)), np.zeros((N, D))
        for r0 in range(0, N, block):
            r1 = min(N, r0 + block)
            ke = r1 if causal else N
            S = ref._scores(qt[r0:r1], kt[:ke], scale, r0, causal, vis)
            P = np.exp(S - lse[r0:r1, None])
            if variant == "dv_transposed":
                dv[:ke] += P @ do[:ke] if P.shape[0] == P.shape[1] else P.T @ do[r0:r1]
            else:
                dv[:ke] += P.T @ do[r0:r1]
            dP = do[r0:r1] @ v[:ke].T
            dS = ref._softmax_grad(P, dP, Drow[r0:r1])
            dq_scale = 1.0 if variant == "dq_no_scale" else scale
            dqt[r0:r1] = dq_scale * (dS @ kt[:ke])
            if variant == "dk_transposed" and dS.shape[0] == dS.shape[1]:
                dkt[:ke] += scale * (dS @ qt[r0:r1])
            else:
                dkt[:ke] += dk_scale * (dS.T @ qt[r0:r1])
        if variant == "dk_rotated_frame":
            return ref.unrotate(dqt, phi), dkt, dv
        return ref.unrotate(dqt, phi), ref.unrotate(dkt, phi), dv
    return f


MUTANTS = {
    "softmax_grad_drops_gamma2": ("_softmax_grad", _mut_softmax_grad_drop_gamma2),
    "rotation_clockwise": ("rotate", _mut_rotate_clockwise),
    "unrotate_wrong_way": ("unrotate", _mut_unrotate_wrong_way),
    "theta_exponent_m_over_D": ("thetas", _mut_thetas_exponent),
    "dalpha_reversed_positions": ("dalpha_chain", _mut_dalpha_reversed_positions),
    "dalpha_theta_not_theta_hat": ("dalpha_chain", _mut_dalpha_theta_not_theta_hat),
    "dalpha_sign": ("dalpha_chain", _mut_dalpha_sign),
    "dalpha_drops_query_part": ("dalpha_chain", _mut_dalpha_keys_only),
    "mask_excludes_diagonal": ("_scores", _mut_scores_strict_mask),
    "lse_drops_sum": ("_logsumexp", _mut_lse_drops_sum),
    "dv_transposed": ("_head_bwd", _mut_head_bwd("dv_transposed")),
    "dk_transposed": ("_head_bwd", _mut_head_bwd("dk_transposed")),
    "dq_no_scale": ("_head_bwd", _mut_head_bwd("dq_no_scale")),
    "dk_left_in_rotated_frame": ("_head_bwd", _mut_head_bwd("dk_rotated_frame")),
    "dk_ignores_scale_argument": ("_head_bwd", _mut_head_bwd("dk_default_scale")),
    "partial_rope_ignored": ("theta_hat", _mut_theta_hat_ignores_rot),
    "partial_rope_one_band_too_many": ("theta_hat", _mut_theta_hat_rot_off_by_one),
    "blocks_of_64_rows": ("block_visible", _mut_block_visible_64),
    "blocks_without_own_block": ("block_visible", _mut_block_visible_no_diagonal),
    "backward_ignores_blocks": ("_head_bwd", _mut_head_bwd_ignores_blocks),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(ref, attr, fn)
    caught = []
    with np.errstate(all="ignore"):
        for pin_name, pin in PIN_SET:
            try:
                pin()
            except (AssertionError, ValueError, FloatingPointError):
                caught.append(pin_name)
    assert caught, f"mutant {name} passed every pin"


def test_unmutated_oracle_passes_pin_set():
    for _, pin in PIN_SET:
        pin()
