"""Pins of the float64 oracle against what the pages and the mathematics fix.

None of these compares the oracle with itself: each check is a closed form,
an invariant the method must satisfy, a special case that reduces to a
library routine (torch's scaled-dot-product attention and autograd), central
finite differences, or an independent derivation (the DTFT surrogate of
LeRoPE, "Theoretical analysis").  ``test_oracle_mutations.py`` plants
mistakes in the oracle and checks that these pins catch them.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import ref

RNG = np.random.default_rng(12345)


def rnd(*shape, scale=1.0):
    return RNG.normal(0.0, scale, size=shape)


def rel(a, b):
    a, b = np.asarray(a), np.asarray(b)
    den = max(np.abs(b).max(), 1e-300)
    return np.abs(a - b).max() / den


def loss(q, k, v, do, base, alpha, causal, p0=0.0, block=512, scale=None, rot=None):
    o, _ = ref.ref_fwd(q, k, v, base, alpha, causal, p0, block, scale=scale, rot=rot)
    return float((o * do).sum())


# ------------------------------------------------------------- rotation pins
def test_rotation_preserves_pair_norms():
    x = rnd(2, 3, 37, 16)
    th = ref.theta_hat(1e4, rnd(8, scale=0.3), 16)
    xt = ref.rotate(x, ref.angles(37, th, 5.0))
    n0 = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    n1 = xt[..., 0::2] ** 2 + xt[..., 1::2] ** 2
    assert rel(n1, n0) < 1e-14


def test_alpha_zero_is_textbook_complex_rope():
    """alpha = 0 is standard RoPE (LeRoPE, initialisation): each pair as a
    complex number times e^{i p theta_m}, theta_m = b^(-2m/D)."""
    N, D, b = 50, 16, 1e4
    x = rnd(N, D)
    xt = ref.rotate(x, ref.angles(N, ref.theta_hat(b, np.zeros(D // 2), D)))
    z = x[:, 0::2] + 1j * x[:, 1::2]
    m = np.arange(D // 2)
    want = z * np.exp(1j * np.arange(N)[:, None] * (b ** (-2.0 * m / D))[None, :])
    got = xt[:, 0::2] + 1j * xt[:, 1::2]
    assert np.abs(got - want).max() < 1e-13
    assert ref.theta_hat(b, None, D)[0] == 1.0  # band 0 is the fastest, rate 1


def test_alpha_trades_against_base():
    """theta_hat depends on (b, alpha) only through exp(alpha_m) b^(-2m/D):
    alpha_m = (2m/D) ln(b/b') at base b equals alpha = 0 at base b'."""
    B, H, N, D = 1, 2, 24, 8
    q, k, v, do = rnd(B, H, N, D), rnd(B, H, N, D), rnd(B, H, N, D), rnd(B, H, N, D)
    b, b2 = 1e4, 37.0
    a = (2.0 * np.arange(D // 2) / D) * np.log(b / b2)
    o1, l1 = ref.ref_fwd(q, k, v, b, a)
    o2, l2 = ref.ref_fwd(q, k, v, b2, None)
    assert rel(o1, o2) < 1e-12 and rel(l1, l2) < 1e-12
    g1 = ref.ref_bwd(q, k, v, o1, do, l1, b, a)
    g2 = ref.ref_bwd(q, k, v, o2, do, l2, b2, None)
    for x, y in zip(g1[:3], g2[:3]):
        assert rel(x, y) < 1e-11


# -------------------------------------------------------------- invariants
@pytest.mark.parametrize("causal", [True, False])
def test_relative_offset_invariance(causal):
    """Scores depend only on i - j, so a global position shift p0 leaves O,
    LSE, dQ, dK, dV and dalpha unchanged."""
    B, H, N, D = 1, 2, 33, 16
    q, k, v, do = rnd(B, H, N, D), rnd(B, H, N, D), rnd(B, H, N, D), rnd(B, H, N, D)
    a = rnd(D // 2, scale=0.2)
    base = 1e4
    o0, l0 = ref.ref_fwd(q, k, v, base, a, causal, 0.0)
    o1, l1 = ref.ref_fwd(q, k, v, base, a, causal, 12345.0)
    assert rel(o1, o0) < 1e-9 and rel(l1, l0) < 1e-9
    g0 = ref.ref_bwd(q, k, v, o0, do, l0, base, a, causal, 0.0)
    g1 = ref.ref_bwd(q, k, v, o1, do, l1, base, a, causal, 12345.0)
    for x, y in zip(g1, g0):
        assert rel(x, y) < 1e-8


@pytest.mark.parametrize("causal", [True, False])
def test_softmax_rows(causal):
    N = 19
    d = ref.ref_dense(rnd(1, 2, N, 8), rnd(1, 2, N, 8), rnd(1, 2, N, 8), rnd(1, 2, N, 8),
                      1e4, rnd(4, scale=0.1), causal)
    P = d["P"]
    assert np.abs(P.sum(-1) - 1.0).max() < 1e-14
    assert (P >= 0).all()
    if causal:
        assert (P[..., np.triu_indices(N, 1)[0], np.triu_indices(N, 1)[1]] == 0).all()
    # gamma = gamma_1 - gamma_2 removes the P-weighted mean of beta: rows of dS sum to 0
    assert np.abs(d["dS"].sum(-1)).max() < 1e-13 * max(1.0, np.abs(d["dP"]).max())


def test_rotational_balance():
    """A common rotation of every query and key pair of band m leaves all
    scores unchanged, so per (b, h, m): sum_i wedge(q_i, dQ_i) +
    sum_j wedge(k_j, dK_j) = 0."""
    B, H, N, D = 2, 2, 40, 16
    q, k, v, do = rnd(B, H, N, D), rnd(B, H, N, D), rnd(B, H, N, D), rnd(B, H, N, D)
    a = rnd(D // 2, scale=0.3)
    o, l = ref.ref_fwd(q, k, v, 1e4, a, block=7)
    dq, dk, dv, da = ref.ref_bwd(q, k, v, o, do, l, 1e4, a, block=7)
    bal = ref.wedge(q, dq).sum(axis=2) + ref.wedge(k, dk).sum(axis=2)
    scale = ref.wedge(q, dq).__abs__().sum(axis=2).max()
    assert np.abs(bal).max() < 1e-12 * scale


def test_linearity():
    B, H, N, D = 1, 2, 21, 8
    q, k, v = rnd(B, H, N, D), rnd(B, H, N, D), rnd(B, H, N, D)
    d1, d2 = rnd(B, H, N, D), rnd(B, H, N, D)
    a = rnd(D // 2, scale=0.2)
    o, l = ref.ref_fwd(q, k, v, 1e4, a)
    g1 = ref.ref_bwd(q, k, v, o, d1, l, 1e4, a)
    g2 = ref.ref_bwd(q, k, v, o, d2, l, 1e4, a)
    g12 = ref.ref_bwd(q, k, v, o, 2.0 * d1 - 3.0 * d2, l, 1e4, a)
    for x, y, z in zip(g1, g2, g12):
        assert rel(z, 2.0 * x - 3.0 * y) < 1e-12
    o2, _ = ref.ref_fwd(q, k, 2.0 * v - 1.5, 1e4, a)
    assert rel(o2, 2.0 * o - 1.5) < 1e-13  # rows of P sum to one


def test_block_size_does_not_change_results():
    B, H, N, D = 1, 2, 45, 8
    q, k, v, do = rnd(B, H, N, D), rnd(B, H, N, D), rnd(B, H, N, D), rnd(B, H, N, D)
    a = rnd(D // 2, scale=0.2)
    for causal in (True, False):
        o1, l1 = ref.ref_fwd(q, k, v, 1e4, a, causal, block=512)
        o2, l2 = ref.ref_fwd(q, k, v, 1e4, a, causal, block=4)
        assert rel(o1, o2) < 1e-13 and rel(l1, l2) < 1e-13
        g1 = ref.ref_bwd(q, k, v, o1, do, l1, 1e4, a, causal, block=512)
        g2 = ref.ref_bwd(q, k, v, o1, do, l1, 1e4, a, causal, block=4)
        for x, y in zip(g1, g2):
            assert rel(x, y) < 1e-12


# ------------------------------------------------------------ closed forms
def test_zero_queries():
    """Q = 0: uniform attention over j <= i, LSE_i = ln(i+1),
    O_i = mean_{j<=i} V_j, dK = 0."""
    B, H, N, D = 1, 2, 30, 8
    q = np.zeros((B, H, N, D))
    k, v, do = rnd(B, H, N, D), rnd(B, H, N, D), rnd(B, H, N, D)
    a = rnd(D // 2, scale=0.2)
    o, l = ref.ref_fwd(q, k, v, 1e4, a, block=8)
    i = np.arange(N)
    assert np.abs(l - np.log(i + 1.0)).max() < 1e-14
    assert np.abs(o - np.cumsum(v, axis=2) / (i + 1.0)[:, None]).max() < 1e-14
    dq, dk, dv, da = ref.ref_bwd(q, k, v, o, do, l, 1e4, a, block=8)
    assert np.abs(dk).max() == 0.0


def test_single_position():
    """N = 1: O = V, LSE = q.k / sqrt(D) (angle 0), dQ = dK = 0, dV = dO,
    dalpha = 0."""
    D = 16
    q, k, v, do = rnd(1, 3, 1, D), rnd(1, 3, 1, D), rnd(1, 3, 1, D), rnd(1, 3, 1, D)
    a = rnd(D // 2, scale=0.2)
    for causal in (True, False):
        o, l = ref.ref_fwd(q, k, v, 1e4, a, causal)
        assert np.array_equal(o, v)
        assert np.abs(l - (q * k).sum(-1) / 4.0).max() < 1e-15
        dq, dk, dv, da = ref.ref_bwd(q, k, v, o, do, l, 1e4, a, causal)
        # dS = P (dP - D) with P = 1 and dP = D = dO.V: zero up to the
        # rounding of two equal dot products
        assert np.abs(dq).max() < 1e-14 and np.abs(dk).max() < 1e-14
        assert np.array_equal(dv, do) and np.abs(da).max() < 1e-14


def test_causal_row_zero():
    """Row 0 only sees key 0: O_0 = V_0, LSE_0 = q_0.k_0/sqrt(D), dQ_0 = 0."""
    B, H, N, D = 1, 2, 17, 8
    q, k, v, do = rnd(B, H, N, D), rnd(B, H, N, D), rnd(B, H, N, D), rnd(B, H, N, D)
    a = rnd(D // 2)
    o, l = ref.ref_fwd(q, k, v, 1e4, a)
    assert np.array_equal(o[:, :, 0], v[:, :, 0])
    assert np.abs(l[:, :, 0] - (q[:, :, 0] * k[:, :, 0]).sum(-1) / np.sqrt(D)).max() < 1e-15
    dq, dk, dv, da = ref.ref_bwd(q, k, v, o, do, l, 1e4, a)
    assert np.abs(dq[:, :, 0]).max() < 1e-15


def test_identical_value_rows():
    """All V rows equal v: O_i = v, dQ = dK = 0, dalpha = 0."""
    B, H, N, D = 1, 2, 26, 8
    q, k, do = rnd(B, H, N, D), rnd(B, H, N, D), rnd(B, H, N, D)
    v = np.broadcast_to(rnd(B, H, 1, D), (B, H, N, D)).copy()
    a = rnd(D // 2, scale=0.3)
    for causal in (True, False):
        o, l = ref.ref_fwd(q, k, v, 1e4, a, causal, block=5)
        assert np.abs(o - v).max() < 1e-13
        dq, dk, dv, da = ref.ref_bwd(q, k, v, o, do, l, 1e4, a, causal, block=5)
        assert np.abs(dq).max() < 1e-13 and np.abs(dk).max() < 1e-13
        assert np.abs(da).max() < 1e-12


def test_brute_force_forward_tiny():
    """Scalar-loop evaluation of the forward (math module, no numpy) on a
    tiny case with several query blocks."""
    B, H, N, D = 1, 1, 7, 4
    q, k, v = rnd(B, H, N, D), rnd(B, H, N, D), rnd(B, H, N, D)
    a, base = rnd(D // 2, scale=0.4), 10.0
    o, l = ref.ref_fwd(q, k, v, base, a, True, block=3)
    th = [math.exp(a[m]) * base ** (-2.0 * m / D) for m in range(D // 2)]

    def rot(x, p):
        out = [0.0] * D
        for m in range(D // 2):
            c, s = math.cos(p * th[m]), math.sin(p * th[m])
            out[2 * m] = x[2 * m] * c - x[2 * m + 1] * s
            out[2 * m + 1] = x[2 * m] * s + x[2 * m + 1] * c
        return out

    for i in range(N):
        qi = rot(list(q[0, 0, i]), i)
        s = [sum(a_ * b_ for a_, b_ in zip(qi, rot(list(k[0, 0, j]), j))) / math.sqrt(D)
             for j in range(i + 1)]
        mx = max(s)
        z = sum(math.exp(x - mx) for x in s)
        assert abs(l[0, 0, i] - (mx + math.log(z))) < 1e-13
        for c in range(D):
            oc = sum(math.exp(s[j] - mx) / z * v[0, 0, j, c] for j in range(i + 1))
            assert abs(o[0, 0, i, c] - oc) < 1e-13


# ----------------------------------------------------- library reductions
torch = pytest.importorskip("torch")


@pytest.mark.parametrize("causal", [True, False])
def test_zero_rotation_is_sdpa(causal):
    """alpha = -inf on every band removes the rotation (theta_hat = 0): the
    result is plain attention, i.e. torch's float64 CPU SDPA with scale
    1/sqrt(D), and its autograd gradients; dalpha = 0."""
    B, H, N, D = 2, 3, 70, 16
    q, k, v, do = rnd(B, H, N, D), rnd(B, H, N, D), rnd(B, H, N, D), rnd(B, H, N, D)
    a = np.full(D // 2, -np.inf)
    o, l = ref.ref_fwd(q, k, v, 1e4, a, causal, block=16)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    to = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal)
    assert rel(o, to.detach().numpy()) < 1e-12
    (to * torch.tensor(do)).sum().backward()
    dq, dk, dv, da = ref.ref_bwd(q, k, v, o, do, l, 1e4, a, causal, block=16)
    assert rel(dq, tq.grad.numpy()) < 1e-11
    assert rel(dk, tk.grad.numpy()) < 1e-11
    assert rel(dv, tv.grad.numpy()) < 1e-11
    assert np.abs(da).max() == 0.0


@pytest.mark.parametrize("causal", [True, False])
def test_autograd_through_complex_rotation(causal):
    """Independent autodiff: rotate with torch complex multiplication by
    polar(1, (p + p0) e^alpha theta), attend with torch SDPA, differentiate
    with torch autograd (Q, K, V and alpha)."""
    B, H, N, D = 1, 2, 48, 16
    base, p0 = 500.0, 3.0
    q, k, v, do = rnd(B, H, N, D), rnd(B, H, N, D), rnd(B, H, N, D), rnd(B, H, N, D)
    a = rnd(D // 2, scale=0.4)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    ta = torch.tensor(a, requires_grad=True)
    m = torch.arange(D // 2, dtype=torch.float64)
    th = torch.exp(ta) * base ** (-2.0 * m / D)
    pos = torch.arange(N, dtype=torch.float64) + p0
    e = torch.polar(torch.ones(N, D // 2, dtype=torch.float64), pos[:, None] * th[None, :])

    def rot(x):
        z = torch.view_as_complex(x.reshape(B, H, N, D // 2, 2).contiguous())
        return torch.view_as_real(z * e).reshape(B, H, N, D)

    to = torch.nn.functional.scaled_dot_product_attention(rot(tq), rot(tk), tv, is_causal=causal)
    (to * torch.tensor(do)).sum().backward()
    o, l = ref.ref_fwd(q, k, v, base, a, causal, p0, block=10)
    assert rel(o, to.detach().numpy()) < 1e-12
    dq, dk, dv, da = ref.ref_bwd(q, k, v, o, do, l, base, a, causal, p0, block=10)
    assert rel(dq, tq.grad.numpy()) < 1e-11
    assert rel(dk, tk.grad.numpy()) < 1e-11
    assert rel(dv, tv.grad.numpy()) < 1e-11
    assert rel(da, ta.grad.numpy()) < 1e-10


@pytest.mark.parametrize("scale,rot,p0", [(0.3, 5, 7.0), (None, 0, 0.0), (0.11, 8, 1000.0)])
def test_autograd_frequency_variants(scale, rot, p0):
    """Partial RoPE, a softmax scale and a position offset, independently:
    torch complex rotation of the first `rot` pairs only (the rest pass
    through), torch SDPA with the given scale, torch autograd for Q, K, V and
    alpha (whose slower, unrotated bands get zero gradient)."""
    B, H, N, D = 1, 2, 40, 16
    base, causal = 300.0, True
    q, k, v, do = rnd(B, H, N, D), rnd(B, H, N, D), rnd(B, H, N, D), rnd(B, H, N, D)
    a = rnd(D // 2, scale=0.4)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    ta = torch.tensor(a, requires_grad=True)
    m = torch.arange(D // 2, dtype=torch.float64)
    live = (m < rot).double()
    th = torch.exp(ta) * base ** (-2.0 * m / D)
    pos = torch.arange(N, dtype=torch.float64) + p0
    e = torch.polar(torch.ones(N, D // 2, dtype=torch.float64), pos[:, None] * (th * live)[None, :])

    def rot_(x):
        z = torch.view_as_complex(x.reshape(B, H, N, D // 2, 2).contiguous())
        return torch.view_as_real(z * e).reshape(B, H, N, D)

    to = torch.nn.functional.scaled_dot_product_attention(rot_(tq), rot_(tk), tv, is_causal=causal,
                                                          scale=scale)
    (to * torch.tensor(do)).sum().backward()
    kw = dict(scale=scale, rot=rot)
    o, l = ref.ref_fwd(q, k, v, base, a, causal, p0, block=9, **kw)
    assert rel(o, to.detach().numpy()) < 1e-12
    dq, dk, dv, da = ref.ref_bwd(q, k, v, o, do, l, base, a, causal, p0, block=9, **kw)
    assert rel(dq, tq.grad.numpy()) < 1e-10
    assert rel(dk, tk.grad.numpy()) < 1e-10
    assert rel(dv, tv.grad.numpy()) < 1e-11
    tg = ta.grad.numpy()
    assert np.abs(tg[rot:]).max(initial=0.0) == 0.0 and np.abs(da[rot:]).max(initial=0.0) == 0.0
    if rot > 0:
        # the offset term of dalpha cancels by rotational balance, so with a
        # large offset the two sides agree to the size of that cancellation
        assert rel(da[:rot], tg[:rot]) < (1e-10 if p0 < 100 else 1e-8)


def test_scale_is_query_scaling():
    """A softmax scale c / sqrt(D) equals the default scale on queries
    multiplied by c (the rotation is linear): same O and LSE, dQ multiplied
    by c, the same dK, dV and dalpha."""
    B, H, N, D, c = 2, 2, 33, 8, 1.7
    q, k, v, do = rnd(B, H, N, D), rnd(B, H, N, D), rnd(B, H, N, D), rnd(B, H, N, D)
    a = rnd(D // 2, scale=0.3)
    o1, l1 = ref.ref_fwd(q, k, v, 50.0, a, True, block=8, scale=c / math.sqrt(D))
    o2, l2 = ref.ref_fwd(c * q, k, v, 50.0, a, True, block=8)
    assert rel(o1, o2) < 1e-13 and np.abs(l1 - l2).max() < 1e-12
    g1 = ref.ref_bwd(q, k, v, o1, do, l1, 50.0, a, True, block=8, scale=c / math.sqrt(D))
    g2 = ref.ref_bwd(c * q, k, v, o2, do, l2, 50.0, a, True, block=8)
    assert rel(g1[0], c * g2[0]) < 1e-12
    for x, y in zip(g1[1:], g2[1:]):
        assert rel(x, y) < 1e-12


# ------------------------------------------------------------ block lists
def _random_blocks(rng, B, H, nb, causal, p=0.4):
    out = []
    for b in range(B):
        out.append([])
        for h in range(H):
            rows = []
            for qb in range(nb):
                cand = range(qb) if causal else range(nb)
                rows.append([kb for kb in cand if kb != qb and rng.random() < p])
            out[b].append(rows)
    return out


@pytest.mark.parametrize("causal", [True, False])
def test_block_list_all_blocks_is_dense(causal):
    """Listing every block reproduces causal (or full) attention exactly."""
    B, H, N, D = 1, 2, 300, 8
    q, k, v, do = rnd(B, H, N, D), rnd(B, H, N, D), rnd(B, H, N, D), rnd(B, H, N, D)
    nb = 3
    allb = [[[list(range(nb)) for _ in range(nb)] for _ in range(H)] for _ in range(B)]
    o1, l1 = ref.ref_fwd(q, k, v, 100.0, None, causal, block=50, blocks=allb)
    o2, l2 = ref.ref_fwd(q, k, v, 100.0, None, causal, block=50)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


@pytest.mark.parametrize("causal", [True, False])
def test_block_list_brute_force(causal):
    """Per query row, a plain softmax over exactly the keys of its visible
    blocks (own block, listed blocks, causal mask), with the rotation in its
    textbook complex form, element by element in Python loops."""
    B, H, N, D, base = 1, 1, 300, 4, 50.0
    rng = np.random.default_rng(7 + causal)
    q, k, v = (rng.normal(size=(B, H, N, D)) for _ in range(3))
    a = rng.normal(0, 0.3, size=D // 2)
    blocks = _random_blocks(rng, B, H, 3, causal, p=0.5)
    o, lse = ref.ref_fwd(q, k, v, base, a, causal, block=64, blocks=blocks)
    th = np.exp(a) * base ** (-2.0 * np.arange(D // 2) / D)
    zq = (q[0, 0, :, 0::2] + 1j * q[0, 0, :, 1::2]) * np.exp(1j * np.arange(N)[:, None] * th)
    zk = (k[0, 0, :, 0::2] + 1j * k[0, 0, :, 1::2]) * np.exp(1j * np.arange(N)[:, None] * th)
    sel = blocks[0][0]
    for i in range(0, N, 7):
        qb = i // 128
        keys = [j for j in range(N) if (j // 128 == qb or j // 128 in sel[qb]) and (not causal or j <= i)]
        s = np.array([np.real(np.sum(zq[i] * np.conj(zk[j]))) / math.sqrt(D) for j in keys])
        mx = s.max()
        w = np.exp(s - mx)
        want_lse = mx + math.log(w.sum())
        want_o = (w[:, None] * v[0, 0, keys]).sum(axis=0) / w.sum()
        assert abs(lse[0, 0, i] - want_lse) < 1e-12
        assert np.abs(o[0, 0, i] - want_o).max() < 1e-12


def test_block_list_lse_merge():
    """Inclusion-exclusion over key sets: with S0 = {own}, S1 = S0 + {b1},
    S2 = S0 + {b2}, S3 = S0 + {b1, b2}: e^L3 = e^L1 + e^L2 - e^L0 and
    e^L3 O3 = e^L1 O1 + e^L2 O2 - e^L0 O0 (non-causal, query block 2)."""
    B, H, N, D = 1, 1, 384, 8
    q, k, v = rnd(B, H, N, D, scale=0.5), rnd(B, H, N, D, scale=0.5), rnd(B, H, N, D)
    res = {}
    for name, extra in (("0", []), ("1", [0]), ("2", [1]), ("3", [0, 1])):
        bl = [[[[], [], extra]]]
        res[name] = ref.ref_fwd(q, k, v, 100.0, None, False, block=64, blocks=bl)
    rows = slice(256, 384)
    e = {n: np.exp(res[n][1][0, 0, rows])[:, None] for n in res}
    o = {n: res[n][0][0, 0, rows] for n in res}
    assert rel(e["3"], e["1"] + e["2"] - e["0"]) < 1e-12
    assert rel(e["3"] * o["3"], e["1"] * o["1"] + e["2"] * o["2"] - e["0"] * o["0"]) < 1e-11


@pytest.mark.parametrize("causal", [True, False])
def test_block_list_finite_differences(causal):
    """Central differences of sum(O * dO) for Q, K, V and alpha under a
    sparse block pattern (N = 260: three blocks, ragged)."""
    B, H, N, D, h, base = 1, 1, 260, 4, 1e-6, 30.0
    rng = np.random.default_rng(11 + causal)
    q, k, v, do = (rng.normal(size=(B, H, N, D)) for _ in range(4))
    a = rng.normal(0, 0.3, size=D // 2)
    bl = [[[[], [0], [1]] if causal else [[2], [], [0, 1]]]]
    o, l = ref.ref_fwd(q, k, v, base, a, causal, block=100, blocks=bl)
    g = ref.ref_bwd(q, k, v, o, do, l, base, a, causal, block=100, blocks=bl)

    def L():
        return float((ref.ref_fwd(q, k, v, base, a, causal, block=100, blocks=bl)[0] * do).sum())
    for gi, x in enumerate((q, k, v)):
        for idx in [(0, 0, i, c) for i in (0, 127, 128, 200, 259) for c in range(D)]:
            x0 = x[idx]
            x[idx] = x0 + h
            lp = L()
            x[idx] = x0 - h
            lm = L()
            x[idx] = x0
            assert abs((lp - lm) / (2 * h) - g[gi][idx]) < 1e-7 * max(1.0, abs(g[gi][idx])), (gi, idx)
    for m in range(D // 2):
        a0 = a[m]
        a[m] = a0 + h
        lp = L()
        a[m] = a0 - h
        lm = L()
        a[m] = a0
        assert abs((lp - lm) / (2 * h) - g[3][m]) < 1e-7 * max(1.0, abs(g[3][m]))


# ---------------------------------------------------- finite differences
FD_CASES = [
    (1, 4, 10.0, True, None, None), (2, 8, 1e4, True, None, None), (5, 4, 10.0, True, None, None),
    (16, 8, 1e4, True, None, None), (5, 8, 1e4, False, None, None), (16, 4, 10.0, False, None, None),
    # frequency-schedule variants: softmax scale and partial rotation
    (5, 8, 1e4, True, 0.21, 3), (9, 8, 10.0, False, 0.6, 1), (6, 4, 10.0, True, None, 0),
]


@pytest.mark.parametrize("N,D,base,causal,scale,rot", FD_CASES)
def test_finite_differences_all_gradients(N, D, base, causal, scale, rot):
    """Central differences (h = 1e-6) of L = sum(O * dO) over every entry of
    Q, K, V and every alpha_m, B = 1, H = 2 (also at a non-default softmax
    scale and with only the first `rot` bands rotated)."""
    B, H, h = 1, 2, 1e-6
    rng = np.random.default_rng(N * 100 + D + int(causal))
    q, k, v, do = (rng.normal(size=(B, H, N, D)) for _ in range(4))
    a = rng.normal(0, 0.3, size=D // 2)
    blk = 3
    kw = dict(scale=scale, rot=rot)
    o, l = ref.ref_fwd(q, k, v, base, a, causal, block=blk, **kw)
    grads = ref.ref_bwd(q, k, v, o, do, l, base, a, causal, block=blk, **kw)
    for gi, x in enumerate((q, k, v)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            x0 = x[idx]
            x[idx] = x0 + h
            lp = loss(q, k, v, do, base, a, causal, block=blk, **kw)
            x[idx] = x0 - h
            lm = loss(q, k, v, do, base, a, causal, block=blk, **kw)
            x[idx] = x0
            fd[idx] = (lp - lm) / (2 * h)
        assert np.abs(fd - grads[gi]).max() < 1e-7 * max(1.0, np.abs(fd).max()), gi
    fa = np.zeros_like(a)
    for m in range(a.size):
        a0 = a[m]
        a[m] = a0 + h
        lp = loss(q, k, v, do, base, a, causal, block=blk, **kw)
        a[m] = a0 - h
        lm = loss(q, k, v, do, base, a, causal, block=blk, **kw)
        a[m] = a0
        fa[m] = (lp - lm) / (2 * h)
    assert np.abs(fa - grads[3]).max() < 1e-7 * max(1.0, np.abs(fa).max())


# ------------------------------------------------------- dalpha three ways
@pytest.mark.parametrize("causal", [True, False])
def test_dalpha_three_derivations(causal):
    """Chain rule (oracle.ref), DTFT surrogate slope (oracle.dtft) and
    finite differences agree."""
    B, H, N, D, base = 2, 2, 12, 8, 10.0
    rng = np.random.default_rng(7)
    q, k, v, do = (rng.normal(size=(B, H, N, D)) for _ in range(4))
    a = rng.normal(0, 0.3, size=D // 2)
    o, l = ref.ref_fwd(q, k, v, base, a, causal)
    chain = ref.ref_bwd(q, k, v, o, do, l, base, a, causal)[3]
    dt = oracle.dalpha_dtft(q, k, v, do, base, a, causal)
    assert rel(dt, chain) < 1e-10
    h = 1e-6
    fd = np.zeros_like(a)
    for m in range(a.size):
        ap, am = a.copy(), a.copy()
        ap[m] += h
        am[m] -= h
        fd[m] = (loss(q, k, v, do, base, ap, causal) - loss(q, k, v, do, base, am, causal)) / (2 * h)
    assert rel(fd, chain) < 1e-7


def test_surrogate_slope_is_its_derivative():
    """P_m'(theta) from the closed-form sum matches central differences of
    P_m(theta) itself."""
    rng = np.random.default_rng(3)
    G = rng.normal(size=(4, 19)) + 1j * rng.normal(size=(4, 19))
    th = rng.uniform(0.01, 2.0, size=4)
    h = 1e-6
    fd = (oracle.surrogate(G, th + h) - oracle.surrogate(G, th - h)) / (2 * h)
    assert rel(oracle.surrogate_slope(G, th), fd) < 1e-8


# --------------------------------------------------- sampled-row evaluation
def test_head_rows_match_full_head():
    N, D = 150, 16
    rng = np.random.default_rng(11)
    q, k, v, do = (rng.normal(size=(1, 1, N, D)) for _ in range(4))
    a = rng.normal(0, 0.2, size=D // 2)
    rows = [0, 1, 63, 64, 149]
    cols = [0, 5, 100, 149]
    for causal in (True, False):
        o, l = ref.ref_fwd(q, k, v, 1e4, a, causal, block=40)
        dq, dk, dv, _ = ref.ref_bwd(q, k, v, o, do, l, 1e4, a, causal, block=40)
        r = ref.ref_head_rows(q[0, 0], k[0, 0], v[0, 0], do[0, 0], 1e4, a, causal,
                              rows, cols, block=32)
        assert rel(r["O"], o[0, 0]) < 1e-14 and rel(r["LSE"], l[0, 0]) < 1e-14
        assert rel(r["dQ"], dq[0, 0, rows]) < 1e-12
        assert rel(r["dK"], dk[0, 0, cols]) < 1e-12
        assert rel(r["dV"], dv[0, 0, cols]) < 1e-12
