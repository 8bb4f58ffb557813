"""Pins of the Gram-threshold selection oracle (CPU).

Each pin checks ``oracle.gram`` against something other than itself: scalar
loops on tiny inputs, closed forms (tokens on a circle, orthogonal tokens,
exact duplicates), invariances, and the cascade's properties stated on
"Cascade token selection for transformer attention acceleration"
(Methodology, steps 1-3; Contributions, Proposition 4), with hand-built
sequences whose outcome follows from the description alone.
"""
import math

import numpy as np
import pytest

from oracle import gram

TAU = 0.30            # the pages' Gram threshold (Experimental results)
THR = 1.0 - TAU ** 2  # 0.91


def _clustered(T, d, seed, n_clusters=6, spreads=(0.02, 0.05, 0.3, 0.8)):
    """Tokens drawn around a few random directions with mixed spreads, so
    that some are near-duplicates of earlier ones and some are not."""
    rng = np.random.default_rng(seed)
    c = rng.normal(size=(n_clusters, d))
    c /= np.linalg.norm(c, axis=1, keepdims=True)
    s = rng.choice(spreads, size=n_clusters)
    z = rng.integers(0, n_clusters, size=T)
    x = c[z] + rng.normal(size=(T, d)) * np.sqrt(s[z] / d)[:, None]
    return x * rng.uniform(0.5, 3.0, size=(T, 1))


def _loops_max_cosine(x):
    """Scalar loops: m_i = max over j < i of the cosine, -inf for i = 0,
    and 0 for a zero token."""
    T = len(x)
    norms = [math.sqrt(math.fsum(v * v for v in row)) for row in x]
    out = []
    for i in range(T):
        best = -math.inf
        for j in range(i):
            if norms[i] == 0 or norms[j] == 0:
                c = 0.0
            else:
                c = math.fsum(a * b for a, b in zip(x[i], x[j])) / (norms[i] * norms[j])
            best = max(best, c)
        out.append(best)
    return np.array(out)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_brute_force_loops(seed):
    x = _clustered(11, 5, seed)
    x[4] = 0.0                      # a zero token
    x[7] = 2.5 * x[2]               # an exact (scaled) duplicate
    want = _loops_max_cosine(x.tolist())
    m, rep = gram.select(x, TAU)
    assert m[0] == -np.inf and want[0] == -math.inf
    np.testing.assert_allclose(m[1:], want[1:], rtol=0, atol=1e-12)
    assert np.array_equal(rep, want < THR)


def test_batched_equals_per_sequence():
    x = np.stack([_clustered(9, 4, s) for s in range(3)])
    m, rep = gram.select(x, TAU)
    for b in range(3):
        mb, rb = gram.select(x[b], TAU)
        assert np.array_equal(m[b], mb) and np.array_equal(rep[b], rb)


def test_duplicates_are_redundant():
    x = _clustered(20, 16, 3, spreads=(0.8,))
    x[12] = 0.7 * x[3]
    x[15] = 4.0 * x[12]
    m, rep = gram.select(x, TAU)
    assert m[12] > 1 - 1e-12 and m[15] > 1 - 1e-12
    assert not rep[12] and not rep[15]
    assert rep[0]                                   # nothing precedes the first token


def test_orthogonal_tokens_are_all_representatives():
    rng = np.random.default_rng(4)
    q, _ = np.linalg.qr(rng.normal(size=(24, 24)))
    x = q[:16] * rng.uniform(0.1, 5.0, size=(16, 1))
    m, rep = gram.select(x, TAU)
    np.testing.assert_allclose(m[1:], 0.0, atol=1e-12)
    assert rep.all()


@pytest.mark.parametrize("phi_deg,all_rep", [(36.8699, True), (20.0, False)])
def test_tokens_on_a_circle(phi_deg, all_rep):
    """x_i = r_i (cos i phi, sin i phi): the nearest earlier token is the
    previous one, so m_i = cos phi for i >= 1.  cos 36.87 deg = 0.8 lies
    between 1 - tau (0.7) and 1 - tau^2 (0.91); cos 20 deg = 0.94 above."""
    phi = math.radians(phi_deg)
    T = int(math.pi / phi)
    i = np.arange(T)
    x = np.stack([np.cos(i * phi), np.sin(i * phi)], axis=1) * (1.0 + i)[:, None]
    m, rep = gram.select(x, TAU)
    np.testing.assert_allclose(m[1:], math.cos(phi), atol=1e-12)
    assert rep[0] and bool(rep[1:].all()) == all_rep and bool(rep[1:].any()) == all_rep


def test_anti_parallel_token_is_not_a_duplicate():
    """The cosine is signed: -x is as far from x as a token can be."""
    x = np.array([[1.0, 2.0, -1.0], [-1.0, -2.0, 1.0]])
    m, rep = gram.select(x, TAU)
    assert m[1] == pytest.approx(-1.0, abs=1e-12) and rep.all()


def test_strict_threshold_at_tau_zero():
    """tau = 0 puts the threshold at exactly 1: an exact duplicate (cosine 1
    computed exactly for axis-aligned tokens) is not below it."""
    x = np.array([[3.0, 0, 0], [0, 2.0, 0], [7.0, 0, 0], [1.0, 1.0, 0]])
    m, rep = gram.select(x, 0.0)
    assert m[2] == 1.0
    assert rep.tolist() == [True, True, False, True]


def test_invariances():
    """Positive scaling of tokens and an orthogonal change of features leave
    every cosine, so every decision, unchanged."""
    rng = np.random.default_rng(5)
    x = _clustered(40, 12, 6)
    q, _ = np.linalg.qr(rng.normal(size=(12, 12)))
    m0, r0 = gram.select(x, TAU)
    for y in (x * rng.uniform(0.01, 100.0, size=(40, 1)), x @ q):
        m, r = gram.select(y, TAU)
        np.testing.assert_allclose(m[1:], m0[1:], atol=1e-12)
        near = np.abs(m0 - THR) < 1e-9
        assert np.array_equal(r[~near], r0[~near])


# ------------------------------------------------------------------ cascade

def _angles(deg):
    a = np.radians(np.asarray(deg, dtype=np.float64))
    return np.stack([np.cos(a), np.sin(a)], axis=1)


def test_cascade_inheriting_everything_is_the_selection():
    x = _clustered(30, 8, 7)
    m0, r0 = gram.select(x, TAU)
    m, r, valid = gram.cascade(x, TAU, np.ones(30))
    assert np.array_equal(r, r0) and np.array_equal(valid, r0)
    np.testing.assert_array_equal(m, m0)


def test_cascade_inheriting_nothing_selects_everything():
    x = _clustered(30, 8, 8)
    m, r, valid = gram.cascade(x, TAU, np.zeros(30))
    assert r.all() and not valid.any() and np.all(m == -np.inf)


@pytest.mark.parametrize("seed", range(6))
def test_cascade_is_conservative(seed):
    """Proposition 4: whatever set is inherited, every representative of the
    selection rule on the same tokens is kept."""
    rng = np.random.default_rng(100 + seed)
    x = _clustered(60, 10, seed)
    _, r0 = gram.select(x, TAU)
    for p in (0.1, 0.5, 0.9):
        prev = rng.random(60) < p
        _, r, _ = gram.cascade(x, TAU, prev)
        assert np.all(r[r0]), (p, np.flatnonzero(r0 & ~r))


def test_cascade_cross_check_uses_valid_members_only():
    """a (0 deg), b (20 deg), c (40 deg); R = {a, b}.  b is within 20 deg of a
    (cos 0.94 >= 0.91), so b is dropped; c is 40 deg from a (cos 0.77) and is
    checked against the valid member a only, so it becomes a representative
    although it is within 20 deg of b.  The selection rule alone keeps only a."""
    x = _angles([0, 20, 40])
    _, r0 = gram.select(x, TAU)
    m, r, valid = gram.cascade(x, TAU, [1, 1, 0])
    assert r0.tolist() == [True, False, False]
    assert valid.tolist() == [True, False, False]
    assert r.tolist() == [True, False, True]
    assert m[2] == pytest.approx(math.cos(math.radians(40)), abs=1e-12)


def test_cascade_member_check_uses_members_only():
    """R = {a, c}: c is validated against a alone (the r x r product), so it
    stays although b, outside R, lies within 20 deg of it; b is then checked
    against the valid members before it (a) and stays out."""
    x = _angles([0, 20, 40])
    m, r, valid = gram.cascade(x, TAU, [1, 0, 1])
    assert valid.tolist() == [True, False, True]
    assert r.tolist() == [True, False, True]
    assert m[1] == pytest.approx(math.cos(math.radians(20)), abs=1e-12)


def test_cascade_cross_check_is_causal():
    """Token 0 is outside R and token 1, its exact duplicate, is in R: no
    valid member precedes token 0, so it becomes a representative; token 1
    has no member before it and stays valid."""
    x = np.array([[1.0, 2.0], [1.0, 2.0], [-2.0, 1.0]])
    m, r, valid = gram.cascade(x, TAU, [0, 1, 0])
    assert valid.tolist() == [False, True, False]
    assert m[0] == -np.inf and m[1] == -np.inf
    assert r.tolist() == [True, True, True]


@pytest.mark.parametrize("seed", [0, 1])
def test_cascade_brute_force(seed):
    """Scalar loops of steps 1-3 on tiny inputs with a random inherited set."""
    rng = np.random.default_rng(seed)
    x = _clustered(12, 4, 50 + seed)
    prev = rng.random(12) < 0.5
    xs = x.tolist()

    def cos(i, j):
        ni = math.sqrt(math.fsum(v * v for v in xs[i]))
        nj = math.sqrt(math.fsum(v * v for v in xs[j]))
        return math.fsum(a * b for a, b in zip(xs[i], xs[j])) / (ni * nj)

    R = [i for i in range(12) if prev[i]]
    want_m = [None] * 12
    valid = set()
    for i in R:
        want_m[i] = max([cos(i, j) for j in R if j < i], default=-math.inf)
        if want_m[i] < THR:
            valid.add(i)
    want_r = [i in valid for i in range(12)]
    for i in range(12):
        if not prev[i]:
            want_m[i] = max([cos(i, j) for j in valid if j < i], default=-math.inf)
            want_r[i] = want_m[i] < THR
    m, r, v = gram.cascade(x, TAU, prev)
    np.testing.assert_allclose(m, np.array(want_m), atol=1e-12)
    assert r.tolist() == want_r
    assert sorted(np.flatnonzero(v).tolist()) == sorted(valid)


def test_jaccard():
    assert gram.jaccard([1, 1, 0, 0], [1, 0, 1, 0]) == pytest.approx(1 / 3)
    assert gram.jaccard([0, 0], [0, 0]) == 1.0


def test_cascade_with_given_decisions():
    """Decisions of step 2 passed in are the ones the cross check uses."""
    x = _angles([0, 20, 40])
    _, r, valid = gram.cascade(x, TAU, [1, 1, 0], valid_given=[1, 1, 0])
    assert valid.tolist() == [True, True, False] and r.tolist() == [True, True, False]


def test_synthetic_layers_are_coherent():
    """The seeded token stacks behave as the pages describe deep layers:
    consecutive layers' representative sets overlap strongly (Jaccard well
    above chance) and the cascade from the previous layer is a superset."""
    from bwd_rope_apply_amd import workloads as W
    wl = W.get_tokens("gram_gpt2_512")
    x0, x1 = (W.storage_to_f64(a)[0] for a in W.make_tokens(wl, layers=2))
    _, r0 = gram.select(x0, wl.tau)
    _, r1 = gram.select(x1, wl.tau)
    _, rc, _ = gram.cascade(x1, wl.tau, r0)
    assert 0.1 < r0.mean() < 0.7
    assert gram.jaccard(r0, r1) > 0.8
    assert np.all(rc[r1])


def test_sampled_rows_match_the_full_definition():
    x = _clustered(50, 6, 9)
    rows = np.array([0, 1, 7, 33, 49])
    m, _ = gram.select(x, TAU)
    np.testing.assert_allclose(gram.max_cosine_rows(x, rows), m[rows], rtol=0, atol=1e-12)
    prev = np.zeros(50, dtype=bool)
    prev[::3] = True
    mc, _, valid = gram.cascade(x, TAU, prev)
    R, V = np.flatnonzero(prev), np.flatnonzero(valid)
    for i in rows:
        want = mc[i]
        got = gram.max_cosine_rows(x, [i], R if prev[i] else V)[0]
        assert got == want or abs(got - want) <= 1e-12
