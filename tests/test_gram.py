"""GPU parity of Gram-threshold token selection and its cascade step against
the float64 oracle (``oracle.gram``), through the C ABI.

Bar (derived in the design notes): the stored bf16 / fp16 values enter the
matrix cores unrounded and their products are exact in float32, so a cosine
carries only float32 accumulation error: |m_gpu - m_ref| <= 2 d 2^-24 +
1e-6 (two d-term sums, the dot product and the norms).  A decision whose
exact maximum lies within that band of 1 - tau^2 is taken by the GPU in its
own float32 precision and checked against its own maximum; every other
decision must equal the oracle's.  The cascade's cross check follows the
GPU's own member decisions (identical to the oracle's outside the band).
"""
import dataclasses

import numpy as np
import pytest

from bwd_rope_apply_amd import workloads as W
import harness as Hn

pytestmark = pytest.mark.gpu


def tol(d: int) -> float:
    return 2.0 * d * 2.0 ** -24 + 1e-6


def _thr32(tau):
    return float(np.float32(1.0 - float(tau) ** 2))


def _compare(m_gpu, rep_gpu, m_ref, rep_ref, tau, d, what):
    thr = 1.0 - tau ** 2
    fin = np.isfinite(m_ref)
    assert np.array_equal(np.isfinite(m_gpu), fin), what
    err = float(np.max(np.abs(m_gpu[fin] - m_ref[fin]))) if fin.any() else 0.0
    band = fin & (np.abs(m_ref - thr) <= tol(d))
    print(what, "max |m err|", err, "band", int(band.sum()), "reps", int(rep_gpu.sum()), flush=True)
    assert err <= tol(d), (what, err)
    assert np.array_equal(rep_gpu[~band].astype(bool), np.asarray(rep_ref)[~band]), what
    own = (m_gpu < _thr32(tau))
    assert np.array_equal(rep_gpu[band].astype(bool), own[band]), what
    return band


def _dev(x):
    return Hn.to_device(np.ascontiguousarray(x))


def _select(x_store, tau):
    from bwd_rope_apply_amd import gram_select
    import torch
    m, rep, cnt = gram_select(_dev(x_store), tau)
    torch.cuda.synchronize()
    return m.cpu().numpy().astype(np.float64), rep.cpu().numpy(), cnt.cpu().numpy()


@pytest.mark.parametrize("name", ["gram_gpt2_512", "gram_gptj_512"])
def test_select_workloads(name):
    """The pages' setting: T = 512, tau = 0.30, d = 768 and 4096."""
    from oracle import gram
    wl = W.get_tokens(name)
    xs = W.make_tokens(wl)[0]
    print(wl.name, flush=True)
    m, rep, cnt = _select(xs, wl.tau)
    x = W.storage_to_f64(xs)
    m_ref, rep_ref = gram.select(x, wl.tau)
    _compare(m, rep, m_ref, rep_ref, wl.tau, wl.d, wl.name)
    assert np.array_equal(cnt, rep.sum(axis=1))


@pytest.mark.parametrize("T,d,dtype", [(1, 64, "bf16"), (2, 64, "bf16"), (5, 128, "fp16"),
                                       (127, 64, "bf16"), (128, 192, "bf16"), (129, 64, "fp16"),
                                       (300, 256, "bf16"), (700, 128, "fp16")])
def test_select_shapes(T, d, dtype):
    """Ragged and exact tile multiples, one token, two sequences, both storage types."""
    from oracle import gram
    wl = dataclasses.replace(W.get_tokens("gram_gpt2_512", B=2, T=T, d=d, seed=40 + T), dtype=dtype)
    xs = W.make_tokens(wl)[0]
    print(wl.name, dtype, flush=True)
    m, rep, cnt = _select(xs, wl.tau)
    m_ref, rep_ref = gram.select(W.storage_to_f64(xs), wl.tau)
    _compare(m, rep, m_ref, rep_ref, wl.tau, d, wl.name)
    assert np.array_equal(cnt, rep.sum(axis=1))


def test_select_many_sequences():
    """16 sequences of 2048 tokens: enough tiles that the library takes its
    large (256 x 256) tiles."""
    from oracle import gram
    wl = W.get_tokens("gram_gpt2_512", B=16, T=2048, d=64, seed=5)
    xs = W.make_tokens(wl)[0]
    m, rep, cnt = _select(xs, wl.tau)
    m_ref, rep_ref = gram.select(W.storage_to_f64(xs), wl.tau)
    _compare(m, rep, m_ref, rep_ref, wl.tau, wl.d, wl.name)
    assert np.array_equal(cnt, rep.sum(axis=1))


def test_select_zero_tokens_duplicates_and_taus():
    """Zero tokens (cosine 0), exact duplicates (cosine 1 up to rounding),
    anti-parallel tokens, and the thresholds tau = 0, 0.3, 0.9."""
    from oracle import gram
    wl = W.get_tokens("gram_gpt2_512", T=260, d=128, seed=77)
    x = W.storage_to_f64(W.make_tokens(wl)[0])[0]
    x[10] = 0.0
    x[200] = 0.0
    x[50] = x[3]
    x[150] = -x[60]
    x[230] = 2.0 * x[229]
    xs = W.f32_to_bf16_bits(x.astype(np.float32))
    xd = W.bf16_bits_to_f64(xs)
    for tau in (0.0, 0.3, 0.9):
        m, rep, _ = _select(xs, tau)
        m_ref, rep_ref = gram.select(xd, tau)
        _compare(m, rep, m_ref, rep_ref, tau, 128, f"tau={tau}")
    assert m[50] == pytest.approx(1.0, abs=tol(128)) and not rep[50]
    assert m[10] == pytest.approx(0.0, abs=1e-7)


def _cascade(x_store, tau, prev):
    from bwd_rope_apply_amd import gram_cascade
    import torch
    p = torch.from_numpy(np.ascontiguousarray(prev.astype(np.uint8))).cuda()
    m, rep, cnt = gram_cascade(_dev(x_store), tau, p)
    torch.cuda.synchronize()
    return m.cpu().numpy().astype(np.float64), rep.cpu().numpy(), int(cnt.cpu().numpy()[0])


def _check_cascade(x_store, x, tau, prev, d, what):
    from oracle import gram
    m, rep, cnt = _cascade(x_store, tau, prev)
    prev = prev.astype(bool)
    valid_gpu = rep.astype(bool) & prev
    # members: the r x r check
    m_ref, rep_ref, valid_ref = gram.cascade(x, tau, prev)
    _compare(m[prev], valid_gpu[prev], m_ref[prev], valid_ref[prev], tau, d, what + " members")
    # others: the cross check against the GPU's kept members
    m_ref2, rep_ref2, _ = gram.cascade(x, tau, prev, valid_given=valid_gpu)
    _compare(m[~prev], rep[~prev], m_ref2[~prev], rep_ref2[~prev], tau, d, what + " others")
    assert cnt == int(rep.sum())
    return m, rep


@pytest.mark.parametrize("name", ["gram_gpt2_512", "gram_gptj_512"])
def test_cascade_workloads(name):
    """Layer 1 with the set the GPU selected on layer 0 (depth chaining),
    against the oracle; the result keeps every representative of the full
    rule on layer 1 (Proposition 4) outside the rounding band."""
    from oracle import gram
    wl = W.get_tokens(name)
    x0s, x1s = (a[0] for a in W.make_tokens(wl, layers=2))
    _, r0, _ = _select(x0s, wl.tau)
    x1 = W.storage_to_f64(x1s)
    m, rep = _check_cascade(x1s, x1, wl.tau, r0.astype(bool), wl.d, wl.name)
    m_full, rep_full = gram.select(x1, wl.tau)
    band = np.abs(m_full - (1 - wl.tau ** 2)) <= tol(wl.d)
    assert np.all(rep.astype(bool)[rep_full & ~band])
    print("jaccard(layer0, layer1 cascade)", gram.jaccard(r0, rep), flush=True)


@pytest.mark.parametrize("T,d,p", [(1, 64, 1.0), (7, 64, 0.5), (300, 128, 0.3), (300, 128, 0.9),
                                   (513, 64, 0.6)])
def test_cascade_random_sets(T, d, p):
    wl = W.get_tokens("gram_gpt2_512", T=T, d=d, seed=300 + T)
    xs = W.make_tokens(wl)[0][0]
    prev = np.random.default_rng(T).random(T) < p
    print(T, d, p, flush=True)
    _check_cascade(xs, W.storage_to_f64(xs), wl.tau, prev, d, f"T{T} p{p}")


def test_cascade_extremes():
    """Inheriting nothing selects every token (maxima -inf); inheriting
    everything is the selection itself, bit for bit (the same products over
    the same tiles)."""
    wl = W.get_tokens("gram_gpt2_512", T=400, d=256, seed=9)
    xs = W.make_tokens(wl)[0][0]
    m, rep, cnt = _cascade(xs, wl.tau, np.zeros(400, dtype=bool))
    assert rep.all() and np.all(m == -np.inf) and cnt == 400
    m1, rep1, _ = _cascade(xs, wl.tau, np.ones(400, dtype=bool))
    m2, rep2, _ = _select(xs, wl.tau)
    assert np.array_equal(m1, m2) and np.array_equal(rep1, rep2)


def test_full_size_8k():
    """T = 8192, d = 4096 (the pages' projected length): selection and one
    cascade step, checked at 96 sampled tokens against the oracle's
    definition evaluated at those rows, plus the count."""
    from oracle import gram
    wl = W.get_tokens("gram_8k")
    x0s, x1s = (a[0] for a in W.make_tokens(wl, layers=2))
    print(wl.name, flush=True)
    m0, r0, c0 = _select(x0s, wl.tau)
    assert int(c0[0]) == int(r0.sum())
    # inheriting every token runs the member check over all of them with the
    # small tiles; the selection at this length takes the large tiles; every
    # maximum is the same float32 sum in the same order, so they agree bit for bit
    ma, ra, _ = _cascade(x0s, wl.tau, np.ones(wl.T, dtype=bool))
    assert np.array_equal(ma, m0) and np.array_equal(ra, r0)
    x0 = W.storage_to_f64(x0s)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, 8191],
                                     np.random.default_rng(1).integers(0, wl.T, 91)]))
    ref = gram.max_cosine_rows(x0, rows)
    thr = 1 - wl.tau ** 2
    _compare(m0[rows], r0[rows], ref, ref < thr, wl.tau, wl.d, "select 8k sampled")
    del x0
    x1 = W.storage_to_f64(x1s)
    prev = r0.astype(bool)
    m1, rep1, c1 = _cascade(x1s, wl.tau, prev)
    assert c1 == int(rep1.sum())
    valid = rep1.astype(bool) & prev
    rows_r, rows_n = rows[prev[rows]], rows[~prev[rows]]
    ref_r = gram.max_cosine_rows(x1, rows_r, np.flatnonzero(prev))
    ref_n = gram.max_cosine_rows(x1, rows_n, np.flatnonzero(valid))
    _compare(m1[rows_r], rep1[rows_r], ref_r, ref_r < thr, wl.tau, wl.d, "cascade 8k members")
    _compare(m1[rows_n], rep1[rows_n], ref_n, ref_n < thr, wl.tau, wl.d, "cascade 8k others")
    print("r/T", r0.mean(), "cascade r/T", rep1.mean(), "kept", valid.sum(), flush=True)
