"""CPU pins of the rounding-point emulator (oracle/emulate.py): it computes
the oracle's function when nothing is rounded, its rounding helpers are the
formats' round-to-nearest-even, its dO scaling is exact, and it orders the
rounding choices the way the precision argument needs."""
import numpy as np
import pytest

from oracle import emulate as E
from oracle import ref as R


def _inputs(B=1, H=2, N=96, D=16, seed=0, qk=1.0):
    rng = np.random.default_rng(seed)
    q, k, v, do = (rng.standard_normal((B, H, N, D)) for _ in range(4))
    alpha = rng.normal(0.0, 0.3, D // 2)
    return q * qk, k, v, do, alpha


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("corner", [0, 40])
def test_exact_rounding_is_the_oracle(causal, corner):
    """With no rounding (and float64 outputs) every output equals oracle.ref
    up to float64 summation order: the emulator's steps compute the same
    function, so its floors measure rounding only."""
    q, k, v, do, a = _inputs()
    o, lse = R.ref_fwd(q, k, v, 500.0, a, causal, scale=0.3)
    dq, dk, dv, da = R.ref_bwd(q, k, v, o, do, lse, 500.0, a, causal, scale=0.3)
    g = E.emulate(q, k, v, do, 500.0, a, causal, E.exact, corner=corner, scale=0.3, block=32,
                  store=False)
    for name, want in (("O", o), ("LSE", lse), ("dQ", dq), ("dK", dk), ("dV", dv), ("dalpha", da)):
        err = np.abs(g[name] - want).max() / np.abs(want).max()
        assert err < 1e-11, (name, err)


def test_bf16_rounding_is_nearest_even():
    """Ties go to the even bfloat16 mantissa; torch's CPU float32 -> bfloat16
    conversion (round to nearest even) agrees on random values."""
    import torch
    one = 1.0
    assert E.bf16(np.array([one + 2.0 ** -8]))[0] == 1.0                  # tie -> even (1)
    assert E.bf16(np.array([one + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6  # tie -> even
    assert E.bf16(np.array([one + 2.0 ** -8 + 2.0 ** -20]))[0] == 1.0 + 2.0 ** -7
    x = np.random.default_rng(1).standard_normal(10000).astype(np.float32) * 7.0
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(E.bf16(x), want)


def test_fp16_rounding_range():
    """binary16: the largest finite value, overflow past the rounding
    boundary, and subnormals down to 2^-24."""
    assert E.fp16(np.array([65519.0]))[0] == 65504.0
    assert np.isinf(E.fp16(np.array([65520.0]))[0])
    assert E.fp16(np.array([2.0 ** -24]))[0] == 2.0 ** -24
    assert E.fp16(np.array([2.0 ** -25]))[0] == 0.0                        # tie -> even (0)
    assert E.fp16(np.array([1.0 + 2.0 ** -11]))[0] == 1.0                 # tie -> even


def test_split_operands_carry_twice_the_bits():
    """hi + lo carries about twice the format's bits while lo stays a normal
    number of the format (for fp16, |x| >= 2^-3)."""
    x = np.random.default_rng(2).standard_normal(10000) * 10.0
    x = x[np.abs(x) >= 0.5]
    for rnd, bits in ((E.fp16, 21), (E.bf16, 15)):
        err = np.abs(E.split(x, rnd) - x) / np.abs(x)
        assert err.max() <= 2.0 ** -bits, (rnd.__name__, err.max())


def test_dO_scale_lands_in_4_to_8():
    rng = np.random.default_rng(3)
    for mag in (1e-30, 1e-6, 0.3, 1.0, 5.0, 7.99, 8.0, 1e9):
        d = rng.standard_normal(200) * mag
        s = E.dO_scale(d)
        assert s == 2.0 ** round(np.log2(s))
        assert 4.0 <= np.abs(d).max() * s < 8.0, mag
    assert E.dO_scale(np.zeros(10)) == 1.0


@pytest.mark.parametrize("shift", [-40, -12, 20])
def test_dO_scaling_is_exact(shift):
    """Per-head power-of-two dO scaling: gradients for dO * 2^shift are the
    unit-scale gradients times 2^shift exactly, and O, LSE do not move."""
    q, k, v, do, a = _inputs(N=64, seed=4)
    g1 = E.emulate(q, k, v, do, 1e4, a, True, E.fp16, corner=16)
    g2 = E.emulate(q, k, v, do * 2.0 ** shift, 1e4, a, True, E.fp16, corner=16)
    for n in ("dQ", "dK", "dV", "dalpha"):
        assert np.array_equal(g2[n], g1[n] * 2.0 ** shift), n
    for n in ("O", "LSE"):
        assert np.array_equal(g2[n], g1[n]), n


def test_dO_scaling_keeps_tiny_gradients_accurate():
    """Without the scale, dO at 2^-30 would sit below fp16's smallest
    subnormal and vanish; with it the floor is the unit-scale floor."""
    q, k, v, do, a = _inputs(N=80, seed=5)
    tiny = do * 2.0 ** -30
    o, lse = R.ref_fwd(q, k, v, 1e4, a, True)
    want = R.ref_bwd(q, k, v, o, tiny, lse, 1e4, a, True)
    g = E.emulate(q, k, v, tiny, 1e4, a, True, E.fp16)
    for n, w in zip(("dQ", "dK", "dV"), want[:3]):
        assert E.reading_a(g[n], w) < 2e-2, n
    assert E.fp16(tiny).max() == 0.0   # what an unscaled conversion would keep


def test_rounding_choices_are_ordered():
    """fp16 operands sit well below bf16 ones on every tensor, and both well
    above the float64 noise of the unrounded path."""
    q, k, v, do, a = _inputs(N=160, D=32, seed=6)
    o, lse = R.ref_fwd(q, k, v, 1e4, a, True)
    dq, dk, dv, da = R.ref_bwd(q, k, v, o, do, lse, 1e4, a, True)
    ref = dict(O=o, dQ=dq, dK=dk, dV=dv, dalpha=da)
    f16 = E.floors(E.emulate(q, k, v, do, 1e4, a, True, E.fp16), ref)
    b16 = E.floors(E.emulate(q, k, v, do, 1e4, a, True, E.bf16), ref)
    for n in ("O", "dQ", "dK", "dV"):
        assert 1e-5 < f16[n][0] < b16[n][0] / 3, (n, f16[n], b16[n])


def test_normaliser_of_rounded_weights_keeps_a_dominant_key():
    """A row whose weight sits on one key: normalising O by the sum of the
    rounded weights the numerator uses cancels that weight's rounding, while
    the unrounded sum leaves it (the running reference makes the weight a
    generic value)."""
    q, k, v, do, _ = _inputs(B=1, H=1, N=64, D=32, seed=7)
    v = E.bf16(v)                                      # stored values: exact in fp16
    a = np.full(16, -np.inf)                           # no rotation: theta_hat = 0
    # key 10 gets score 14 with query row 40: weight 1 - O(e^-10) on it
    k[0, 0, 10] = q[0, 0, 40] * 14.0 * np.sqrt(32) / np.sum(q[0, 0, 40] ** 2)
    o, lse = R.ref_fwd(q, k, v, 1e4, a, True)
    on = E.emulate(q, k, v, None, 1e4, a, True, E.fp16, norm_rounded=True, store=False)
    off = E.emulate(q, k, v, None, 1e4, a, True, E.fp16, norm_rounded=False, store=False)
    e_on = np.abs(on["O"][0, 0, 40] - o[0, 0, 40]).max()
    e_off = np.abs(off["O"][0, 0, 40] - o[0, 0, 40]).max()
    assert e_on < e_off / 10, (e_on, e_off)


def test_readings():
    """Reading A pools the tensor's RMS; reading B takes each row's own RMS
    (floored at 1e-3 of the tensor's)."""
    ref = np.array([[1.0, 1.0], [100.0, 100.0]])
    got = ref + np.array([[0.1, 0.0], [1.0, 0.0]])
    rms = np.sqrt(np.mean(ref ** 2))
    assert E.reading_a(got, ref) == pytest.approx(1.0 / rms)
    assert E.reading_b(got, ref) == pytest.approx(0.1)


def test_floor_table_design_choice():
    """The committed table generator on layer_2k (two full-length heads): the
    design's rounding points (fp16 operands and the split-fp16 corner) stay
    under the 2e-2 bar on every tensor under reading A, while bf16 operands
    do not; without the corner the early rows raise reading A while reading
    B (per row) does not move."""
    from oracle import floor_table as F
    rows = {v: fl for _, v, _, fl in F.table(["layer_2k"], heads=2, workers=4)}
    design, nocorner, bf = (rows[v] for v, _, _ in F.VARIANTS)
    for n in F.NAMES:
        assert design[n][0] < 2e-2 and design[n][1] < 2e-2, (n, design[n])
        assert nocorner[n][0] > design[n][0], n
        assert abs(nocorner[n][1] - design[n][1]) < 1e-3, n
    assert max(bf[n][0] for n in F.NAMES) > 2e-2
    assert "| layer_2k | fp16 + corner (design) | 128 |" in F.markdown(
        [("layer_2k", v, 128, rows[v]) for v, _, _ in F.VARIANTS])
