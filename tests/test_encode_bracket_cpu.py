"""The encoders' division-free step, checked on the CPU in binary32.

The lane kernels of the INT4 symmetric and NVFP4 encoders take a code that
depends on q = fl(v / d) from x = fl(v * fl(1 / d)) instead: when the code of
fl(x * (1 - 2^-20)) equals the code of fl(x * (1 + 2^-20)) they use it,
otherwise they divide. The claim is that agreement at the two ends implies
the code of fl(v / d) ("Why 4-Bit Quantization Is King" section 1 for INT4,
section 5 for NVFP4: both divide in binary32). Here numpy's float32
arithmetic (IEEE, round to nearest even) replays those steps on random
quotients and on quotients placed a few ulps from every rounding boundary,
and every agreeing case is compared with the code of the true quotient.
"""
import numpy as np

F = np.float32
K_BELOW = F(1.0) - F(2.0 ** -20)
K_ABOVE = F(1.0) + F(2.0 ** -20)


def int4_code(q):
    return np.clip(np.rint(q), -8, 7)  # rint is round half to even


E2M1_MID = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)


def e2m1_code(q, tie_even):
    """Code magnitude (0..7) and sign of q: the number of midpoints below |q|
    (saturating at 6), an exact midpoint going up only to an even code when
    tie_even, else staying at the lower code."""
    a = np.minimum(np.abs(q), F(6.0))
    c = np.zeros(q.shape, np.int64)
    for i, m in enumerate(E2M1_MID):
        c += (a > m) | (tie_even & (i % 2 == 1) & (a == m))
    return c + 8 * np.signbit(q)


def _bracket(v, d, code):
    inv = F(1.0) / d
    x = (v * inv).astype(F)
    lo = code((x * K_BELOW).astype(F))
    hi = code((x * K_ABOVE).astype(F))
    exact = code((v / d).astype(F))
    agree = lo == hi
    return agree, lo, exact


def _near_boundaries(rng, boundaries, d, n_per):
    """v such that v / d lies within +-6 ulps of each boundary, both signs."""
    vs = []
    for b in boundaries:
        for sgn in (1.0, -1.0):
            t = np.full(n_per, sgn * b, np.float32)
            steps = rng.integers(-6, 7, n_per)
            towards = np.where(steps > 0, np.inf, -np.inf).astype(F)
            t = np.nextafter(t, towards)  # at least one step off
            for _ in range(5):
                more = rng.integers(0, 2, n_per).astype(bool)
                t = np.where(more, np.nextafter(t, towards), t)
            t = np.where(steps == 0, F(sgn * b), t)
            vs.append((t.astype(np.float64) * d.astype(np.float64)).astype(F))
    return np.concatenate(vs)


def test_int4_bracket_implies_the_divided_code():
    rng = np.random.default_rng(20)
    n = 200_000
    amax = (10.0 ** rng.uniform(-30, 30, n)).astype(F)
    d = (amax / F(7.0)).astype(F)
    v_rand = (rng.uniform(-1, 1, n) * amax).astype(F)
    v_near = _near_boundaries(rng, [k + 0.5 for k in range(-8, 8)], d[:4000], 4000)
    v_ties = (rng.integers(-14, 15, n) * F(0.5) * d).astype(F)  # exact and near-exact half-integers
    for v, dd, name in ((v_rand, d, "random"), (v_near, np.tile(d[:4000], len(v_near) // 4000), "near"),
                        (v_ties, d, "ties")):
        agree, got, want = _bracket(v, dd, int4_code)
        assert np.array_equal(got[agree], want[agree]), name
        if name == "random":
            assert agree.mean() > 0.999  # the division is the rare path
        if name == "near":
            assert not agree.all()  # ... and it is taken next to a boundary


def test_e2m1_bracket_implies_the_divided_code():
    rng = np.random.default_rng(21)
    n = 200_000
    t = (10.0 ** rng.uniform(-30, 30, n)).astype(F)
    v_rand = (rng.uniform(-7, 7, n) * t).astype(F)
    mids = list(E2M1_MID) + [6.0]
    v_near = _near_boundaries(rng, mids, t[:4000], 4000)
    for tie_even in (True, False):
        code = lambda q: e2m1_code(q, tie_even)
        for v, tt in ((v_rand, t), (v_near, np.tile(t[:4000], len(v_near) // 4000))):
            agree, got, want = _bracket(v, tt, code)
            assert np.array_equal(got[agree], want[agree])


def test_bracket_margin_is_needed():
    """With no margin (both ends equal to x) the shortcut would be wrong
    somewhere near a boundary, so the test above can fail."""
    rng = np.random.default_rng(22)
    d = (10.0 ** rng.uniform(-3, 3, 4000)).astype(F)
    v = _near_boundaries(rng, [k + 0.5 for k in range(-8, 8)], d, 4000)
    dd = np.tile(d, len(v) // 4000)
    x = (v * (F(1.0) / dd)).astype(F)
    assert (int4_code(x) != int4_code((v / dd).astype(F))).any()
