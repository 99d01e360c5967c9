"""Pins for the oracle's dot products (GEMV rows and sampled GEMM entries):
brute force in exact rational arithmetic on small cases, and the dyadic case
where every partial sum is exact."""
from fractions import Fraction

import numpy as np

import oracle
import workloads
from exact import frac


def _exact_dot(wrow, x):
    return sum(frac(a) * frac(b) for a, b in zip(wrow, x))


def test_gemv_rows_vs_exact_rationals_all_formats():
    for c, (n, k) in ((1, (5, 64)), (2, (4, 48)), (3, (3, 512))):
        inp = workloads.workload(c, n=n, k=k, seed=77 + c)
        fmt = {"mxfp4": oracle.MXFP4, "nvfp4": oracle.NVFP4, "q4_k": oracle.Q4_K}[inp["fmt"]]
        rows = list(range(n))[::-1]
        W = oracle.dequant_rows(fmt, inp["data"], inp["scales"], inp["scale2"], k, rows)
        xv = (np.array([oracle.bf16_value(int(b)) for b in inp["x"]]) if inp["x"].dtype == np.uint16
              else inp["x"].astype(np.float64))
        y, S = oracle.gemv_rows(fmt, inp["data"], inp["scales"], inp["scale2"], k, inp["x"], rows)
        for i in range(n):
            exact = _exact_dot(W[i], xv)
            assert abs(Fraction(y[i]) - exact) <= Fraction(1, 2**52) * abs(exact) + Fraction(1, 2**100)
            s_exact = sum(abs(frac(a) * frac(b)) for a, b in zip(W[i], xv))
            assert abs(Fraction(S[i]) - s_exact) <= Fraction(k, 2**52) * s_exact


def test_dyadic_dot_is_exact():
    # small-integer activations times MXFP4 weights at scales >= 2^-4: every
    # partial sum is exactly representable, so the dot has one right answer
    rng = np.random.default_rng(4)
    n, k = 4, 256
    codes = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    scales = (127 + rng.integers(-4, 3, (n, k // 32))).astype(np.uint8)
    x = rng.integers(-8, 9, k).astype(np.float32)
    y, _ = oracle.gemv_rows(oracle.MXFP4, codes, scales, 1.0, k, x, range(n))
    W = oracle.dequant_rows(oracle.MXFP4, codes, scales, 1.0, k, range(n))
    for i in range(n):
        assert Fraction(y[i]) == _exact_dot(W[i], x)


def test_gemm_entries_match_gemv_rows():
    inp = workloads.workload(4, n=16, k=128, m=6, seed=5)
    ms = [0, 5, 3, 3, 1]
    ns = [15, 0, 7, 8, 7]
    Y, S = oracle.gemm_entries(oracle.MXFP4, inp["data"], inp["scales"], 1.0, 128, inp["X"], ms, ns)
    W = oracle.dequant_rows(oracle.MXFP4, inp["data"], inp["scales"], 1.0, 128, range(16))
    for i, (m, n) in enumerate(zip(ms, ns)):
        xv = [oracle.bf16_value(int(b)) for b in inp["X"][m]]
        exact = _exact_dot(W[n], xv)
        assert abs(Fraction(Y[i]) - exact) <= Fraction(1, 2**52) * abs(exact) + Fraction(1, 2**100)


def test_bf16_activation_decoding_in_dots():
    # a bf16 activation vector decodes to the upper half of a binary32
    x = np.array([0x3F80, 0xBF80, 0x4000, 0x0001, 0x8000, 0x3E80] + [0] * 26, np.uint16)
    vals = [oracle.bf16_value(int(b)) for b in x[:6]]
    assert vals[:3] == [1.0, -1.0, 2.0]
    assert vals[3] == 2.0 ** -133 and vals[4] == 0.0 and vals[5] == 0.25
    codes = np.full((1, 16), 0x22, np.uint8)  # all 1.0
    y, S = oracle.gemv_rows(oracle.MXFP4, codes, np.array([[127]], np.uint8), 1.0, 32, x, [0])
    assert y[0] == 1.0 - 1.0 + 2.0 + 2.0 ** -133 + 0.25


def test_compensated_sum_survives_cancellation():
    # x = [2^60, 1, -2^60, ...] with unit weights: a plain binary64 running sum
    # loses the 1; the oracle's compensated sum must return exactly 1.
    codes = np.full((1, 16), 0x44, np.uint8)  # code 4 -> 2.0, at scale 2^-1 -> 1.0
    x = np.zeros(32, np.float32)
    x[0], x[1], x[2] = 2.0 ** 60, 1.0, -(2.0 ** 60)
    y, S = oracle.gemv_rows(oracle.MXFP4, codes, np.array([[126]], np.uint8), 1.0, 32, x, [0])
    assert y[0] == 1.0
    assert S[0] == 2.0 ** 61 + 1.0


def test_rows_with_weights_beyond_binary32_follow_ieee_sums():
    """MXFP4 scale byte 254 with E2M1 codes >= 2 decodes beyond binary32 to
    +-inf (IEEE overflow, no saturation). The dot of such a row is then fixed
    by IEEE addition alone: infinities of one sign with finite terms give that
    infinity, infinities of both signs give NaN. A compensated sum must not
    turn the first case into NaN through its inf - inf correction term."""
    k = 64
    x = np.linspace(0.5, 1.5, k).astype(np.float32)
    nib = np.zeros((4, k), np.uint8)
    nib[0, :] = 7                 # +6 everywhere: every weight +inf
    nib[1, :] = 15                # -6 everywhere: every weight -inf
    nib[2, :] = 2                 # +1: finite, 2^127 each
    nib[3, :] = 2
    nib[3, 5], nib[3, 40] = 7, 15  # one +inf and one -inf weight
    nib[2, 33] = 7                # one +inf weight among finite ones
    codes = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    scales = np.full((4, k // 32), 254, np.uint8)
    W = oracle.dequant_rows(oracle.MXFP4, codes, scales, 1.0, k, range(4))
    assert np.isposinf(W[0]).all() and np.isneginf(W[1]).all()
    y, S = oracle.gemv_rows(oracle.MXFP4, codes, scales, 1.0, k, x, range(4))
    assert y[0] == np.inf and y[1] == -np.inf and y[2] == np.inf and np.isnan(y[3])
    assert np.isposinf(S).all()
    Xb = workloads.bf16_bits_from_f32(np.tile(x, (2, 1)))
    Y, _ = oracle.gemm_entries(oracle.MXFP4, codes, scales, 1.0, k, Xb, [0, 1, 1, 0], [0, 1, 2, 3])
    assert Y[0] == np.inf and Y[1] == -np.inf and Y[2] == np.inf and np.isnan(Y[3])
