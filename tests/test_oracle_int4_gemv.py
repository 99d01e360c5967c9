"""Pins for the oracle's GEMV over the int4 layouts (GPTQ, AWQ: the K x N
logical matrix, w = s * (q - z); Q4_0: rows of 18-byte blocks, w = d * (q - 8);
"Bit Packing Architecture", "Real layouts compared"): brute force in exact
rational arithmetic, unit activations that read single weights back, the same
logical matrix through both packed layouts, and a zero-point case with a
closed form."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads
from exact import frac


def _exact_col(W, x, c):
    return sum(frac(W[k, c]) * frac(x[k]) for k in range(W.shape[0]))


def _xvals(x):
    return (np.array([oracle.bf16_value(int(b)) for b in x]) if x.dtype == np.uint16 else x.astype(np.float64))


@pytest.mark.parametrize("xdt", ["f32", "bf16"])
def test_gemv_kn_vs_exact_rationals(xdt):
    rng = np.random.default_rng(11)
    K, N = 96, 7
    W = (rng.standard_normal((K, N)) * 10.0 ** rng.uniform(-3, 3, (K, N))).astype(np.float32)
    x32 = rng.standard_normal(K).astype(np.float32)
    x = x32 if xdt == "f32" else workloads.bf16_bits_from_f32(x32)
    cols = [6, 0, 3, 3]
    y, S = oracle.gemv_kn(W, x, cols)
    xv = _xvals(x)
    for i, c in enumerate(cols):
        exact = _exact_col(W, xv, c)
        assert abs(Fraction(y[i]) - exact) <= Fraction(1, 2**52) * abs(exact) + Fraction(1, 2**100)
        s_exact = sum(abs(frac(W[k, c]) * frac(xv[k])) for k in range(K))
        assert abs(Fraction(S[i]) - s_exact) <= Fraction(K, 2**52) * s_exact


@pytest.mark.parametrize("fmt", ["gptq4", "awq4"])
def test_int4_gemv_vs_exact_rationals(fmt):
    inp = workloads.workload(7, n=16, k=256, seed=21)
    K, N, g = inp["K"], inp["N"], inp["group"]
    data = inp["gptq"] if fmt == "gptq4" else inp["awq"]
    q = oracle.gptq_unpack(data) if fmt == "gptq4" else oracle.awq_unpack(data)
    W = oracle.affine_dequant(q, inp["scales"].view(np.uint16), inp["zeros"], g)
    cols = list(range(N))[::-1]
    y, S = oracle.int4_gemv(fmt, data, inp["scales"], inp["zeros"], g, inp["x"], cols)
    for i, c in enumerate(cols):
        exact = _exact_col(W, inp["x"], c)
        assert abs(Fraction(y[i]) - exact) <= Fraction(1, 2**52) * abs(exact) + Fraction(1, 2**100)


def test_int4_unit_activation_reads_weights():
    inp = workloads.workload(7, n=24, k=128, seed=3)
    K, N, g = inp["K"], inp["N"], inp["group"]
    q = oracle.gptq_unpack(inp["gptq"])
    W = oracle.affine_dequant(q, inp["scales"].view(np.uint16), inp["zeros"], g)
    for kk in (0, 7, 8, 127):
        x = np.zeros(K, np.float32)
        x[kk] = 1.0
        y, S = oracle.int4_gemv("gptq4", inp["gptq"], inp["scales"], inp["zeros"], g, x, range(N))
        assert np.array_equal(y, W[kk].astype(np.float64))
        assert np.array_equal(S, np.abs(W[kk]).astype(np.float64))


def test_int4_same_matrix_both_layouts():
    """One logical matrix packed as GPTQ and as AWQ gives the same outputs."""
    rng = np.random.default_rng(5)
    K, N, g = 256, 32, 64
    q = rng.integers(0, 16, (K, N)).astype(np.uint8)
    s = rng.uniform(1e-3, 1e-2, (K // g, N)).astype(np.float16)
    z = rng.integers(0, 16, (K // g, N)).astype(np.uint8)
    x = rng.standard_normal(K).astype(np.float32)
    ya, Sa = oracle.int4_gemv("gptq4", oracle.gptq_pack(q), s, z, g, x, range(N))
    yb, Sb = oracle.int4_gemv("awq4", oracle.awq_pack(q), s, z, g, x, range(N))
    assert np.array_equal(ya, yb) and np.array_equal(Sa, Sb)


def test_int4_codes_at_the_zero_point_give_zero():
    """q == z everywhere: every weight is 0, so y = 0 and S = 0; q = z + 1 in
    one group gives s * sum of that group's x."""
    rng = np.random.default_rng(8)
    K, N, g = 128, 8, 32
    z = rng.integers(0, 15, (K // g, N)).astype(np.uint8)
    q = np.repeat(z, g, axis=0)
    s = np.full((K // g, N), 0.5, np.float16)
    x = rng.integers(-8, 9, K).astype(np.float32)
    y, S = oracle.int4_gemv("gptq4", oracle.gptq_pack(q), s, z, g, x, range(N))
    assert (y == 0).all() and (S == 0).all()
    q2 = q.copy()
    q2[g:2 * g] += 1
    y2, _ = oracle.int4_gemv("gptq4", oracle.gptq_pack(q2), s, z, g, x, range(N))
    assert np.array_equal(y2, np.full(N, 0.5 * float(x[g:2 * g].sum())))


def test_q4_0_gemv_vs_exact_rationals():
    inp = workloads.workload(7, n=9, k=160, seed=2)
    K, N = inp["K"], inp["N"]
    blocks = inp["q4_0"]
    W = oracle.dequant_rows(oracle.Q4_0, blocks, None, 1.0, K, range(N))
    y, S = oracle.gemv_rows(oracle.Q4_0, blocks, None, 1.0, K, inp["x"], range(N))
    for n in range(N):
        exact = sum(frac(W[n, k]) * frac(inp["x"][k]) for k in range(K))
        assert abs(Fraction(y[n]) - exact) <= Fraction(1, 2**52) * abs(exact) + Fraction(1, 2**100)
