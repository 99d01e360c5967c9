"""Pins for the oracle's integer-exact NVFP4 x Q8_K decode ("Chapter 7 -
NVFP4: the native lane", section 7.4.2): the Q1 / Q9 integer decoders, the
binary16 output rounding, the exact integer block totals, and the four pinned
binary32 steps with their block order."""
import json
import os
from fractions import Fraction

import numpy as np
import torch

import oracle
import workloads
from exact import frac

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_q1_is_twice_the_codebook():
    book = json.load(open(os.path.join(GOLDEN, "e2m1_codebook.json")))["values"]
    for c in range(16):
        assert oracle.e2m1_q1(c) == 2 * book[c]
    assert sorted({abs(oracle.e2m1_q1(c)) for c in range(16)}) == [0, 1, 2, 3, 4, 6, 8, 12]


def test_q9_exhaustive_against_torch_float8():
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for b in range(256):
        if np.isnan(t[b]):
            assert b in (0x7F, 0xFF) and oracle.e4m3fn_q9(b) == 0
            continue
        v = Fraction(float(t[b])) * 512
        assert v.denominator == 1, b  # every finite E4M3FN value is a multiple of 2^-9
        assert oracle.e4m3fn_q9(b) == v.numerator
    assert oracle.e4m3fn_q9(0x7E) == 448 * 512 and oracle.e4m3fn_q9(0x01) == 1


def test_f16_rne_matches_numpy():
    rng = np.random.default_rng(0)
    f16 = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = ((f16[:-1] + f16[1:]) / 2).astype(np.float32)  # exact ties (representable in binary32)
    vals = np.concatenate([
        rng.standard_normal(4000).astype(np.float32) * np.float32(10) ** rng.integers(-9, 6, 4000),
        mids[rng.integers(0, mids.size, 3000)], -mids[rng.integers(0, mids.size, 500)],
        np.array([0.0, -0.0, 65504, 65519.99, 65520, 65536, 1e6, -1e6, np.inf, -np.inf, 2.0 ** -24,
                  2.0 ** -25, 2.0 ** -25 * 1.0000001, 2.0 ** -14, 2.0 ** -14 * (1 - 2.0 ** -11)], np.float32),
    ]).astype(np.float32)
    with np.errstate(over="ignore"):
        want = vals.astype(np.float16).view(np.uint16)
    assert np.array_equal(oracle.f16_rne(vals), want)
    assert oracle.f16_rne(np.array([np.nan], np.float32))[0] & 0x7FFF > 0x7C00


def _nvfp4(rng, n, k):
    codes, scales = workloads.nvfp4_weights(rng, n, k)
    return codes, scales


def test_block_totals_are_exact_integers_and_result_within_four_roundings():
    """The block total is 1024 * sum(w * q) with w = e2m1 * e4m3 taken exactly
    (the binary32 dequantization with scale2 = 1 is exact); the result is the
    exact sum of total * 2^-10 * d * scale2 up to the rounding of the four
    binary32 steps, and its binary16 bits are numpy's rounding of it."""
    rng = np.random.default_rng(1)
    n, k = 6, 1024
    codes, scales = _nvfp4(rng, n, k)
    x = workloads.x_f32(rng, k)
    q, d, _ = oracle.q8_quantize(x)
    scale2 = float(np.float32(0.01))
    y32, y16 = oracle.nvfp4_a16q8_rows(codes, scales, scale2, k, q, d, range(n))
    W = oracle.dequant_rows(oracle.NVFP4, codes, scales, 1.0, k, range(n))
    for r in range(n):
        exact = Fraction(0)
        bound = Fraction(0)
        for b in range(k // 256):
            tot = sum(frac(W[r, i]) * int(q[i]) for i in range(256 * b, 256 * b + 256)) * 1024
            assert tot.denominator == 1
            term = tot * Fraction(1, 1024) * frac(d[b]) * frac(np.float32(scale2))
            exact += term
            bound += abs(term)
        err = abs(frac(y32[r]) - exact)
        assert err <= (k // 256 + 3) * Fraction(1, 2 ** 24) * bound + Fraction(1, 2 ** 140)
    assert np.array_equal(y16, y32.astype(np.float16).view(np.uint16))


def _one_weight_block(codes, scales, x, b, code, scale_byte, xval, scale_of_block):
    """Block b of row 0 holds a single nonzero weight (element 256b) and its
    activations quantize with inverse scale 1 / scale_of_block: element
    256b + 255 is -127 * scale_of_block (weight 0), element 256b is xval."""
    codes[0, 128 * b] = code
    scales[0, 16 * b] = scale_byte
    x[256 * b + 255] = -127.0 * scale_of_block
    x[256 * b] = xval


def test_exact_case_and_ascending_block_order():
    """Block totals 1024, 1, 1 with activation scales 1, 2^-14, 2^-14 and
    scale2 = 1 give contributions 1, 2^-24, 2^-24. Added in ascending block
    order each 2^-24 is a tie that rounds back to 1 (nearest even), so the
    result is exactly 1; any other order would give 1 + 2^-23."""
    k = 768
    codes = np.zeros((1, k // 2), np.uint8)
    scales = np.zeros((1, k // 16), np.uint8)
    x = np.zeros(k, np.float32)
    # Q1(code 6) = 8, Q9(0x28 = 0.25) = 128, q = 1: total 1024
    _one_weight_block(codes, scales, x, 0, 6, 0x28, 1.0, 1.0)
    # Q1(code 1) = 1, Q9(0x01 = 2^-9) = 1, q = 1: total 1
    _one_weight_block(codes, scales, x, 1, 1, 0x01, 2.0 ** -14, 2.0 ** -14)
    _one_weight_block(codes, scales, x, 2, 1, 0x01, 2.0 ** -14, 2.0 ** -14)
    q, d, _ = oracle.q8_quantize(x)
    assert list(d) == [1.0, 2.0 ** -14, 2.0 ** -14] and q[0] == 1 and q[256] == 1 and q[512] == 1
    y32, y16 = oracle.nvfp4_a16q8_rows(codes, scales, 1.0, k, q, d, [0])
    assert y32[0] == 1.0 and y16[0] == 0x3C00
    # the same contributions in the other order do not round away
    assert np.float32(np.float32(2.0 ** -24) + np.float32(2.0 ** -24)) + np.float32(1.0) != np.float32(1.0)


def test_exact_dyadic_rows():
    """Small power-of-two scales keep every step exact: the result is then the
    exact real sum of w * d * q * scale2."""
    rng = np.random.default_rng(4)
    n, k = 3, 512
    codes = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    scales = rng.choice(np.array([0x30, 0x38, 0x40], np.uint8), (n, k // 16))  # 0.5, 1, 2
    x = np.zeros(k, np.float32)
    x[:] = rng.integers(-20, 21, k).astype(np.float32)
    x[0] = -127.0
    x[256] = -127.0 * 0.5
    q, d, _ = oracle.q8_quantize(x)
    assert list(d) == [1.0, 0.5]
    y32, _ = oracle.nvfp4_a16q8_rows(codes, scales, 0.25, k, q, d, range(n))
    W = oracle.dequant_rows(oracle.NVFP4, codes, scales, 1.0, k, range(n))
    for r in range(n):
        exact = sum(frac(W[r, i]) * int(q[i]) * frac(d[i // 256]) for i in range(k)) * Fraction(1, 4)
        assert frac(y32[r]) == exact
