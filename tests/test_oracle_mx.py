"""Pins for the oracle's MX activation quantizer (OCP MX: E8M0 scale per 32,
shared exponent floor(log2 max|x|) - emax, elements rounded to nearest with
ties to even and saturated) and the exact MX x MXFP4 product.

Page facts: "Why 4-Bit Quantization Is King", section 5 (an MXFP4 code of
value 3 under the group scale 2^-1 reconstructs 1.5; the OCP specification is
the contract); "Four Bits, Three Contracts", sections 1 and 3 (the E2M1 grid,
E8M0 = 2^(b-127))."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from exact import frac

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
E2M1 = json.load(open(os.path.join(GOLDEN, "e2m1_codebook.json")))["values"]


def test_e2m1_rne_facts():
    # midpoints of the E2M1 grid go to the code with an even last bit
    facts = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0,
             0.2: 0.0, 0.3: 0.5, 2.6: 3.0, 4.9: 4.0, 5.1: 6.0, 6.0: 6.0, 7.0: 6.0, 1e9: 6.0, 1e30: 6.0,
             3e38: 6.0}
    for v, want in facts.items():
        assert E2M1[oracle.e2m1_rne(v)] == want, v
        assert E2M1[oracle.e2m1_rne(-v)] == -want, -v
    assert oracle.e2m1_rne(-0.0) == 8 and oracle.e2m1_rne(0.0) == 0


def test_e2m1_rne_is_nearest():
    rng = np.random.default_rng(0)
    grid = np.array(E2M1[:8])
    for v in np.concatenate([rng.uniform(-7, 7, 3000), np.arange(-7, 7.01, 0.125)]):
        c = oracle.e2m1_rne(float(v))
        best = np.abs(np.abs(v) - grid).min()
        assert abs(abs(v) - abs(E2M1[c])) == best or abs(v) > 6
        assert (c >= 8) == bool(np.signbit(v))


def test_e4m3fn_rne_against_torch():
    rng = np.random.default_rng(1)
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    finite = np.sort(np.unique(np.abs(t[np.isfinite(t)])))
    mids = (finite[:-1] + finite[1:]) / 2  # exact ties, representable in binary32
    vals = np.concatenate([rng.uniform(-448, 448, 5000), rng.standard_normal(3000) * 0.01, mids, -mids,
                           finite, -finite]).astype(np.float32)
    want = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3fn_rne(float(v)) for v in vals], np.uint8)
    # torch keeps -0 for negative values that round to zero, as the oracle does
    assert np.array_equal(got, want)
    for v in (448.0, 449.0, 464.0, 1e6, 3e38):
        assert oracle.e4m3fn_rne(v) == 0x7E and oracle.e4m3fn_rne(-v) == 0xFE


def test_mx_scale_rule_and_page_fact():
    x = np.zeros((4, 64), np.float32)
    x[0, 0], x[0, 1] = 1.5, 3.0           # max 3: floor(log2 3) - 2 = -1, scale 2^-1
    x[1, :32] = 7.0 * 2.0 ** 5            # max 7 * 2^5: scale 2^5, 7 saturates to 6
    x[2, 40] = 2.0 ** -140                # far below the E8M0 range: scale byte 0
    x[3, :32] = 448.0                     # E2M1: 448 = 1.75 * 2^8 -> scale 2^6, 7 -> 6
    codes, scales = oracle.mx_quantize(x, oracle.MXFP4)
    assert scales[0, 0] == 126 and (codes[0, 0] & 15) == 5 and (codes[0, 0] >> 4) == 7
    assert E2M1[codes[0, 0] & 15] * 2.0 ** (int(scales[0, 0]) - 127) == 1.5  # code 3 at scale 2^-1 is 1.5
    assert scales[1, 0] == 127 + 5 and (codes[1, :16] == 0x77).all()
    assert scales[0, 1] == 0 and (codes[0, 16:] == 0).all()  # all-zero block
    assert scales[2, 1] == 0 and (codes[2, 20] >> 4) == 0      # 2^-140 / 2^-127 rounds to 0
    assert scales[3, 0] == 127 + 6 and (codes[3, :16] == 0x77).all()
    c8, s8 = oracle.mx_quantize(x, oracle.MXFP8)
    assert s8[3, 0] == 127 and (c8[3, :32] == 0x7E).all()       # E4M3: 448 exactly, scale 1
    assert s8[0, 0] == 127 + 1 - 8                               # floor(log2 3) - 8


@pytest.mark.parametrize("xfmt", ["mxfp4", "mxfp8"])
def test_mx_quantize_is_nearest_grid_point(xfmt):
    """Each element is the nearest point of the scaled element grid (brute
    force over every code), with the block's scale from the largest element."""
    rng = np.random.default_rng(2)
    m, k = 3, 128
    x = (rng.standard_normal((m, k)) * np.repeat(10.0 ** rng.uniform(-3, 3, (m, k // 32)), 32, axis=1))
    x = x.astype(np.float32)
    fmt = oracle.MXFP4 if xfmt == "mxfp4" else oracle.MXFP8
    codes, scales = oracle.mx_quantize(x, fmt)
    if xfmt == "mxfp4":
        vals = np.array(E2M1)
        emax = 2
        q = np.stack([codes & 15, codes >> 4], axis=2).reshape(m, k)
    else:
        vals = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        vals = np.where(np.isnan(vals), np.inf, vals)
        emax = 8
        q = codes
    for i in range(m):
        for b in range(k // 32):
            blk = x[i, 32 * b: 32 * b + 32].astype(np.float64)
            # the OCP shared scale puts the block's largest magnitude into the
            # element format's top binade [2^emax, 2^(emax+1)), checked in
            # exact rationals from the stored byte alone
            e = int(scales[i, b]) - 127
            top = Fraction(float(np.abs(blk).max())) / Fraction(2) ** e
            assert Fraction(2) ** emax <= top < Fraction(2) ** (emax + 1), (i, b, e)
            s = 2.0 ** e
            for j in range(32):
                got = vals[q[i, 32 * b + j]] * s
                assert abs(blk[j] - got) == np.abs(blk[j] - vals[np.isfinite(vals)] * s).min()


@pytest.mark.parametrize("xfmt", ["mxfp4", "mxfp8"])
def test_mx_gemm_entries_exact(xfmt):
    rng = np.random.default_rng(3)
    m, n, k = 3, 4, 96
    X = rng.standard_normal((m, k)).astype(np.float32)
    fmt = oracle.MXFP4 if xfmt == "mxfp4" else oracle.MXFP8
    xc, xs = oracle.mx_quantize(X, fmt)
    wc = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    ws = (127 + rng.integers(-3, 3, (n, k // 32))).astype(np.uint8)
    W = oracle.dequant_rows(oracle.MXFP4, wc, ws, 1.0, k, range(n))
    if xfmt == "mxfp4":
        Xh = oracle.dequant_rows(oracle.MXFP4, xc, xs, 1.0, k, range(m))
    else:
        f8 = torch.from_numpy(xc).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        Xh = f8 * np.repeat(2.0 ** (xs.astype(np.float64) - 127), 32, axis=1)
    ms, ns = np.meshgrid(np.arange(m), np.arange(n), indexing="ij")
    y, S = oracle.mx_gemm_entries(wc, ws, k, fmt, xc, xs, ms.ravel(), ns.ravel())
    for t, (i, j) in enumerate(zip(ms.ravel(), ns.ravel())):
        exact = sum(frac(Xh[i, e]) * frac(W[j, e]) for e in range(k))
        assert y[t] == float(exact)
        assert S[t] == float(sum(abs(frac(Xh[i, e]) * frac(W[j, e])) for e in range(k)))


@pytest.mark.parametrize("xfmt,emax", [("mxfp4", 2), ("mxfp8", 8)])
def test_mx_scale_at_the_ends_of_binary32(xfmt, emax):
    """Blocks whose top binade would need a scale below 2^-127 take byte 0
    (the clamp of the shared exponent); the largest binary32 block takes the
    byte that puts 2^127 into the top binade; an all-zero block takes byte 0."""
    fmt = oracle.MXFP4 if xfmt == "mxfp4" else oracle.MXFP8
    x = np.zeros((1, 96), np.float32)
    x[0, :32] = np.float32(2.0 ** -140) * np.arange(1, 33, dtype=np.float32) / 32   # binary32 subnormals
    x[0, 32:64] = np.float32(3.0e38) * np.linspace(-1, 1, 32, dtype=np.float32)
    codes, scales = oracle.mx_quantize(x, fmt)
    assert scales[0, 0] == 0
    top = Fraction(float(np.abs(x[0, 32:64]).max())) / Fraction(2) ** (int(scales[0, 1]) - 127)
    assert Fraction(2) ** emax <= top < Fraction(2) ** (emax + 1)
    assert scales[0, 2] == 0 and not codes[0, (64 if xfmt == "mxfp8" else 32):].any()
