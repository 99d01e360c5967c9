"""Pins for the oracle's encode side: E2M1 rounding under both tie rules
("Four Bits, Three Contracts" section 2, the lowest unsigned code on an exact
tie; the Muser chapter section 7.2, ModelOpt's ties-to-even midpoints), the
NVFP4 quantizer (x = q * s_block * s_global, "Why 4-Bit Quantization Is
King" section 5), signed INT4 symmetric quantization (the same page's
section 1 example), and bit-plane splitting ("Bit Packing Architecture",
"Odd widths")."""
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
E2M1 = json.load(open(os.path.join(GOLDEN, "e2m1_codebook.json")))["values"]


def test_e2m1_tie_rules_at_every_midpoint():
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    even = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]     # the neighbour whose code is even
    lowest = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0]   # the lower code (smaller magnitude)
    for v, e, lo in zip(mids, even, lowest):
        assert E2M1[oracle.e2m1_round(v, oracle.TIE_EVEN)] == e
        assert E2M1[oracle.e2m1_round(v, oracle.TIE_LOWEST)] == lo
        assert E2M1[oracle.e2m1_round(-v, oracle.TIE_EVEN)] == -e
        assert E2M1[oracle.e2m1_round(-v, oracle.TIE_LOWEST)] == -lo
    # the page's ambiguous 1.25 row: 1.0 and 1.5 equally distant
    assert E2M1[oracle.e2m1_round(1.25, oracle.TIE_LOWEST)] == 1.0


@pytest.mark.parametrize("tie", [0, 1])
def test_e2m1_round_is_nearest(tie):
    rng = np.random.default_rng(tie)
    grid = np.array(E2M1[:8])
    for v in np.concatenate([rng.uniform(-8, 8, 3000), np.arange(-7, 7.01, 0.125)]):
        c = oracle.e2m1_round(float(v), tie)
        d = np.abs(min(abs(v), 6.0) - grid)
        assert abs(min(abs(v), 6.0) - abs(E2M1[c])) == d.min()
        assert (c >= 8) == bool(np.signbit(v))


def test_nvfp4_quantize_page_example():
    # global scale 2 and a block maximum of 6: block scale 6 / (6 * 2) = 0.5;
    # x = 3 becomes code 3.0, reconstructing 3 * 0.5 * 2 = 3
    x = np.zeros((1, 16), np.float32)
    x[0, 0], x[0, 1] = 6.0, 3.0
    codes, scales = oracle.nvfp4_quantize(x, 2.0, oracle.TIE_EVEN)
    assert oracle.e4m3fn(int(scales[0, 0])) == 0.5
    assert E2M1[codes[0, 0] >> 4] == 3.0 and E2M1[codes[0, 0] & 15] == 6.0


@pytest.mark.parametrize("tie", [0, 1])
def test_nvfp4_quantize_brute_force(tie):
    rng = np.random.default_rng(5 + tie)
    m, k, scale2 = 4, 64, np.float32(0.01)
    X = (rng.standard_normal((m, k)) * np.repeat(10.0 ** rng.uniform(-2, 1, (m, k // 16)), 16, axis=1))
    X = X.astype(np.float32)
    X[1, 16:32] = 0.0
    codes, scales = oracle.nvfp4_quantize(X, float(scale2), tie)
    grid = np.array(E2M1[:8])
    for i in range(m):
        for b in range(k // 16):
            blk = X[i, 16 * b:16 * b + 16]
            q = np.float32(np.abs(blk).max()) / np.float32(6 * scale2)
            want = torch.tensor([float(q)], dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).item()
            assert scales[i, b] == want
            t = np.float32(np.float32(oracle.e4m3fn(int(want))) * scale2)
            for j in range(16):
                c = (codes[i, 8 * b + j // 2] >> (4 * (j % 2))) & 15
                if t == 0:
                    assert c == 0
                    continue
                v = float(np.float32(blk[j] / t))
                d = np.abs(min(abs(v), 6.0) - grid)
                assert abs(min(abs(v), 6.0) - abs(E2M1[c])) == d.min()


def test_int4_sym_page_example():
    # w = [-1, 0.25, 0.875, 1.75]: s = 1.75 / 7 = 0.25, q = [-4, 1, 4, 7],
    # nibbles C, 1, 4, 7, bytes 0x1C and 0x74 (earlier code in the low nibble)
    codes, scales = oracle.int4_sym_quantize(np.array([[-1.0, 0.25, 0.875, 1.75]], np.float32), 4)
    assert scales[0, 0] == 0.25
    assert list(codes[0]) == [0x1C, 0x74]


def test_int4_sym_brute_force():
    rng = np.random.default_rng(6)
    m, k, g = 3, 96, 32
    W = rng.standard_normal((m, k)).astype(np.float32)
    W[2, 32:64] = 0.0
    codes, scales = oracle.int4_sym_quantize(W, g)
    for i in range(m):
        for kk in range(k):
            s = scales[i, kk // g]
            assert s == np.float32(np.abs(W[i, (kk // g) * g:(kk // g + 1) * g]).max()) / np.float32(7)
            nib = int((codes[i, kk // 2] >> (4 * (kk % 2))) & 15)
            q = nib - 16 if nib >= 8 else nib
            if s == 0:
                assert q == 0
                continue
            r = float(np.float32(W[i, kk] / s))
            cands = np.arange(-8, 8)
            best = np.abs(cands - r).min()
            assert abs(q - r) == best and (abs(q - r) < 0.5 or q % 2 == 0)


def test_int4_sym_ties_round_half_to_even():
    """Exact ties: with max |w| = 7 the scale is exactly 1, so w / s = w.
    Round half to even sends 2.5 -> 2, -2.5 -> -2, 0.5 -> 0, -0.5 -> 0,
    3.5 -> 4, 1.5 -> 2, -6.5 -> -6 (written out by hand)."""
    w = np.array([[7.0, 2.5, -2.5, 0.5, -0.5, 3.5, 1.5, -6.5]], np.float32)
    codes, scales = oracle.int4_sym_quantize(w, 8)
    assert scales[0, 0] == 1.0
    want = [7, 2, -2, 0, 0, 4, 2, -6]
    got = [int((codes[0, i // 2] >> (4 * (i % 2))) & 15) for i in range(8)]
    assert [q - 16 if q >= 8 else q for q in got] == want


def test_bit_planes_split_6_bit():
    rng = np.random.default_rng(7)
    v = rng.integers(0, 64, 96).astype(np.uint32)
    lo_w, hi_w = oracle.pack_planes(v, 6, 4)
    assert lo_w.size == 96 * 4 // 32 and hi_w.size == 96 * 2 // 32
    assert np.array_equal(oracle.unpack_bits(lo_w, 4, 96), v & 15)
    assert np.array_equal(oracle.unpack_bits(hi_w, 2, 96), v >> 4)
    assert np.array_equal(oracle.unpack_planes(lo_w, hi_w, 96, 6, 4), v)
    # no value straddles a word in either plane, unlike the 6-bit sequential stream
    assert any((i * 6) // 32 != (i * 6 + 5) // 32 for i in range(96))
