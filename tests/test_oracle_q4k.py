"""Pins for the oracle's Q4_K and Q4_0 block decoders."""
import json
import os
from fractions import Fraction

import numpy as np

import oracle
from exact import round_f32, same_f32, same_val, frac

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def f16_bits(v) -> int:
    return int(np.array([v], np.float16).view(np.uint16)[0])


def make_block(d, dmin, s, m, qs):
    blk = np.zeros(144, np.uint8)
    blk[0:2] = np.array([d], np.float16).view(np.uint8)
    blk[2:4] = np.array([dmin], np.float16).view(np.uint8)
    blk[4:16] = oracle.q4k_pack_scales(s, m)
    blk[16:144] = np.asarray(qs, np.uint8)
    return blk


def test_q4k_block_size_facts():
    g = golden("q4k_fixture.json")["block_bytes"]
    assert 128 + 4 + 12 == g["total"]
    assert g["total"] * 8 / g["weights"] == g["bpw"]


def test_q4k_lanes_0_and_32_fixture():
    g = golden("q4k_fixture.json")["lanes"]
    s = [g["pairs"][0][0], g["pairs"][1][0]] + [0] * 6
    m = [g["pairs"][0][1], g["pairs"][1][1]] + [0] * 6
    for key in ("byte_a5", "byte_00", "byte_ff_derived"):
        qs = np.zeros(128, np.uint8)
        qs[0] = g[key]["byte"]
        blk = make_block(g["d"], g["dmin"], s, m, qs)
        row = oracle.dequant_rows(oracle.Q4_K, blk[None, None, :], None, 1.0, 256, [0])[0]
        assert row[0] == g[key]["lane0"], key
        assert row[32] == g[key]["lane32"], key


def test_q4k_metadata_fact_and_bijection():
    g = golden("q4k_fixture.json")["metadata"]
    B = np.zeros(12, np.uint8)
    B[0] = g["B0"]
    B[8] = g["B8"]
    s, m = oracle.q4k_unpack_scales(B)
    assert s[4] == g["s4"]
    # reading B[4] as the scale of pair 4 would give a different number
    assert s[4] != B[4]
    # 96 bits <-> sixteen 6-bit fields: both directions are bijective
    rng = np.random.default_rng(11)
    for _ in range(2000):
        B = rng.integers(0, 256, 12).astype(np.uint8)
        s, m = oracle.q4k_unpack_scales(B)
        assert all(0 <= v < 64 for v in s + m)
        assert np.array_equal(oracle.q4k_pack_scales(s, m), B)
    for _ in range(2000):
        s = rng.integers(0, 64, 8).tolist()
        m = rng.integers(0, 64, 8).tolist()
        assert oracle.q4k_unpack_scales(oracle.q4k_pack_scales(s, m)) == (s, m)
    # each single bit of the 12 bytes moves exactly one field by a power of two
    seen = set()
    for byte in range(12):
        for bit in range(8):
            B = np.zeros(12, np.uint8)
            B[byte] = 1 << bit
            s, m = oracle.q4k_unpack_scales(B)
            nz = [(("s", j), v) for j, v in enumerate(s) if v] + [(("m", j), v) for j, v in enumerate(m) if v]
            assert len(nz) == 1 and (nz[0][1] & (nz[0][1] - 1)) == 0
            key = (nz[0][0], nz[0][1])
            assert key not in seen
            seen.add(key)
    assert len(seen) == 96


def test_q4k_all_256_destinations_asymmetric():
    # Distinct (scale, min) per sub-block and distinct nibbles per byte: every
    # output must come from the page's lane map (Four Bits, Three Contracts,
    # section 5): byte 32c+l low nibble -> output 64c+l (sub-block 2c), high
    # nibble -> output 64c+32+l (sub-block 2c+1).
    d, dmin = np.float16(0.0078125), np.float16(0.001953125)
    s = [5, 63, 17, 40, 33, 1, 58, 22]
    m = [9, 2, 61, 30, 47, 12, 0, 55]
    qs = np.array([((3 * i + 1) & 15) | (((7 * i + 5) & 15) << 4) for i in range(128)], np.uint8)
    blk = make_block(d, dmin, s, m, qs)
    row = oracle.dequant_rows(oracle.Q4_K, blk[None, None, :], None, 1.0, 256, [0])[0]
    for out in range(256):
        c, rest = divmod(out, 64)
        half, l = divmod(rest, 32)
        byte = int(qs[32 * c + l])
        q = (byte >> 4) if half else (byte & 15)
        j = 2 * c + half
        want = round_f32(frac(d) * s[j] * q - frac(dmin) * m[j])
        assert same_val(row[out], want), out


def test_q4k_exact_single_rounding_random():
    # w = RN_f32(d*s*q - dmin*m) against exact rationals, random blocks with
    # d and dmin spread over many binades (includes fp16 subnormals)
    rng = np.random.default_rng(5)
    nb = 24
    blocks = np.zeros((1, nb, 144), np.uint8)
    for b in range(nb):
        d = np.float16(rng.uniform(-1, 1) * 2.0 ** rng.integers(-24, 12))
        dmin = np.float16(rng.uniform(-1, 1) * 2.0 ** rng.integers(-24, 12))
        s = rng.integers(0, 64, 8).tolist()
        m = rng.integers(0, 64, 8).tolist()
        blocks[0, b] = make_block(d, dmin, s, m, rng.integers(0, 256, 128))
    row = oracle.dequant_rows(oracle.Q4_K, blocks, None, 1.0, 256 * nb, [0])[0]
    for b in range(nb):
        blk = blocks[0, b]
        d = frac(blk[0:2].view(np.float16)[0])
        dmin = frac(blk[2:4].view(np.float16)[0])
        s, m = oracle.q4k_unpack_scales(blk[4:16])
        for out in range(0, 256, 7):
            c, rest = divmod(out, 64)
            half, l = divmod(rest, 32)
            byte = int(blk[16 + 32 * c + l])
            q = (byte >> 4) if half else (byte & 15)
            j = 2 * c + half
            exact = d * s[j] * q - dmin * m[j]
            assert same_val(row[256 * b + out], round_f32(exact)), (b, out)


def test_q4k_toy_subblock_and_w4a8_identity():
    g = golden("q4k_fixture.json")["toy_subblock"]
    s = [0] * 8
    m = [0] * 8
    s[0], m[0] = g["s"], g["m"]
    qs = np.zeros(128, np.uint8)
    qs[0:3] = g["codes"]
    blk = make_block(g["d"], g["dmin"], s, m, qs)
    row = oracle.dequant_rows(oracle.Q4_K, blk[None, None, :], None, 1.0, 256, [0])[0]
    d = frac(np.float16(g["d"]))
    dmin = frac(np.float16(g["dmin"]))
    for i, q in enumerate(g["codes"]):
        exact = d * g["s"] * q - dmin * g["m"]
        assert same_val(row[i], round_f32(exact))
        # the page's decimal values hold to fp16 precision of d and dmin
        assert abs(float(row[i]) - g["recon_exact"][i]) < 1e-3
    # exact-arithmetic identity of the page's W4A8 example
    step, off = Fraction(3, 10), Fraction(1, 10)
    qx = g["w4a8"]["q_x"]
    sx = Fraction(g["w4a8"]["s_x"])
    idot = sum(a * b for a, b in zip(g["codes"], qx))
    csum = sum(qx)
    assert idot == g["w4a8"]["int_dot"] and csum == g["w4a8"]["code_sum"]
    assert sx * step * idot - sx * off * csum == Fraction(3, 10)
    assert sum((step * q - off) * Fraction(x) for q, x in zip(g["codes"], g["x"])) == Fraction(3, 10)
    # and the oracle's dot on the fp16-rounded block is close to 0.30
    x = np.zeros(256, np.float32)
    x[0:3] = g["x"]
    y, S = oracle.gemv_rows(oracle.Q4_K, blk[None, None, :], None, 1.0, 256, x, [0])
    assert abs(y[0] - g["dot_exact"]) < 1e-3


def test_q4_0_block_decode():
    g = golden("int4_layouts.json")["q4_0"]
    rng = np.random.default_rng(2)
    nb = 6
    blocks = np.zeros((2, nb, 18), np.uint8)
    for r in range(2):
        for b in range(nb):
            blocks[r, b, 0:2] = np.array([rng.uniform(-2, 2)], np.float16).view(np.uint8)
            blocks[r, b, 2:18] = rng.integers(0, 256, 16)
    out = oracle.dequant_rows(oracle.Q4_0, blocks, None, 1.0, 32 * nb, [1, 0])
    for oi, r in enumerate([1, 0]):
        for b in range(nb):
            d = frac(blocks[r, b, 0:2].view(np.float16)[0])
            for j in range(16):
                byte = int(blocks[r, b, 2 + j])
                assert same_val(out[oi, 32 * b + j], round_f32(d * ((byte & 15) - g["offset"])))
                assert same_val(out[oi, 32 * b + j + 16], round_f32(d * ((byte >> 4) - g["offset"])))
    assert g["block_bytes"] * 8 / g["weights"] == 4.5
