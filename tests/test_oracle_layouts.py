"""Pins for the oracle's int4 layouts (GPTQ, AWQ, Q4_0), the generic b-bit
word stream, the signed INT4 toy and the affine dequantization."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads
from exact import round_f32, same_val, frac

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def brute_pack(vals, bits):
    """Independent bit-level statement of the word stream: one big integer
    whose bit i*b.. holds element i, cut into little-endian 32-bit words."""
    big = 0
    for i, v in enumerate(vals):
        big |= int(v) << (i * bits)
    nwords = (len(vals) * bits + 31) // 32
    return np.array([(big >> (32 * w)) & 0xFFFFFFFF for w in range(nwords)], np.uint32)


@pytest.mark.parametrize("bits", [2, 3, 4, 6, 8])
def test_bit_stream_vs_brute_force(bits):
    rng = np.random.default_rng(bits)
    for count in (32, 64, 96, 160):
        vals = rng.integers(0, 1 << bits, count).astype(np.uint32)
        words = oracle.pack_bits(vals, bits)
        assert np.array_equal(words, brute_pack(vals, bits))
        assert np.array_equal(oracle.unpack_bits(words, bits, count), vals)


def test_three_bit_straddles():
    g = golden("int4_layouts.json")["three_bit"]
    assert 32 * 3 == 3 * 32  # 32 values fill exactly three words
    for idx in g["straddle_indices"]:
        vals = np.zeros(32, np.uint32)
        vals[idx] = 7
        words = oracle.pack_bits(vals, 3)
        nonzero = [w for w in range(3) if words[w]]
        assert len(nonzero) == 2 and nonzero[1] == nonzero[0] + 1, idx
    straddlers = [i for i in range(32) if (i * 3) // 32 != (i * 3 + 2) // 32]
    assert straddlers == g["straddle_indices"]


def test_int4_toy():
    g = golden("int4_layouts.json")["int4_toy"]
    codes = [oracle.int4_sym_code(w, g["s"]) for w in g["w"]]
    assert codes == g["nibbles"]
    assert [oracle.int4_sym_value(c) for c in codes] == g["q"]
    packed = [codes[0] | (codes[1] << 4), codes[2] | (codes[3] << 4)]
    assert packed == g["bytes"]
    deq = [g["s"] * oracle.int4_sym_value(c) for c in codes]
    assert deq == g["dequant"]
    assert sum(a * b for a, b in zip(deq, g["x"])) == g["dot_recon"]
    assert sum(a * b for a, b in zip(g["w"], g["x"])) == g["dot_orig"]


def test_gptq_words():
    g = golden("int4_layouts.json")["gptq"]
    q = np.zeros((8, 3), np.uint8)
    q[:, 1] = np.arange(8)
    qw = oracle.gptq_pack(q)
    assert qw.shape == (1, 3)
    assert int(qw[0, 1]) == int(g["column_codes_0_to_7_word"], 16)
    assert int(qw[0, 0]) == 0 and int(qw[0, 2]) == 0
    # row 8r+j at bits 4j of word [r][n]
    rng = np.random.default_rng(1)
    q = rng.integers(0, 16, (64, 5)).astype(np.uint8)
    qw = oracle.gptq_pack(q)
    for r in range(8):
        for n in range(5):
            for j in range(8):
                assert (int(qw[r, n]) >> (4 * j)) & 15 == q[8 * r + j, n]


def test_awq_words_and_reader_shifts():
    g = golden("int4_layouts.json")["awq"]
    q = np.zeros((2, 16), np.uint8)
    q[1, 8:16] = np.arange(8)
    qw = oracle.awq_pack(q)
    assert qw.shape == (2, 2)
    assert int(qw[1, 1]) == int(g["row_codes_0_to_7_word"], 16)
    # the reader's view: column c of a group sits at shift reader_shifts[c]
    rng = np.random.default_rng(2)
    q = rng.integers(0, 16, (5, 64)).astype(np.uint8)
    qw = oracle.awq_pack(q)
    for kk in range(5):
        for n in range(64):
            sh = g["reader_shifts"][n % 8]
            assert (int(qw[kk, n // 8]) >> sh) & 15 == q[kk, n]
    # and the slot order is the inverse permutation of the shifts
    order = g["slot_order"]
    assert [order.index(c) * 4 for c in range(8)] == g["reader_shifts"]


def test_q4_0_byte_rule():
    K, N = 64, 3
    rng = np.random.default_rng(3)
    q = rng.integers(0, 16, (K, N)).astype(np.uint8)
    d = rng.integers(0, 2**16, (N, K // 32)).astype(np.uint16)
    blocks = oracle.q4_0_pack(q, d)
    for n in range(N):
        for b in range(K // 32):
            blk = blocks[n, b]
            assert int(blk[0]) | (int(blk[1]) << 8) == d[n, b]
            for j in range(16):
                assert blk[2 + j] & 15 == q[32 * b + j, n]
                assert blk[2 + j] >> 4 == q[32 * b + j + 16, n]


def test_verification_probes_round_trip():
    g = golden("int4_layouts.json")["probes"]
    K, N = g["K"], g["N"]
    for probe in workloads.layout_probes(K, N):
        assert np.array_equal(oracle.gptq_unpack(oracle.gptq_pack(probe)), probe)
        assert np.array_equal(oracle.awq_unpack(oracle.awq_pack(probe)), probe)
        d = np.arange(N * (K // 32), dtype=np.uint16).reshape(N, K // 32)
        q2, d2 = oracle.q4_0_unpack(oracle.q4_0_pack(probe, d), K, N)
        assert np.array_equal(q2, probe) and np.array_equal(d2, d)
    # all-15: the top slot's high bit is the int32 sign bit; unpacking a signed
    # view must still give 15 everywhere
    full = workloads.layout_probes(K, N)[2]
    qw = oracle.gptq_pack(full).view(np.int32)
    assert (qw == -1).all()
    assert np.array_equal(oracle.gptq_unpack(qw), full)
    assert np.array_equal(oracle.awq_unpack(oracle.awq_pack(full).view(np.int32)), full)


def test_wrong_axis_or_order_is_visible():
    # Failure modes: reading GPTQ along N, or ignoring AWQ's interleave, must
    # scramble the patterned probe.
    K, N = 64, 64
    pat = workloads.layout_probes(K, N)[0]
    awq = oracle.awq_pack(pat)
    plain = np.stack([oracle.pack_bits(pat[kk].reshape(-1), 4) for kk in range(K)])
    assert not np.array_equal(awq, plain)
    gptq = oracle.gptq_pack(pat)
    assert not np.array_equal(oracle.awq_unpack(gptq.reshape(K, N // 8)), pat)


def test_affine_dequant_and_cross_layout_identity():
    rng = np.random.default_rng(9)
    K, N, g = 128, 16, 64
    q = rng.integers(0, 16, (K, N)).astype(np.uint8)
    s = rng.uniform(-0.01, 0.01, (K // g, N)).astype(np.float16)
    z = rng.integers(0, 16, (K // g, N)).astype(np.uint8)
    z[0, :4] = 8  # make sure some groups carry Q4_0's fixed zero point
    w = oracle.affine_dequant(q, s.view(np.uint16), z, g)
    for kk in range(0, K, 3):
        for n in range(N):
            want = round_f32(frac(s[kk // g, n]) * (int(q[kk, n]) - int(z[kk // g, n])))
            assert same_val(w[kk, n], want)
    # the same logical matrix through GPTQ and AWQ dequantizes bit-identically
    wa = oracle.affine_dequant(oracle.gptq_unpack(oracle.gptq_pack(q)), s.view(np.uint16), z, g)
    wb = oracle.affine_dequant(oracle.awq_unpack(oracle.awq_pack(q)), s.view(np.uint16), z, g)
    assert np.array_equal(wa.view(np.uint32), wb.view(np.uint32))
    # Q4_0 with d = the group scale equals the affine rule wherever z = 8
    dq = np.repeat(s.view(np.uint16).T, g // 32, axis=1)  # [N][K/32]
    blocks = oracle.q4_0_pack(q, np.ascontiguousarray(dq))
    w40 = oracle.dequant_rows(oracle.Q4_0, blocks, None, 1.0, K, list(range(N))).T  # [K][N]
    z8 = np.repeat(z, g, axis=0) == 8
    assert z8.any()
    assert np.array_equal(w40[z8].view(np.uint32), w[z8].view(np.uint32))
    w_all8 = oracle.affine_dequant(q, s.view(np.uint16), np.full_like(z, 8), g)
    assert np.array_equal(np.ascontiguousarray(w40).view(np.uint32), w_all8.view(np.uint32))
