"""Pins for the oracle's W4A8 path: int8 activation quantization and the
Q4_K x int8 dot ("Why 4-Bit Quantization Is King", section 7 and its worked
W4A8 example; section 7b step 4; section 7c).

The activation quantizer is the Q8_K rule of "Chapter 7 - NVFP4: the native
lane", section 7.4.2: per 256 activations, the first element of largest
magnitude mx (signed), iscale = RN32(-127 / mx), codes RNE(RN32(x * iscale))
clamped at 127, scale d = RN32(1 / iscale).
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from exact import frac
from test_oracle_q4k import make_block

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def pack_codes(codes):
    """128 code bytes from 256 logical codes: byte 32c+l holds element 64c+l
    in its low nibble and 64c+32+l in its high nibble (the lane map pinned by
    the Q4_K fixture)."""
    codes = np.asarray(codes, np.uint8)
    qs = np.zeros(128, np.uint8)
    for c in range(4):
        for l in range(32):
            qs[32 * c + l] = codes[64 * c + l] | (codes[64 * c + 32 + l] << 4)
    return qs


def random_row(rng, nb, d_choices=None, dmin_choices=None):
    """One Q4_K row of nb blocks plus its logical parameters."""
    blocks, params = [], []
    for _ in range(nb):
        d = rng.choice(d_choices) if d_choices is not None else rng.uniform(1e-4, 1e-3)
        dmin = rng.choice(dmin_choices) if dmin_choices is not None else rng.uniform(0, 1e-3)
        s = rng.integers(0, 64, 8)
        m = rng.integers(0, 64, 8)
        codes = rng.integers(0, 16, 256)
        blk = make_block(d, dmin, s, m, pack_codes(codes))
        blocks.append(blk)
        params.append((frac(blk[0:2].view(np.float16)[0]), frac(blk[2:4].view(np.float16)[0]), s, m, codes))
    return np.stack(blocks), params


def test_w4a8_worked_example():
    g = golden("q4k_fixture.json")["toy_subblock"]
    w = g["w4a8"]
    # codes of the page's activations at s_x = 0.5 (inverse scale 2)
    assert [oracle.q8_code(v, 1.0 / w["s_x"]) for v in g["x"]] == w["q_x"]
    # the integer route: dot 3, code sum 3, 0.45 - 0.15 = 0.30
    v, idot, csum = oracle.w4a8_term(0.30, 0.10, w["s_x"], g["codes"], w["q_x"])
    assert idot == w["int_dot"] and csum == w["code_sum"]
    assert abs(v - g["dot_exact"]) < 1e-15
    v1, _, _ = oracle.w4a8_term(0.30, 0.0, w["s_x"], g["codes"], w["q_x"])
    v2, _, _ = oracle.w4a8_term(0.0, 0.10, w["s_x"], g["codes"], w["q_x"])
    assert abs(v1 - w["terms"][0]) < 1e-15 and abs(-v2 - w["terms"][1]) < 1e-15


def test_w4a8_worked_example_through_quantizer_and_rows():
    """A block whose first largest-magnitude element is -63.5 has
    iscale = -127 / -63.5 = 2 and scale 1 / 2 = 0.5, the page's s_x, so the
    page's activations quantize to its codes; the Q4_K row built from the
    page's sub-block (d, dmin rounded to fp16) then gives the page's 0.30."""
    g = golden("q4k_fixture.json")["toy_subblock"]
    x = np.zeros(256, np.float32)
    x[0:3] = g["x"]
    x[100] = -63.5  # sub-block 3, whose scale and min are 0
    q, d, bs = oracle.q8_quantize(x)
    assert d[0] == 0.5
    assert list(q[0:3]) == g["w4a8"]["q_x"] and q[100] == -127
    assert bs[0] == g["w4a8"]["code_sum"] and bs[3] == -127
    # a positive maximum flips the sign convention: d = -0.5, codes negated
    x[100] = 63.5
    qn, dn, _ = oracle.q8_quantize(x)
    assert dn[0] == -0.5 and list(qn[0:3]) == [-c for c in g["w4a8"]["q_x"]] and qn[100] == -127
    s = [g["s"]] + [0] * 7
    m = [g["m"]] + [0] * 7
    codes = np.zeros(256, np.uint8)
    codes[0:3] = g["codes"]
    blk = make_block(g["d"], g["dmin"], s, m, pack_codes(codes))
    y, S = oracle.q4k_w4a8_rows(blk[None, None, :], 256, q, d, [0])
    d16 = frac(np.float16(g["d"]))
    dm16 = frac(np.float16(g["dmin"]))
    # sub-block 0 holds 32 elements; codes 0 at elements 3..31 still carry -dmin*m
    exact = sum((d16 * g["s"] * int(codes[i]) - dm16 * g["m"]) * Fraction(1, 2) * int(q[i]) for i in range(32))
    assert y[0] == float(exact)
    assert abs(y[0] - g["dot_exact"]) < 1e-3


def test_q8_textbook_case_is_round_half_even():
    """With a first maximum of -127 the inverse scale is 1 (the scale 1), with
    +127 it is -1, so every code is +-x rounded to the nearest integer, ties to
    even (numpy.rint)."""
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.integers(-252, 253, 512) / 2.0, rng.uniform(-126, 126, 512)]).astype(np.float32)
    x = x.reshape(4, 256)  # only the planted elements below reach magnitude 127
    x[:, 7] = -127.0
    x[1, 7] = 127.0
    x[1, 200] = -127.0  # a later tie of the same magnitude does not change the first maximum
    x = x.ravel()
    q, d, bs = oracle.q8_quantize(x)
    sign = np.array([1.0, -1.0, 1.0, 1.0], np.float32)
    assert np.array_equal(d, sign)
    assert np.array_equal(q.astype(np.float32), np.rint(x * np.repeat(sign, 256)))
    assert q[256 + 7] == -127 and q[256 + 200] == 127


def test_q8_scale_is_reciprocal_of_inverse_scale():
    """d is RN32(1 / RN32(-127 / mx)), which differs in its last bit from
    RN32(-mx / 127) for these maxima; the codes use the inverse scale."""
    from exact import round_f32
    for mx in (30.953386306762695, 57.052589416503906, 19.053972244262695):
        x = np.zeros(256, np.float32)
        x[5] = mx
        x[6] = np.float32(mx / 3)
        q, d, _ = oracle.q8_quantize(x)
        isc = round_f32(Fraction(-127) / frac(np.float32(mx)))
        assert float(d[0]) == round_f32(Fraction(1) / Fraction(isc))
        assert float(d[0]) != round_f32(-frac(np.float32(mx)) / 127)
        prod = round_f32(frac(x[6]) * Fraction(isc))
        assert q[6] == round(Fraction(prod)) and q[5] == -127


@pytest.mark.parametrize("bf16", [False, True])
def test_q8_invariants(bf16):
    rng = np.random.default_rng(11)
    nb = 24
    x = (rng.standard_normal(256 * nb) * rng.uniform(1e-3, 30, 256 * nb)).astype(np.float32)
    x[256 * 2: 256 * 3] = 0.0                 # an all-zero block
    x[256 * 3: 256 * 4] = 0.0
    x[256 * 3 + 17] = -5e-30                  # a block with one tiny negative value
    x[256 * 4: 256 * 5] = 1e30                # a constant huge block
    x[256 * 5: 256 * 6] *= 1e-39              # amax far below 2^-118 (subnormal values): treated as zero
    x[256 * 6: 256 * 7] = 0.0
    x[256 * 6 + 40] = 2.0 ** -118             # exactly at the threshold: quantized
    x[256 * 6 + 41] = -2.0 ** -119
    x[256 * 7: 256 * 8] = 0.0
    x[256 * 7 + 3] = np.float32(2.0 ** -118) * np.float32(1 - 2.0 ** -24)  # just below it
    if bf16:
        from workloads import bf16_bits_from_f32
        xb = bf16_bits_from_f32(x)
        xv = (xb.astype(np.uint32) << 16).view(np.float32)
        q, d, bs = oracle.q8_quantize(xb)
        q2, d2, bs2 = oracle.q8_quantize(xv)   # bf16 input means its binary32 value
        assert np.array_equal(q, q2) and np.array_equal(d, d2) and np.array_equal(bs, bs2)
        x = xv
    else:
        q, d, bs = oracle.q8_quantize(x)
    X = x.reshape(nb, 256).astype(np.float64)
    Q = q.reshape(nb, 256).astype(np.int64)
    assert np.array_equal(bs, Q.reshape(-1, 32).sum(1))
    for b in range(nb):
        amax = np.abs(X[b]).max()
        if amax < 2.0 ** -118:
            assert d[b] == 0 and (Q[b] == 0).all()
            continue
        # the first element of largest magnitude gets code -127, and d has the opposite sign
        i = int(np.abs(X[b]).argmax())  # argmax returns the first occurrence
        assert Q[b, i] == -127
        assert np.sign(d[b]) == -np.sign(X[b, i])
        # |d| is amax / 127 to within two roundings of binary32
        assert abs(abs(float(d[b])) * 127 - amax) <= amax * 2.0 ** -22
        # every code is the nearest integer to x / d, up to binary32 rounding of iscale and the product
        assert (np.abs(X[b] / float(d[b]) - Q[b]) <= 0.5 + 1e-4).all()
        assert (np.abs(Q[b]) <= 127).all()
        # codes are monotone in x * sign(iscale)
        o = np.argsort(X[b] * -np.sign(X[b, i]), kind="stable")
        assert (np.diff(Q[b][o]) >= 0).all()
    assert d[3] > 0 and Q[3, 17] == -127
    if not bf16:
        assert d[5] == 0 and d[7] == 0
        assert Q[6, 40] == -127 and Q[6, 41] == 64  # -2^-119 * (-127 / 2^-118) = 63.5, ties to even


def test_w4a8_rows_exact_on_dyadic_blocks():
    """Power-of-two d and dmin make every weight a short binary fraction, so
    the exact sum of w * d_x * q_x can be formed with fractions and must be
    what the compensated binary64 sum returns, to its last bit or one ulp."""
    rng = np.random.default_rng(5)
    nb, nrows = 4, 3
    k = 256 * nb
    rows, params = [], []
    for _ in range(nrows):
        blk, p = random_row(rng, nb, d_choices=[2.0 ** -8, 2.0 ** -6], dmin_choices=[2.0 ** -9, 2.0 ** -7, 0.0])
        rows.append(blk)
        params.append(p)
    W = np.stack(rows)
    x = (rng.standard_normal(k) * np.repeat(rng.uniform(0.1, 10, nb), 256)).astype(np.float32)
    q, d, _ = oracle.q8_quantize(x)
    y, S = oracle.q4k_w4a8_rows(W, k, q, d, [2, 0, 1])
    for oi, r in enumerate([2, 0, 1]):
        exact = Fraction(0)
        sabs = Fraction(0)
        for b, (db, dmb, s, m, codes) in enumerate(params[r]):
            dx = frac(d[b])
            for i in range(256):
                j = i // 32
                t = (db * int(s[j]) * int(codes[i]) - dmb * int(m[j])) * dx * int(q[256 * b + i])
                exact += t
                sabs += abs(t)
        assert abs(y[oi] - float(exact)) <= np.spacing(abs(float(exact))) + 2.0 ** -60
        assert abs(S[oi] - float(sabs)) <= 1e-12 * float(sabs)


def test_w4a8_rows_equal_the_subblock_identity():
    """Summing the page's per-sub-block identity (integer dot, code sum,
    scale, min correction, activation scale) over a row of random blocks gives
    the row's element-wise dot."""
    rng = np.random.default_rng(9)
    nb = 3
    k = 256 * nb
    blk, params = random_row(rng, nb)
    x = rng.standard_normal(k).astype(np.float32)
    q, d, bs = oracle.q8_quantize(x)
    total = 0.0
    for b, (db, dmb, s, m, codes) in enumerate(params):
        for j in range(8):
            qx = q[256 * b + 32 * j: 256 * b + 32 * j + 32]
            v, _, csum = oracle.w4a8_term(float(db) * int(s[j]), float(dmb) * int(m[j]), float(d[b]),
                                          codes[32 * j: 32 * j + 32], qx)
            assert csum == bs[8 * b + j]
            total += v
    y, S = oracle.q4k_w4a8_rows(blk[None], k, q, d, [0])
    assert abs(y[0] - total) <= 1e-13 * S[0]


def test_w4a8_rows_near_weight_only_dot():
    """Against the binary32 dequantization (one rounding per weight) times the
    same x_hat: the two differ by at most 2^-24 of sum |w x_hat|."""
    from workloads import workload
    inp = workload(3, n=12, k=1024, seed=4)
    q, d, _ = oracle.q8_quantize(inp["x"])
    xhat = np.repeat(d.astype(np.float64), 256) * q.astype(np.float64)
    rows = np.arange(12)
    W = oracle.dequant_rows(oracle.Q4_K, inp["data"], None, 1.0, 1024, rows).astype(np.float64)
    y, S = oracle.q4k_w4a8_rows(inp["data"], 1024, q, d, rows)
    assert np.allclose(S, np.abs(W) @ np.abs(xhat), rtol=1e-6)
    assert (np.abs(y - W @ xhat) <= 2.0 ** -23 * S + 1e-12).all()
    # and x_hat approximates x: the quantization error is at most d / 2 per element
    assert (np.abs(xhat - inp["x"]) <= np.repeat(np.abs(d), 256) * 0.5001).all()
