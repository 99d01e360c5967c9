"""Pins for the oracle's GPTQ metadata conventions ("Bit Packing
Architecture", "Real layouts compared" and "Repacking between formats"):
qzeros packed along the output dimension as a 4-bit stream (column 8c + j at
bits 4j of word c), version 1 storing z - 1, version 2 storing z; act-order
g_idx resolved by ordering rows by group, which must leave every output of
the layer unchanged once the activations are permuted alike."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from exact import frac


def test_qzeros_bit_positions_from_the_layout_rule():
    # columns 0..7 with zero points 0..7 (version 2): nibble j = column j
    z = np.arange(8, dtype=np.uint8).reshape(1, 8)
    assert oracle.qzeros_pack(z, 2)[0, 0] == 0x76543210
    # one column set: column 5 of the second word is bits 20..23 of word 1
    z = np.zeros((1, 16), np.uint8)
    z[0, 13] = 0xA
    qz = oracle.qzeros_pack(z, 2)
    assert qz[0, 0] == 0 and qz[0, 1] == 0xA << 20


def test_qzeros_version_1_stores_z_minus_one():
    z = np.full((2, 8), 8, np.uint8)
    assert (oracle.qzeros_pack(z, 1) == 0x77777777).all()
    assert (oracle.qzeros_unpack(np.full((2, 1), 0x77777777, np.uint32), 1) == 8).all()
    # reading a version-1 tensor as version 2 shifts every zero point by one
    rng = np.random.default_rng(1)
    z = rng.integers(1, 17, (3, 24)).astype(np.uint8)
    assert np.array_equal(oracle.qzeros_unpack(oracle.qzeros_pack(z, 1), 2).astype(int), z.astype(int) - 1)


def test_qzeros_round_trips_and_unsigned_reading():
    rng = np.random.default_rng(2)
    z2 = rng.integers(0, 16, (5, 40)).astype(np.uint8)
    assert np.array_equal(oracle.qzeros_unpack(oracle.qzeros_pack(z2, 2), 2), z2)
    z1 = rng.integers(1, 17, (5, 40)).astype(np.uint8)
    assert np.array_equal(oracle.qzeros_unpack(oracle.qzeros_pack(z1, 1), 1), z1)
    # a top nibble >= 8 makes the stored int32 negative; it must read back unsigned
    qz = np.array([[-0x10000000]], dtype=np.int32)  # 0xF0000000
    assert list(oracle.qzeros_unpack(qz.view(np.uint32), 2)[0]) == [0] * 7 + [15]
    # version 1 cannot hold zero point 0: it reads back as 16
    assert oracle.qzeros_unpack(oracle.qzeros_pack(np.zeros((1, 8), np.uint8), 1), 1)[0, 0] == 16


def test_resolve_g_idx_monotonic_is_identity():
    K, g = 256, 32
    rc, perm = oracle.resolve_g_idx(np.arange(K) // g, g)
    assert rc == 0 and np.array_equal(perm, np.arange(K))


def test_resolve_g_idx_orders_by_group_stably():
    rng = np.random.default_rng(3)
    K, g = 128, 16
    g_idx = rng.permutation(np.arange(K) // g).astype(np.int32)
    rc, perm = oracle.resolve_g_idx(g_idx, g)
    assert rc == 0
    assert sorted(perm.tolist()) == list(range(K))                # a permutation
    assert np.array_equal(g_idx[perm], np.arange(K) // g)          # groups contiguous, in order
    for gi in range(K // g):
        assert np.all(np.diff(perm[gi * g:(gi + 1) * g]) > 0)      # original order inside a group


def test_resolve_g_idx_errors():
    g_idx = np.arange(64) // 16
    bad = g_idx.copy()
    bad[3] = 4
    assert oracle.resolve_g_idx(bad, 16)[0] == -1
    bad = g_idx.copy()
    bad[3] = 1  # group 0 now holds 15 rows, group 1 holds 17
    assert oracle.resolve_g_idx(bad, 16)[0] == -2


def test_act_order_resolution_preserves_the_layer():
    """y = sum_k s[g_idx[k]] (q[k] - z[g_idx[k]]) x[k] with a scattered g_idx
    equals the resolved layout's output on the permuted activations."""
    rng = np.random.default_rng(4)
    K, N, g = 128, 16, 32
    q = rng.integers(0, 16, (K, N)).astype(np.uint8)
    s = rng.uniform(1e-3, 1e-2, (K // g, N)).astype(np.float16)
    z = rng.integers(0, 16, (K // g, N)).astype(np.uint8)
    x = rng.standard_normal(K).astype(np.float32)
    g_idx = rng.permutation(np.arange(K) // g).astype(np.int32)
    rc, perm = oracle.resolve_g_idx(g_idx, g)
    assert rc == 0
    y, _ = oracle.int4_gemv("gptq4", oracle.gptq_pack(q[perm]), s, z, g, x[perm], range(N))
    for n in range(N):
        exact = sum(frac(np.float32(float(s[g_idx[k], n]) * (int(q[k, n]) - int(z[g_idx[k], n])))) * frac(x[k])
                    for k in range(K))
        assert abs(Fraction(y[n]) - exact) <= Fraction(1, 2**50) * abs(exact) + Fraction(1, 2**100)
