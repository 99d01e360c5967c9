"""Pins of the oracle's int4 GEMM entries (Y = X @ W_hat, X bfloat16 [M][K],
W_hat the int4 weight of "Bit Packing Architecture", 'Real layouts compared':
s * (q - z) for GPTQ / AWQ, d * (q - 8) for Q4_0).

Every entry must equal the product of the bfloat16 activations with the
weight dequantized element by element from those definitions, computed here
independently with numpy's float64 matmul; the three layouts of one logical
weight (zero point 8, group 32, d = s) must give the same entries."""
import numpy as np

import oracle


def _bf16_f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _setup(seed, K=96, N=40, M=5, g=32):
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 16, (K, N)).astype(np.uint8)
    s = rng.uniform(1e-3, 1e-2, (K // g, N)).astype(np.float16)
    z = rng.integers(0, 16, (K // g, N)).astype(np.uint8)
    X = rng.standard_normal((M, K)).astype(np.float32)
    Xb = (X.view(np.uint32) >> 16).astype(np.uint16)  # any bfloat16 bit patterns will do
    return q, s, z, Xb


def _all_entries(M, N):
    ms, ns = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    return ms.ravel(), ns.ravel()


def test_gptq_and_awq_entries_equal_the_float64_product():
    for g in (32, 96):
        q, s, z, Xb = _setup(1 + g, g=g)
        K, N = q.shape
        M = Xb.shape[0]
        W = s.astype(np.float64).repeat(g, axis=0) * (q.astype(np.float64) - z.astype(np.float64).repeat(g, axis=0))
        want = _bf16_f64(Xb) @ W
        ms, ns = _all_entries(M, N)
        for fmt, data in (("gptq4", oracle.gptq_pack(q)), ("awq4", oracle.awq_pack(q))):
            y, S = oracle.int4_gemm_entries(fmt, data, s, z, g, Xb, ms, ns)
            assert np.allclose(y, want[ms, ns], rtol=0, atol=1e-12 * S.max()), fmt
            assert np.allclose(S, (np.abs(_bf16_f64(Xb)) @ np.abs(W))[ms, ns], rtol=1e-12)


def test_q4_0_entries_equal_the_float64_product():
    q, s, _, Xb = _setup(7)
    K, N = q.shape
    M = Xb.shape[0]
    d_bits = np.ascontiguousarray(s.T.view(np.uint16))  # [N][K/32]: one d per block
    blocks = oracle.q4_0_pack(q, d_bits)
    W = s.astype(np.float64).repeat(32, axis=0) * (q.astype(np.float64) - 8.0)
    want = _bf16_f64(Xb) @ W
    ms, ns = _all_entries(M, N)
    y, S = oracle.int4_gemm_entries("q4_0", blocks, None, None, 32, Xb, ms, ns)
    assert np.allclose(y, want[ms, ns], rtol=0, atol=1e-12 * S.max())


def test_three_layouts_of_one_weight_agree():
    q, s, _, Xb = _setup(11)
    K, N = q.shape
    M = Xb.shape[0]
    z8 = np.full((K // 32, N), 8, np.uint8)
    ms, ns = _all_entries(M, N)
    a, _ = oracle.int4_gemm_entries("gptq4", oracle.gptq_pack(q), s, z8, 32, Xb, ms, ns)
    b, _ = oracle.int4_gemm_entries("awq4", oracle.awq_pack(q), s, z8, 32, Xb, ms, ns)
    blocks = oracle.q4_0_pack(q, np.ascontiguousarray(s.T.view(np.uint16)))
    c, S = oracle.int4_gemm_entries("q4_0", blocks, None, None, 32, Xb, ms, ns)
    assert np.array_equal(a, b)
    assert np.allclose(a, c, rtol=0, atol=1e-13 * S.max())


def test_sampled_entries_follow_their_rows():
    """Entries requested in any order (and repeated) come back in that order."""
    q, s, z, Xb = _setup(13)
    ms = np.array([4, 0, 4, 2, 0])
    ns = np.array([39, 0, 1, 17, 0])
    y, _ = oracle.int4_gemm_entries("gptq4", oracle.gptq_pack(q), s, z, 32, Xb, ms, ns)
    full, _ = oracle.int4_gemm_entries("gptq4", oracle.gptq_pack(q), s, z, 32, Xb, *_all_entries(5, 40))
    assert np.array_equal(y, full.reshape(5, 40)[ms, ns])
