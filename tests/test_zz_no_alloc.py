"""GPU: qbn_repack_noalloc (the repack whose refusal-scan partials live in
the library's file-scope scratch instead of a caller workspace) against
qbn_repack, called through the C ABI: the same destination bytes and the
same result word, on accepted and refused inputs, on two calls in a row
whose second input is smaller."""
import ctypes

import numpy as np
import pytest
import torch

import bit_block_quantized_nibble_amd as qbn
import oracle
from gpu_util import DEV, dev, host_bits, say

pytestmark = pytest.mark.gpu


def _gptq(K, N, g, seed, bad_zero=None):
    rng = np.random.default_rng(seed)
    q = rng.integers(0, 16, (K, N)).astype(np.uint8)
    scales = rng.uniform(0.001, 0.01, (K // g, N)).astype(np.float16).view(np.uint16)
    zeros = np.full((K // g, N), 8, np.uint8)
    if bad_zero is not None:
        zeros.reshape(-1)[bad_zero] = 3
    return q, qbn.QTensor("gptq4", N, K, dev(oracle.gptq_pack(q)), dev(scales), dev(zeros), group=g)


def _both(src, dst_format, g=None):
    """Run qbn_repack and qbn_repack_noalloc into fresh, identically filled
    destinations; returns both destinations and both result words."""
    lib = qbn._load()
    outs = []
    for fn in ("qbn_repack", "qbn_repack_noalloc"):
        dst = qbn.repack_target(src, dst_format, g)
        dst.data.fill_(0x3C if dst.data.dtype == torch.uint8 else 0x3C3C3C3C)
        if dst.format != "q4_0" and src.format == "q4_0":
            dst.scales.fill_(0)
            dst.zeros.fill_(0)
        words = torch.full((qbn.REPACK_STATUS_WORDS,), 99, dtype=torch.int64, device=DEV)
        cs, cd = src._c(), dst._c()
        say(fn, src.format, "->", dst_format, src.n, src.k)
        st = getattr(lib, fn)(ctypes.byref(cs), ctypes.byref(cd), ctypes.c_void_p(words.data_ptr()),
                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == 0, (fn, st)
        torch.cuda.synchronize()
        outs.append((dst, int(words[0].item())))
    return outs


def _same(a, b):
    assert np.array_equal(host_bits(a.data), host_bits(b.data))
    for x, y in ((a.scales, b.scales), (a.zeros, b.zeros)):
        if x is not None:
            assert np.array_equal(host_bits(x), host_bits(y))


@pytest.mark.parametrize("K,N,g", [(512, 264, 128), (256, 64, 64)])  # the second call is smaller
def test_noalloc_matches_repack_accepted_and_refused(K, N, g):
    q, src = _gptq(K, N, g, seed=K + N)
    (a, ra), (b, rb) = _both(src, "q4_0")
    assert ra == rb == -1
    _same(a, b)
    want = oracle.q4_0_pack(q, np.ascontiguousarray(np.repeat(host_bits(src.scales).view(np.uint16).reshape(K // g, N).T,
                                                              g // 32, axis=1)))
    assert np.array_equal(host_bits(b.data).reshape(want.shape), want)
    # back to AWQ through the scratch path too
    (c, rc), (d, rd) = _both(b, "awq4", g)
    assert rc == rd == -1
    _same(c, d)
    assert np.array_equal(host_bits(d.data).view(np.uint32), oracle.awq_pack(q))
    # a zero point of 3: both refuse at the same index and leave the destination alone
    bad = (K // g) * N // 2 + 5
    _, src_bad = _gptq(K, N, g, seed=K + N, bad_zero=bad)
    (e, re_), (f, rf) = _both(src_bad, "q4_0")
    assert re_ == rf == bad
    assert (e.data == 0x3C).all().item() and (f.data == 0x3C).all().item()


def test_noalloc_two_calls_in_a_row_smaller_second():
    """Back-to-back calls share the scratch: a large refused call followed by
    a smaller accepted one must still report the second call's own result."""
    _, big = _gptq(1024, 512, 128, seed=5, bad_zero=7)
    q, small = _gptq(256, 72, 128, seed=6)
    (a1, r1), (b1, s1) = _both(big, "q4_0")
    (a2, r2), (b2, s2) = _both(small, "q4_0")
    assert r1 == s1 == 7 and r2 == s2 == -1
    _same(a2, b2)
