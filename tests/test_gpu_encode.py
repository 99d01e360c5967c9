"""GPU parity of the encode side, bit for bit against the oracle: NVFP4
quantization under both tie rules, signed INT4 symmetric quantization, and
b-bit packing (single streams with straddles, and bit planes) both ways."""
import numpy as np
import pytest
import torch

import bit_block_quantized_nibble_amd as qbn
import oracle
import workloads
from gpu_util import DEV, dev, host_bits, say, x_dev

pytestmark = pytest.mark.gpu


def _x(rng, m, k, spread=True):
    X = rng.standard_normal((m, k))
    if spread:
        X = X * np.repeat(10.0 ** rng.uniform(-4, 3, (m, k // 16)), 16, axis=1)
    X = X.astype(np.float32)
    if m > 1 and k >= 32:
        X[1, 16:32] = 0.0                      # a zero block
        X[0, :16] = np.float32(0.5) * rng.integers(-12, 13, 16)  # exact E2M1 midpoints at scale 1 / 6
    return X


@pytest.mark.parametrize("m,k", [(1, 16), (5, 96), (64, 4096), (130, 160)])
@pytest.mark.parametrize("xdt", ["f32", "bf16"])
@pytest.mark.parametrize("tie", [0, 1])
@pytest.mark.parametrize("scale2", [1.0, 0.01, 2.0 ** -20])
def test_quantize_nvfp4_bit_exact(m, k, xdt, tie, scale2):
    rng = np.random.default_rng(m * 3 + k + tie)
    X32 = _x(rng, m, k)
    X = X32 if xdt == "f32" else workloads.bf16_bits_from_f32(X32)
    say("quantize_nvfp4", m, k, xdt, tie, scale2)
    codes, scales = qbn.quantize_nvfp4(x_dev(X), float(np.float32(scale2)), tie)
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.nvfp4_quantize(X, float(np.float32(scale2)), tie)
    assert np.array_equal(scales.cpu().numpy(), s_ref)
    got = codes.cpu().numpy()
    bad = np.argwhere(got != c_ref)
    assert bad.size == 0, "%d code bytes differ, first %s: 0x%02x vs 0x%02x" % (
        len(bad), tuple(bad[0]), got[tuple(bad[0])], c_ref[tuple(bad[0])])


def test_quantize_nvfp4_round_trip_through_the_gemv():
    """Quantize on the device, then run the NVFP4 GEMV on the result: the
    outputs match the oracle's GEMV of the oracle's own encoding."""
    rng = np.random.default_rng(4)
    n, k, scale2 = 96, 2048, np.float32(0.01)
    W = _x(rng, n, k, spread=False)
    codes, scales = qbn.quantize_nvfp4(dev(W), float(scale2), 0)
    x = workloads.x_f32(rng, k)
    w = qbn.QTensor("nvfp4", n, k, codes, scales, scale2=float(scale2))
    say("nvfp4 encode + gemv")
    y = qbn.quantized_gemv(w, dev(x))
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.nvfp4_quantize(W, float(scale2), 0)
    y_ref, sa = oracle.gemv_rows(oracle.NVFP4, c_ref, s_ref, float(scale2), k, x, range(n))
    err = np.abs(y.cpu().numpy().astype(np.float64) - y_ref)
    assert (err <= 1e-5 * sa + 1e-6).all()


@pytest.mark.parametrize("m,k,g", [(1, 4, 4), (7, 96, 32), (64, 4096, 128), (3, 64, 2)])
@pytest.mark.parametrize("xdt", ["f32", "bf16"])
def test_quantize_int4_sym_bit_exact(m, k, g, xdt):
    rng = np.random.default_rng(m + k + g)
    W32 = rng.standard_normal((m, k)).astype(np.float32)
    if m == 1 and k == 4:
        W32[0] = [-1.0, 0.25, 0.875, 1.75]  # the page's example: bytes 0x1C 0x74
    if m > 2:
        W32[2, :g] = 0.0
    W = W32 if xdt == "f32" else workloads.bf16_bits_from_f32(W32)
    say("quantize_int4_sym", m, k, g, xdt)
    codes, scales = qbn.quantize_int4_sym(x_dev(W), g)
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.int4_sym_quantize(W, g)
    assert np.array_equal(codes.cpu().numpy(), c_ref)
    assert np.array_equal(host_bits(scales).reshape(s_ref.shape), s_ref.view(np.uint32))


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("count", [1, 31, 32, 96, 1000, 100003])
def test_pack_bits_sequential(bits, count):
    rng = np.random.default_rng(bits * 7 + count)
    v = rng.integers(0, 256, count).astype(np.uint8)  # bits above `bits` must be ignored
    say("pack_bits", bits, count)
    lo, hi = qbn.pack_bits(dev(v), bits)
    torch.cuda.synchronize()
    want = oracle.pack_bits((v & ((1 << bits) - 1)).astype(np.uint32), bits)
    assert np.array_equal(host_bits(lo), want)
    back = qbn.unpack_bits(lo, None, count, bits)
    torch.cuda.synchronize()
    assert np.array_equal(back.cpu().numpy(), v & ((1 << bits) - 1))


@pytest.mark.parametrize("bits,lo_bits", [(6, 4), (3, 2), (5, 1), (8, 4), (7, 3)])
def test_pack_bits_planes(bits, lo_bits):
    rng = np.random.default_rng(bits * 11 + lo_bits)
    count = 4096
    v = rng.integers(0, 1 << bits, count).astype(np.uint8)
    say("pack_bits planes", bits, lo_bits)
    lo, hi = qbn.pack_bits(dev(v), bits, lo_bits)
    torch.cuda.synchronize()
    lo_ref, hi_ref = oracle.pack_planes(v.astype(np.uint32), bits, lo_bits)
    assert np.array_equal(host_bits(lo), lo_ref) and np.array_equal(host_bits(hi), hi_ref)
    back = qbn.unpack_bits(lo, hi, count, bits, lo_bits)
    torch.cuda.synchronize()
    assert np.array_equal(back.cpu().numpy(), v)


@pytest.mark.parametrize("g", [8, 16, 64, 256, 512, 1024, 24])
@pytest.mark.parametrize("xdt", ["f32", "bf16"])
def test_quantize_int4_sym_group_sizes(g, xdt):
    """Group sizes 8 L for L = 1 .. 64 lanes per group (the lane kernel), and
    1024 and 24 (one thread per group), each with a zero group."""
    m, k = 9, 3072
    rng = np.random.default_rng(g * 5 + len(xdt))
    W32 = (rng.standard_normal((m, k)) * 10.0 ** rng.uniform(-3, 3, (m, 1))).astype(np.float32)
    W32[4, g:2 * g] = 0.0
    W = W32 if xdt == "f32" else workloads.bf16_bits_from_f32(W32)
    say("quantize_int4_sym group", g, xdt)
    codes, scales = qbn.quantize_int4_sym(x_dev(W), g)
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.int4_sym_quantize(W, g)
    assert np.array_equal(codes.cpu().numpy(), c_ref)
    assert np.array_equal(host_bits(scales).reshape(s_ref.shape), s_ref.view(np.uint32))


@pytest.mark.parametrize("pad,off", [(8, 0), (3, 0), (8, 1)])
@pytest.mark.parametrize("xdt", ["f32", "bf16"])
def test_quantize_int4_sym_strided_rows(pad, off, xdt):
    """Rows inside a wider matrix: a 16-byte row stride and base (pad 8, no
    offset) keep the lane kernel; an odd stride or a base one element in
    takes the one-thread-per-group kernel. Both bit-exact."""
    m, k, g = 6, 512, 32
    rng = np.random.default_rng(pad * 3 + off + len(xdt))
    W32 = rng.standard_normal((m, k + pad)).astype(np.float32)
    W = W32 if xdt == "f32" else workloads.bf16_bits_from_f32(W32)
    Wd = x_dev(W)[:, off:off + k]
    say("quantize_int4_sym strided", pad, off, xdt)
    codes, scales = qbn.quantize_int4_sym(Wd, g)
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.int4_sym_quantize(np.ascontiguousarray(W[:, off:off + k]), g)
    assert np.array_equal(codes.cpu().numpy(), c_ref)
    assert np.array_equal(host_bits(scales).reshape(s_ref.shape), s_ref.view(np.uint32))


@pytest.mark.parametrize("bits,lo_bits", [(3, 0), (5, 0), (8, 0), (6, 4)])
@pytest.mark.parametrize("count", [33, 1000, 100003])
def test_pack_bits_unaligned_values(bits, lo_bits, count):
    """Values starting one byte past a 16-byte boundary (byte loads) against
    the same values aligned (16-byte loads): both equal the oracle."""
    rng = np.random.default_rng(bits * 13 + count + lo_bits)
    v = rng.integers(0, 1 << bits, count).astype(np.uint8)
    buf = torch.zeros(count + 1, dtype=torch.uint8, device=DEV)
    buf[1:] = dev(v)
    say("pack_bits unaligned", bits, lo_bits, count)
    lo, hi = qbn.pack_bits(buf[1:], bits, lo_bits)
    lo_a, hi_a = qbn.pack_bits(dev(v), bits, lo_bits)
    torch.cuda.synchronize()
    if lo_bits:
        lo_ref, hi_ref = oracle.pack_planes(v.astype(np.uint32), bits, lo_bits)
        assert np.array_equal(host_bits(hi), hi_ref) and np.array_equal(host_bits(hi_a), hi_ref)
    else:
        lo_ref = oracle.pack_bits(v.astype(np.uint32), bits)
    assert np.array_equal(host_bits(lo), lo_ref) and np.array_equal(host_bits(lo_a), lo_ref)


@pytest.mark.parametrize("pad,off", [(16, 0), (3, 0), (16, 1)])
@pytest.mark.parametrize("xdt", ["f32", "bf16"])
@pytest.mark.parametrize("tie", [0, 1])
def test_quantize_nvfp4_strided_rows(pad, off, xdt, tie):
    """Rows inside a wider matrix: a 16-byte row stride and base keep the
    two-lanes-per-block kernel; an odd stride or a base one element in take
    the one-thread-per-block kernel. Both bit-exact."""
    m, k, scale2 = 7, 1024, 0.01
    rng = np.random.default_rng(pad * 5 + off + tie + len(xdt))
    X32 = _x(rng, m, k + 16)[:, :k + pad] if pad <= 16 else None
    X = X32 if xdt == "f32" else workloads.bf16_bits_from_f32(X32)
    X = np.ascontiguousarray(X)
    Xd = x_dev(X)[:, off:off + k]
    say("quantize_nvfp4 strided", pad, off, xdt, tie)
    codes, scales = qbn.quantize_nvfp4(Xd, float(np.float32(scale2)), tie)
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.nvfp4_quantize(np.ascontiguousarray(X[:, off:off + k]), float(np.float32(scale2)), tie)
    assert np.array_equal(scales.cpu().numpy(), s_ref)
    assert np.array_equal(codes.cpu().numpy(), c_ref)


@pytest.mark.parametrize("xdt", ["f32", "bf16"])
@pytest.mark.parametrize("tie", [0, 1])
def test_quantize_nvfp4_quotient_overflow(xdt, tie):
    """A tiny per-tensor scale under large weights: the block scale saturates
    at 448 and x / t overflows binary32 to infinity, whose code still
    saturates at magnitude 6 (sign kept); zeros and a negative zero too."""
    rng = np.random.default_rng(77 + tie)
    X32 = (rng.standard_normal((4, 64)) * 1e12).astype(np.float32)
    X32[0, :16] = 0.0
    X32[1, 0] = -0.0
    X = X32 if xdt == "f32" else workloads.bf16_bits_from_f32(X32)
    scale2 = float(np.float32(1e-30))
    say("quantize_nvfp4 overflow", xdt, tie)
    codes, scales = qbn.quantize_nvfp4(x_dev(X), scale2, tie)
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.nvfp4_quantize(X, scale2, tie)
    assert np.array_equal(scales.cpu().numpy(), s_ref)
    assert np.array_equal(codes.cpu().numpy(), c_ref)
