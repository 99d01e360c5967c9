"""GPU parity over seeded random shapes: every GEMV format, both activation
dtypes, row counts from 1 to a few hundred and reduction lengths that are
arbitrary multiples of the format's block (so each launcher's shape switch,
the generic kernels and the ragged tails all get drawn), compared element
by element with the oracle within |y - y_ref| <= 1e-5 * sum|w x| + 1e-6.
The shape list is fixed by the seed, so a failure names a reproducible case."""
import numpy as np
import pytest
import torch

import bit_block_quantized_nibble_amd as qbn
import oracle
import workloads
from gpu_util import DEV, assert_within_tolerance, dev, host_bits, say, x_dev

pytestmark = pytest.mark.gpu

# (format, k block, largest k multiple): k = block * U{1..kmax}
FORMATS = {
    "mxfp4": (32, 300),
    "nvfp4": (16, 600),
    "q4_k": (256, 40),
    "q4_0": (32, 300),
    "nvfp4_cke": (64, 150),
    "gptq4": (None, None),
    "awq4": (None, None),
}


def _cases(per_format=12, seed=31337):
    rng = np.random.default_rng(seed)
    out = []
    for fmt, (blk, kmax) in FORMATS.items():
        for i in range(per_format):
            xdt = "bf16" if i % 2 else "f32"
            if fmt in ("gptq4", "awq4"):
                g = int(rng.choice([32, 64, 128]))
                k = g * int(rng.integers(1, 33))
                n = 8 * int(rng.integers(1, 97)) if fmt == "awq4" or i % 3 else int(rng.integers(1, 700))
                out.append((fmt, n, k, g, xdt))
            else:
                k = blk * int(rng.integers(1, kmax + 1))
                n = int(rng.integers(1, 700))
                out.append((fmt, n, k, 0, xdt))
    return out


def _x(rng, k, xdt):
    x32 = rng.standard_normal(k).astype(np.float32)
    return x32 if xdt == "f32" else workloads.bf16_bits_from_f32(x32)


@pytest.mark.parametrize("fmt,n,k,g,xdt", _cases())
def test_gemv_random_shapes(fmt, n, k, g, xdt):
    rng = np.random.default_rng(n * 7919 + k * 31 + g)
    x = _x(rng, k, xdt)
    if fmt in ("gptq4", "awq4"):
        qweight, scales, zeros = workloads.int4_affine(rng, k, n, g)
        data = qweight if fmt == "gptq4" else rng.integers(0, 2**32, size=(k, n // 8), dtype=np.uint32)
        w = qbn.QTensor(fmt, n, k, dev(data), dev(scales.view(np.uint16)), dev(zeros), group=g)
        y_ref, s_ref = oracle.int4_gemv(fmt, data, scales, zeros, g, x, range(n))
    else:
        if fmt == "q4_0":
            data, scales, scale2, ofmt = workloads.q4_0_blocks(rng, n, k), None, 1.0, oracle.Q4_0
        elif fmt == "nvfp4_cke":
            data, scales, scale2, ofmt = workloads.cke_blocks(rng, n, k), None, 0.01, oracle.NVFP4_CKE
        else:
            inp = workloads.workload({"mxfp4": 1, "nvfp4": 2, "q4_k": 3}[fmt], n=n, k=k, seed=int(rng.integers(1 << 30)))
            data, scales, scale2 = inp["data"], inp["scales"], inp["scale2"]
            ofmt = {"mxfp4": oracle.MXFP4, "nvfp4": oracle.NVFP4, "q4_k": oracle.Q4_K}[fmt]
        w = qbn.QTensor(fmt, n, k, dev(data), None if scales is None else dev(scales), scale2=scale2)
        y_ref, s_ref = oracle.gemv_rows(ofmt, data, scales, scale2, k, x, range(n))
    say("gemv sweep", fmt, n, k, g, xdt)
    y = qbn.quantized_gemv(w, x_dev(x))
    torch.cuda.synchronize()
    assert_within_tolerance(y.cpu().numpy(), y_ref, s_ref, "gemv %s n=%d k=%d g=%d x=%s" % (fmt, n, k, g, xdt))


# ------------------------------------------------------------------ GEMMs
# Random (m, n, k) for the MXFP4 bf16 GEMM and the three int4 layouts; about
# half the draws reach the 256-row workgroup tiles (m >= 256). Every entry
# is checked: bf16 outputs inside [RNE(y_ref - T), RNE(y_ref + T)].
def _gemm_cases(count=12, seed=4711):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        m = int(rng.integers(256, 520)) if i % 2 else int(rng.integers(1, 256))
        n = int(rng.integers(1, 520))
        k = 32 * int(rng.integers(1, 33))
        out.append(("mxfp4", m, n, k, 0))
    for fmt in ("gptq4", "awq4", "q4_0"):
        for i in range(count):
            g = int(rng.choice([32, 64, 128]))
            k = g * int(rng.integers(1, 1024 // g + 1))
            m = int(rng.integers(256, 520)) if i % 2 else int(rng.integers(1, 256))
            n = int(rng.integers(1, 66)) * 8 if fmt == "awq4" else int(rng.integers(1, 520))
            out.append((fmt, m, n, k, g if fmt != "q4_0" else 32))
    return out


@pytest.mark.parametrize("fmt,m,n,k,g", _gemm_cases())
def test_gemm_random_shapes(fmt, m, n, k, g):
    ms, ns = np.divmod(np.arange(m * n), n)
    if fmt == "mxfp4":
        from test_gpu_gemm import _check_entries, _run
        inp = workloads.workload(4, n=n, k=k, m=m, seed=m * 131 + n * 7 + k)
        Ybits = _run(inp, "sweep")
        _check_entries(inp, Ybits, ms, ns, "gemm mxfp4 m=%d n=%d k=%d" % (m, n, k))
        return
    from test_gpu_gemm_int4 import _check, _inputs, _qt, _ref
    inp = _inputs(m * 131 + n * 7 + k + g, m, n, k, g)
    w = _qt(fmt, inp, k, n, g)
    X = dev(inp["X"]).view(torch.bfloat16)
    say("gemm sweep", fmt, m, n, k, g)
    Y = qbn.quantized_gemm(w, X)
    torch.cuda.synchronize()
    y_ref, s_ref = _ref(fmt, inp, g, ms, ns)
    _check(Y, y_ref, s_ref, ms, ns, "gemm %s m=%d n=%d k=%d g=%d" % (fmt, m, n, k, g))


# ------------------------------------------------------------------ dequant and repack
def _dequant_cases(per_format=5, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for fmt, (blk, kmax) in FORMATS.items():
        for _ in range(per_format):
            if fmt in ("gptq4", "awq4"):
                g = int(rng.choice([8, 32, 64, 128])) if fmt == "gptq4" else int(rng.choice([32, 64, 128]))
                k = g * int(rng.integers(1, 512 // g + 1))
                n = 8 * int(rng.integers(1, 80)) if fmt == "awq4" else int(rng.integers(1, 600))
                out.append((fmt, n, k, g))
            else:
                out.append((fmt, int(rng.integers(1, 300)), blk * int(rng.integers(1, min(kmax, 4096 // blk) + 1)), 0))
    return out


@pytest.mark.parametrize("fmt,n,k,g", _dequant_cases())
def test_dequant_random_shapes(fmt, n, k, g):
    """Bit-exact dequantization, every output dtype and layout."""
    from test_gpu_dequant import _check_all
    rng = np.random.default_rng(n * 131 + k + g)
    if fmt in ("gptq4", "awq4"):
        q = rng.integers(0, 16, (k, n)).astype(np.uint8)
        scales = rng.uniform(-0.02, 0.02, (k // g, n)).astype(np.float16)
        zeros = rng.integers(0, 16, (k // g, n)).astype(np.uint8)
        data = oracle.gptq_pack(q) if fmt == "gptq4" else oracle.awq_pack(q)
        w = qbn.QTensor(fmt, n, k, dev(data), dev(scales.view(np.uint16)), dev(zeros), group=g)
        ref = np.ascontiguousarray(oracle.affine_dequant(q, scales.view(np.uint16), zeros, g).T)
    else:
        if fmt == "q4_0":
            data, scales, scale2, ofmt = workloads.q4_0_blocks(rng, n, k), None, 1.0, oracle.Q4_0
        elif fmt == "nvfp4_cke":
            data, scales, scale2, ofmt = workloads.cke_blocks(rng, n, k), None, 0.01, oracle.NVFP4_CKE
        else:
            inp = workloads.workload({"mxfp4": 1, "nvfp4": 2, "q4_k": 3}[fmt], n=n, k=k, seed=int(rng.integers(1 << 30)))
            data, scales, scale2 = inp["data"], inp["scales"], inp["scale2"]
            ofmt = {"mxfp4": oracle.MXFP4, "nvfp4": oracle.NVFP4, "q4_k": oracle.Q4_K}[fmt]
        w = qbn.QTensor(fmt, n, k, dev(data), None if scales is None else dev(scales), scale2=scale2)
        ref = oracle.dequant_rows(ofmt, data, scales, scale2, k, range(n))
    _check_all(w, ref, "sweep %s %dx%d g%d" % (fmt, n, k, g))


def _repack_cases(count=4, seed=99):
    from test_gpu_repack import DIRS
    rng = np.random.default_rng(seed)
    out = []
    for src, dst in DIRS:
        for _ in range(count):
            g = int(rng.choice([32, 64, 128, 256]))
            K = g * int(rng.integers(1, 2048 // g + 1))
            N = 8 * int(rng.integers(1, 100)) if "awq4" in (src, dst) else int(rng.integers(1, 600))
            out.append((src, dst, K, N, g))
    return out


@pytest.mark.parametrize("src,dst,K,N,g", _repack_cases())
def test_repack_random_shapes(src, dst, K, N, g):
    """Bit-exact repacks in all six directions; the Q4_0 directions with
    every zero point 8 (the only one Q4_0 holds), so none is refused."""
    from test_gpu_repack import _expect, _mk
    rng = np.random.default_rng(K * 7 + N + g)
    q = rng.integers(0, 16, (K, N)).astype(np.uint8)
    scales = rng.uniform(-0.01, 0.01, (K // g, N)).astype(np.float16).view(np.uint16)
    zeros = rng.integers(0, 16, (K // g, N)).astype(np.uint8)
    if "q4_0" in (src, dst):
        zeros[:] = 8
    w = _mk(src, q, scales, zeros, g)
    say("repack sweep", src, "->", dst, K, N, g)
    out = qbn.repack(w, dst, dst_group=g if dst != "q4_0" else None)
    torch.cuda.synchronize()
    want = _expect(dst, q, scales, g)
    assert np.array_equal(host_bits(out.data).reshape(want.shape).view(np.uint8), want.view(np.uint8))
    if dst != "q4_0":
        assert np.array_equal(host_bits(out.scales).view(np.uint16).reshape(scales.shape), scales)
        assert np.array_equal(host_bits(out.zeros).reshape(zeros.shape), zeros)


# ------------------------------------------------------------------ quantizers and the W4A4 / W4A8 routes
def _mx_cases(count=10, seed=777):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        m = int(rng.integers(256, 520)) if i % 2 else int(rng.integers(1, 256))
        n = int(rng.integers(1, 520)) if i % 3 else int(rng.integers(256, 520))
        k = 32 * int(rng.integers(1, 65))
        out.append((m, n, k))
    return out


@pytest.mark.parametrize("m,n,k", _mx_cases())
def test_gemm_mx_random_shapes(m, n, k):
    """MXFP4 x MXFP4 on the block-scaled matrix cores, every entry, float32
    and bf16 outputs."""
    from test_gpu_mx import _check, _inputs
    rng = np.random.default_rng(m * 17 + n * 3 + k)
    xc, xs, wc, ws = _inputs(rng, m, n, k)
    ms, ns = np.divmod(np.arange(m * n), n)
    _check(wc, ws, xc, xs, m, n, k, ms, ns, "sweep %dx%dx%d" % (m, n, k))


def _q8_cases(count=8, seed=555):
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(1, 400)), 256 * int(rng.integers(1, 57)), "bf16" if i % 2 else "f32")
            for i in range(count)]


@pytest.mark.parametrize("n,k,xdt", _q8_cases())
def test_quantize_q8_and_w4a8_gemv_random_shapes(n, k, xdt):
    """Q8_K activation quantization bit for bit, then the Q4_K x Q8_K GEMV
    within tolerance of the oracle on the oracle's own codes."""
    from test_gpu_w4a8 import _check_quantize
    rng = np.random.default_rng(n * 13 + k)
    x = _x(rng, k, xdt)
    q, d, bs = _check_quantize(x, "sweep k=%d %s" % (k, xdt))
    inp = workloads.workload(3, n=n, k=k, seed=int(rng.integers(1 << 30)))
    w = qbn.QTensor("q4_k", n, k, dev(inp["data"]), None)
    say("gemv_q8 sweep", n, k, xdt)
    y = qbn.quantized_gemv_q8(w, dev(q), dev(d), dev(bs))
    torch.cuda.synchronize()
    y_ref, s_ref = oracle.q4k_w4a8_rows(inp["data"], k, q, d, range(n))
    assert_within_tolerance(y.cpu().numpy(), y_ref, s_ref, "w4a8 sweep n=%d k=%d" % (n, k))


def _encode_cases(count=8, seed=333):
    rng = np.random.default_rng(seed)
    return [(int(rng.integers(1, 300)), 16 * int(rng.integers(1, 300)), "bf16" if i % 2 else "f32", i % 2,
             float(np.float32(rng.choice([1.0, 0.01, 2.0 ** -10])))) for i in range(count)]


@pytest.mark.parametrize("m,k,xdt,tie,scale2", _encode_cases())
def test_quantize_nvfp4_random_shapes(m, k, xdt, tie, scale2):
    """NVFP4 encode bit for bit (codes and E4M3FN scale bytes), both tie rules."""
    from test_gpu_encode import _x as enc_x
    rng = np.random.default_rng(m * 5 + k + tie)
    X32 = enc_x(rng, m, k)
    X = X32 if xdt == "f32" else workloads.bf16_bits_from_f32(X32)
    say("quantize_nvfp4 sweep", m, k, xdt, tie, scale2)
    codes, scales = qbn.quantize_nvfp4(x_dev(X), scale2, tie)
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.nvfp4_quantize(X, scale2, tie)
    assert np.array_equal(scales.cpu().numpy(), s_ref)
    assert np.array_equal(codes.cpu().numpy(), c_ref)


def _int4_cases(count=12, seed=4242):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        g = int(rng.choice([8, 16, 32, 64, 128, 256, 512])) if i % 3 else 2 * int(rng.integers(1, 40))
        k = g * int(rng.integers(1, max(2, 8192 // g)))
        out.append((int(rng.integers(1, 200)), k, g, "bf16" if i % 2 else "f32", int(rng.choice([0, 8, 3])),
                    bool(i % 4 == 1)))
    return out


@pytest.mark.parametrize("m,k,g,xdt,pad,ties", _int4_cases())
def test_quantize_int4_sym_random_shapes(m, k, g, xdt, pad, ties):
    """INT4 symmetric encode bit for bit on random shapes, groups and row
    strides (the lane kernel and the one-thread-per-group kernel). `ties`
    draws half-integer multiples of a power of two, so most quotients sit
    exactly on a rounding boundary or an integer."""
    rng = np.random.default_rng(m + 3 * k + g)
    if ties:
        W32 = (rng.integers(-14, 15, (m, k + pad)) * 0.5 * 2.0 ** rng.integers(-3, 4, (m, 1))).astype(np.float32)
    else:
        W32 = (rng.standard_normal((m, k + pad)) * 10.0 ** rng.uniform(-3, 3, (m, 1))).astype(np.float32)
    W = W32 if xdt == "f32" else workloads.bf16_bits_from_f32(W32)
    say("quantize_int4_sym sweep", m, k, g, xdt, pad, ties)
    codes, scales = qbn.quantize_int4_sym(x_dev(W)[:, :k], g)
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.int4_sym_quantize(np.ascontiguousarray(W[:, :k]), g)
    assert np.array_equal(codes.cpu().numpy(), c_ref)
    assert np.array_equal(host_bits(scales).reshape(s_ref.shape), s_ref.view(np.uint32))


def _pack_cases(count=12, seed=8080):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        bits = int(rng.integers(1, 9))
        lo = int(rng.integers(1, bits)) if bits > 1 and i % 3 == 2 else 0
        out.append((int(rng.integers(1, 200000)), bits, lo, int(i % 2)))
    return out


@pytest.mark.parametrize("count,bits,lo,off", _pack_cases())
def test_pack_bits_random_shapes(count, bits, lo, off):
    """b-bit packing (one stream or two planes) bit for bit on random counts,
    from 16-byte-aligned and unaligned values, and the unpack back."""
    rng = np.random.default_rng(count + bits + lo)
    v = rng.integers(0, 1 << bits, count).astype(np.uint8)
    buf = torch.zeros(count + off, dtype=torch.uint8, device=DEV)
    buf[off:] = dev(v)
    say("pack_bits sweep", count, bits, lo, off)
    w_lo, w_hi = qbn.pack_bits(buf[off:], bits, lo)
    torch.cuda.synchronize()
    if lo:
        lo_ref, hi_ref = oracle.pack_planes(v.astype(np.uint32), bits, lo)
        assert np.array_equal(host_bits(w_hi), hi_ref)
    else:
        lo_ref = oracle.pack_bits(v.astype(np.uint32), bits)
    assert np.array_equal(host_bits(w_lo), lo_ref)
    back = qbn.unpack_bits(w_lo, w_hi, count, bits, lo)
    torch.cuda.synchronize()
    assert np.array_equal(back.cpu().numpy(), v)


def _act_order_cases(count=8, seed=1212):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        g = int(rng.choice([8, 16, 32, 64, 128]))
        K = g * int(rng.integers(1, 1 + min(1100, 16384 // g)))
        out.append((K, int(rng.integers(1, 700)), g))
    return out


@pytest.mark.parametrize("K,N,g", _act_order_cases())
def test_resolve_g_idx_random_shapes(K, N, g):
    """Act-order resolution bit for bit on random K, N and group sizes (both
    placement paths: up to 512 groups and beyond)."""
    rng = np.random.default_rng(K + N + g)
    qw = rng.integers(0, 2**32, (K // 8, N), dtype=np.uint32)
    g_idx = rng.permutation(np.arange(K) // g).astype(np.int32)
    say("resolve g_idx sweep", K, N, g)
    out, perm, status = qbn.gptq_resolve_g_idx(dev(qw), dev(g_idx), g)
    torch.cuda.synchronize()
    rc, perm_ref = oracle.resolve_g_idx(g_idx, g)
    assert int(status.cpu()[0]) == rc == 0
    assert np.array_equal(perm.cpu().numpy(), perm_ref)
    want = oracle.gptq_pack(oracle.gptq_unpack(qw)[perm_ref])
    assert np.array_equal(host_bits(out).reshape(want.shape), want)
