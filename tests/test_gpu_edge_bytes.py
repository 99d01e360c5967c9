"""GPU parity on the scale bytes at the ends of their ranges, inside the fused
kernels themselves (the exhaustive decode sweeps of `dequantize` do not run
the GEMV's or the GEMM's own scale decode).

Every E8M0 byte 0..254 and every finite E4M3FN byte (both signs, the
subnormals, the zero scales) reaches the GEMV's row kernel and its generic
kernel ("Four Bits, Three Contracts" sections 3 and 4 define the two scale
encodings; Muser, ch. 7 section 7.2, asks that what can be checked completely
be checked completely). Each weight row holds one nonzero block, which carries
the byte under test; the activations over that block are scaled by a power of
two that brings the row's result near 1, so the 1e-5 relative tolerance is
what decides, not the 1e-6 absolute floor. The GEMM gets the E8M0 bytes whose
bf16 weights are subnormal (0, 1, 2) or near overflow (252..254) the same way,
checked against the bf16 band.

Weights that overflow binary32 (E8M0 254 with |E2M1| >= 2, 253 with
|E2M1| >= 4, NVFP4 with a large scale2) decode to +-inf in the oracle. The
kernels factor the block scale out of the block sum, so they agree with the
oracle where every such product overflows by itself (activations >= 1 and one
sign per row): those rows must come out +-inf with the oracle's sign."""
import numpy as np
import pytest
import torch

import bit_block_quantized_nibble_amd as qbn
import oracle
import workloads
from gpu_util import DEV, assert_within_tolerance, dev, host_bits, say, x_dev

pytestmark = pytest.mark.gpu

E4M3FN_FINITE = np.array([b for b in range(256) if b not in (0x7F, 0xFF)], dtype=np.uint8)


def _e8m0_code_cap(byte):
    """Largest E2M1 magnitude code (0..7 for 0, 0.5, 1, 1.5, 2, 3, 4, 6)
    whose weight stays finite in binary32 under this E8M0 byte."""
    return 3 if byte == 254 else 5 if byte == 253 else 7


def _nibbles(rng, size, cap):
    mag = rng.integers(0, cap + 1, size)
    return (mag | (rng.integers(0, 2, size) << 3)).astype(np.uint8)


def _pack(nib):
    """[n][k] nibbles -> [n][k/2] bytes, the even element in the low nibble."""
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)


def _x_host(rng, k, shift, block, xdt):
    """Activations u * 2^shift[k // block], |u| in [0.5, 2), random signs."""
    u = rng.uniform(0.5, 2.0, k) * rng.choice([-1.0, 1.0], k)
    x32 = (u * np.exp2(np.repeat(shift, block).astype(np.float64))).astype(np.float32)
    assert np.isfinite(x32).all() and (np.abs(x32) >= np.float32(2.0 ** -126)).all()
    return x32 if xdt == "f32" else workloads.bf16_bits_from_f32(x32)


def _gemv(fmt, n, k, data, scales, scale2, x, what):
    w = qbn.QTensor(fmt, n, k, dev(data), dev(scales), scale2=scale2)
    say("gemv edge bytes", what, fmt, n, k, x.dtype)
    y = qbn.quantized_gemv(w, x_dev(x))
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _single_block_rows(rng, n, nb, block, row_byte, cap_of):
    """Row r is zero except in block sigma[r], which has scale byte
    row_byte[r] and random codes up to cap_of(byte); every other scale byte of
    the row is drawn from the finite bytes."""
    sigma = rng.permutation(nb)[:n] if n <= nb else np.arange(n) % nb
    nib = np.zeros((n, nb * block), np.uint8)
    for r in range(n):
        j = sigma[r]
        nib[r, block * j:block * (j + 1)] = _nibbles(rng, block, cap_of(row_byte[r]))
    return sigma, _pack(nib)


@pytest.mark.parametrize("k", [8192, 8160])  # 256 blocks: the row kernel; 255: the generic kernel
@pytest.mark.parametrize("xdt", ["f32", "bf16"])
def test_gemv_mxfp4_every_e8m0_byte(k, xdt):
    rng = np.random.default_rng(k + (xdt == "bf16"))
    nb = k // 32
    n = nb
    row_byte = (rng.permutation(n) % 255).astype(np.uint8)  # 0..254, each at least once
    sigma, data = _single_block_rows(rng, n, nb, 32, row_byte, _e8m0_code_cap)
    scales = rng.integers(0, 255, (n, nb)).astype(np.uint8)
    scales[np.arange(n), sigma] = row_byte
    shift = np.zeros(nb, np.int64)
    shift[sigma] = np.clip(127 - row_byte.astype(np.int64), -100, 119)
    x = _x_host(rng, k, shift, 32, xdt)
    y = _gemv("mxfp4", n, k, data, scales, 1.0, x, "e8m0 sweep")
    y_ref, s_ref = oracle.gemv_rows(oracle.MXFP4, data, scales, 1.0, k, x, range(n))
    # every row's terms are large enough that the relative part of the bound decides
    assert np.isfinite(y_ref).all() and (s_ref > 2.0 ** -10).all()
    assert_within_tolerance(y, y_ref, s_ref, "mxfp4 every E8M0 byte, k=%d x=%s" % (k, xdt))


def _e4m3fn_values(b):
    return torch.from_numpy(np.asarray(b, np.uint8)).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)


@pytest.mark.parametrize("k", [4096, 4080])  # 256 blocks: the row kernel; 255: the generic kernel
@pytest.mark.parametrize("xdt", ["f32", "bf16"])
@pytest.mark.parametrize("scale2", [1.0, 0.37])
def test_gemv_nvfp4_every_finite_e4m3fn_byte(k, xdt, scale2):
    rng = np.random.default_rng(k * 3 + (xdt == "bf16") + int(scale2 * 100))
    nb = k // 16
    n = nb
    row_byte = E4M3FN_FINITE[rng.permutation(n) % E4M3FN_FINITE.size]
    sigma, data = _single_block_rows(rng, n, nb, 16, row_byte, lambda b: 7)
    scales = E4M3FN_FINITE[rng.integers(0, E4M3FN_FINITE.size, (n, nb))]
    scales[np.arange(n), sigma] = row_byte
    mag = np.abs(_e4m3fn_values(row_byte))
    shift = np.zeros(nb, np.int64)
    shift[sigma] = np.where(mag > 0, -np.floor(np.log2(np.where(mag > 0, mag, 1.0))), 0).astype(np.int64)
    x = _x_host(rng, k, shift, 16, xdt)
    s2 = float(np.float32(scale2))
    y = _gemv("nvfp4", n, k, data, scales, s2, x, "e4m3fn sweep")
    y_ref, s_ref = oracle.gemv_rows(oracle.NVFP4, data, scales, s2, k, x, range(n))
    assert np.isfinite(y_ref).all()
    zero_rows = mag == 0
    assert zero_rows.sum() >= 2 and (y_ref[zero_rows] == 0).all()
    assert (s_ref[~zero_rows] > 0.25).all()
    assert_within_tolerance(y, y_ref, s_ref, "nvfp4 every finite E4M3FN byte, k=%d x=%s scale2=%g" % (k, xdt, s2))
    # a zero scale gives a zero row, whatever its codes
    assert (y[zero_rows] == 0).all()


def _overflow_rows(rng, k, block, big_byte, small_byte):
    """Four rows: 0 all blocks at big_byte with positive codes >= 2 (every
    weight beyond binary32 when big_byte is), 1 its negation, 2 a finite
    control row at small_byte, 3 the control row with one block of row 0."""
    nb = k // block
    nib = np.zeros((4, k), np.uint8)
    nib[0] = rng.integers(4, 8, k)            # E2M1 2, 3, 4, 6
    nib[1] = nib[0] | 8                        # the same, negative
    nib[2] = _nibbles(rng, k, 7)
    nib[3] = nib[2]
    j = nb // 3
    nib[3, block * j:block * (j + 1)] = nib[0, block * j:block * (j + 1)]
    scales = np.full((4, nb), small_byte, np.uint8)
    scales[0:2] = big_byte
    scales[3, j] = big_byte
    return _pack(nib), scales


def _check_overflow_rows(y, y_ref, s_ref, what):
    assert y_ref[0] == np.inf and y_ref[1] == -np.inf and y_ref[3] == np.inf, what
    assert y[0] == np.inf and y[1] == -np.inf and y[3] == np.inf, "%s: got %r" % (what, y)
    assert_within_tolerance(y[2:3], y_ref[2:3], s_ref[2:3], what + " control row")


@pytest.mark.parametrize("k", [8192, 8160])
@pytest.mark.parametrize("xdt", ["f32", "bf16"])
def test_gemv_mxfp4_overflowing_rows(k, xdt):
    rng = np.random.default_rng(k + 5)
    data, scales = _overflow_rows(rng, k, 32, 254, 120)
    x = _x_host(rng, k, np.zeros(k // 32, np.int64), 32, xdt)
    x = np.abs(x) if xdt == "f32" else (x & np.uint16(0x7FFF))  # positive, 0.5 .. 2
    y = _gemv("mxfp4", 4, k, data, scales, 1.0, x, "overflow rows")
    y_ref, s_ref = oracle.gemv_rows(oracle.MXFP4, data, scales, 1.0, k, x, range(4))
    _check_overflow_rows(y, y_ref, s_ref, "mxfp4 overflow rows k=%d x=%s" % (k, xdt))


@pytest.mark.parametrize("k", [4096, 4080])
@pytest.mark.parametrize("xdt", ["f32", "bf16"])
def test_gemv_nvfp4_overflowing_rows(k, xdt):
    rng = np.random.default_rng(k + 6)
    # scale2 2^120: E4M3FN 448 (0x7E) times E2M1 >= 2 overflows; the control
    # rows' scale 2^-9 (0x01, the smallest subnormal) keeps them finite
    data, scales = _overflow_rows(rng, k, 16, 0x7E, 0x01)
    x = _x_host(rng, k, np.zeros(k // 16, np.int64), 16, xdt)
    x = np.abs(x) if xdt == "f32" else (x & np.uint16(0x7FFF))
    s2 = 2.0 ** 120
    y = _gemv("nvfp4", 4, k, data, scales, s2, x, "overflow rows")
    y_ref, s_ref = oracle.gemv_rows(oracle.NVFP4, data, scales, s2, k, x, range(4))
    _check_overflow_rows(y, y_ref, s_ref, "nvfp4 overflow rows k=%d x=%s" % (k, xdt))


# ------------------------------------------------------------------ GEMM

def _bf16_value(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def _gemm(n, k, data, scales, X, what):
    m = X.shape[0]
    w = qbn.QTensor("mxfp4", n, k, dev(data), dev(scales))
    say("gemm edge bytes", what, m, n, k)
    Y = qbn.quantized_gemm(w, dev(X).view(torch.bfloat16))
    torch.cuda.synchronize()
    return host_bits(Y).reshape(m, n)


GEMM_EDGE_BYTES = np.array([0, 1, 2, 252, 253, 254, 127, 100], np.uint8)


# the 256 x 256 kernel's chunked interior path; its per-k-tile interior path
# with ragged edge tiles; the 128 x 128 kernel
@pytest.mark.parametrize("m,n,k", [(256, 256, 2048), (300, 260, 1088), (96, 200, 1024)])
def test_gemm_edge_e8m0_bytes(m, n, k):
    """E8M0 0, 1, 2 put bf16-subnormal weights (down to 2^-128) into the
    matrix cores; 252..254 weights up to 1.5 * 2^127. Each weight row has one
    nonzero block; block column j carries byte GEMM_EDGE_BYTES[j % 8] in the
    rows that use it, and X over column j is scaled to bring the products
    near 1."""
    rng = np.random.default_rng(m + n + k)
    nb = k // 32
    col_byte = GEMM_EDGE_BYTES[np.arange(nb) % GEMM_EDGE_BYTES.size]
    active = rng.integers(0, nb, n)
    nib = np.zeros((n, k), np.uint8)
    for r in range(n):
        j = active[r]
        nib[r, 32 * j:32 * (j + 1)] = _nibbles(rng, 32, _e8m0_code_cap(col_byte[j]))
    data = _pack(nib)
    scales = rng.integers(0, 255, (n, nb)).astype(np.uint8)
    scales[np.arange(n), active] = col_byte[active]
    shift = np.clip(127 - col_byte.astype(np.int64), -100, 119)
    u = rng.uniform(0.5, 2.0, (m, k)) * rng.choice([-1.0, 1.0], (m, k))
    X = workloads.bf16_bits_from_f32((u * np.exp2(np.repeat(shift, 32))[None, :]).astype(np.float32))
    Y = _gemm(n, k, data, scales, X, "edge e8m0")
    ms, ns = np.meshgrid(np.arange(m), np.arange(n), indexing="ij")
    ms, ns = ms.ravel(), ns.ravel()
    y_ref, s_ref = oracle.gemm_entries(oracle.MXFP4, data, scales, 1.0, k, X, ms, ns)
    assert np.isfinite(y_ref).all()
    sub = np.isin(col_byte[active[ns]], [0, 1, 2])
    assert sub.sum() > 0 and (s_ref > 2.0 ** -8).all()
    T = 1e-5 * s_ref + 1e-6
    lo = _bf16_value(oracle.bf16_rne_array((y_ref - T).astype(np.float32)))
    hi = _bf16_value(oracle.bf16_rne_array((y_ref + T).astype(np.float32)))
    got = _bf16_value(Y[ms, ns])
    bad = ~((lo <= got) & (got <= hi))
    if bad.any():
        i = int(np.argwhere(bad)[0][0])
        raise AssertionError("gemm %dx%dx%d: %d of %d entries outside the band; first (m=%d, n=%d, byte %d): got %r, "
                             "ref %r" % (m, n, k, int(bad.sum()), bad.size, ms[i], ns[i], col_byte[active[ns[i]]],
                                         got[i], y_ref[i]))


@pytest.mark.parametrize("m,n,k", [(256, 256, 2048), (96, 200, 1024)])
def test_gemm_overflowing_weight_rows(m, n, k):
    """Weight rows 0 and 1 at E8M0 254 with codes >= 2 (every weight beyond
    binary32 and bf16) against positive X: columns 0 and 1 of Y are +inf and
    -inf; the other columns are ordinary and checked against the band."""
    rng = np.random.default_rng(m * 7 + k)
    nb = k // 32
    nib = _nibbles(rng, (n, k), 7)
    nib[0] = rng.integers(4, 8, k)
    nib[1] = nib[0] | 8
    data = _pack(nib)
    scales = (120 + rng.integers(0, 8, (n, nb))).astype(np.uint8)
    scales[0:2] = 254
    X = workloads.bf16_bits_from_f32(rng.uniform(1.0, 2.0, (m, k)).astype(np.float32))
    Y = _gemm(n, k, data, scales, X, "overflow rows")
    assert (Y[:, 0] == 0x7F80).all() and (Y[:, 1] == 0xFF80).all()
    ms, ns = np.meshgrid(np.arange(0, m, 5), np.arange(2, n, 3), indexing="ij")
    ms, ns = ms.ravel(), ns.ravel()
    y_ref, s_ref = oracle.gemm_entries(oracle.MXFP4, data, scales, 1.0, k, X, ms, ns)
    T = 1e-5 * s_ref + 1e-6
    lo = _bf16_value(oracle.bf16_rne_array((y_ref - T).astype(np.float32)))
    hi = _bf16_value(oracle.bf16_rne_array((y_ref + T).astype(np.float32)))
    got = _bf16_value(Y[ms, ns])
    assert ((lo <= got) & (got <= hi)).all()
    y0, _ = oracle.gemm_entries(oracle.MXFP4, data, scales, 1.0, k, X, [0, 0], [0, 1])
    assert y0[0] == np.inf and y0[1] == -np.inf


# ------------------------------------------------------------------ Q4_K

# fp16 bit patterns for d across the binades: subnormals (2^-24 upward), the
# smallest normal, ordinary values, the largest finite value, and negatives
Q4K_D_BITS = [0x0001, 0x0155, 0x03FF, 0x0400, 0x1234, 0x2C00, 0x3555, 0x3C00, 0x4A00, 0x6400, 0x7BFF, 0xBC00,
              0x8201]


def _f16_value(bits):
    return float(np.array([bits], np.uint16).view(np.float16)[0])


def _q4k_edge_rows(rng, nb):
    """nb rows, row r nonzero only in super-block r: d from Q4K_D_BITS (then
    random), dmin = d times 2^U{-2..2} (same sign, clamped to the fp16 range),
    6-bit sub-scales and mins with 0 and 63 forced in some sub-blocks, random
    codes; every other super-block has d = dmin = 0."""
    blocks = workloads.q4k_weights(rng, nb, 256 * nb)
    blocks[:, :, 0:4] = 0
    mags = np.zeros(nb)
    for r in range(nb):
        dbits = Q4K_D_BITS[r] if r < len(Q4K_D_BITS) else int(rng.integers(0x0001, 0x7C00))
        d = _f16_value(dbits)
        dmin = float(np.float16(np.clip(abs(d) * 2.0 ** int(rng.integers(-2, 3)), 2.0 ** -24, 65504.0)))
        s = rng.integers(0, 64, 8)
        m = rng.integers(0, 64, 8)
        s[r % 8], m[(r + 3) % 8] = 63, 63
        s[(r + 5) % 8], m[(r + 6) % 8] = 0, 0
        blk = blocks[r, r]
        blk[0:2] = np.array([dbits], np.uint16).view(np.uint8)
        blk[2:4] = np.array([dmin], np.float16).view(np.uint8)
        blk[4:16] = oracle.q4k_pack_scales(s, m)
        mags[r] = max(abs(d) * 63 * 15, dmin * 63)
    return blocks, mags


@pytest.mark.parametrize("k", [4096, 3840])  # 16 super-blocks: the row-loop kernel; 15: the generic kernel
@pytest.mark.parametrize("xdt", ["f32", "bf16"])
def test_gemv_q4k_scale_edges(k, xdt):
    """Q4_K super-block scales at the ends of fp16 (subnormal d and dmin,
    the largest finite d, negative d) and 6-bit sub-scales and mins of 0 and
    63 ("Four Bits, Three Contracts", sections 5 and 6), through the fused
    GEMV; activations over each super-block scaled so its products are near 1."""
    rng = np.random.default_rng(k + (xdt == "bf16"))
    nb = k // 256
    blocks, mags = _q4k_edge_rows(rng, nb)
    shift = -np.floor(np.log2(mags)).astype(np.int64)
    x = _x_host(rng, k, shift, 256, xdt)
    inp = dict(fmt="q4_k", n=nb, k=k, data=blocks, scales=None, scale2=1.0)
    w = qbn.QTensor("q4_k", nb, k, dev(blocks), None)
    say("gemv q4_k scale edges", k, xdt)
    y = qbn.quantized_gemv(w, x_dev(x))
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    y_ref, s_ref = oracle.gemv_rows(oracle.Q4_K, blocks, None, 1.0, k, x, range(nb))
    assert np.isfinite(y_ref).all() and (s_ref > 2.0 ** -6).all()
    assert_within_tolerance(y, y_ref, s_ref, "q4_k scale edges k=%d x=%s" % (k, xdt))


# ------------------------------------------------------------------ Q4_0

@pytest.mark.parametrize("k", [4096, 16384])  # x staged in LDS; x read from global memory (k > 14560)
@pytest.mark.parametrize("xdt", ["f32", "bf16"])
def test_gemv_q4_0_d_edges(k, xdt):
    """Q4_0 block scales d across fp16 ("Bit Packing Architecture", 'Real
    layouts compared': w = d (q - 8)): every subnormal binade, the smallest
    normal, the largest finite value, negative values and both zeros, one
    nonzero block per row, the activations over it scaled so the products
    are near 1; zero scales give zero rows."""
    rng = np.random.default_rng(k * 7 + (xdt == "bf16"))
    nb = k // 32
    dvals = [2.0 ** e if e < -14 else float(np.float16(2.0 ** e * (1 + int(rng.integers(0, 1024)) / 1024.0)))
             for e in range(-24, 16)] + [65504.0, -65504.0, -(2.0 ** -24), -0.375, 0.0, -0.0]
    n = len(dvals)
    blocks = workloads.q4_0_blocks(rng, n, k)
    blocks[:, :, 0:2] = 0
    sigma = rng.permutation(nb)[:n]
    shift = np.zeros(nb, np.int64)
    for r, dv in enumerate(dvals):
        blocks[r, sigma[r], 0:2] = np.array([dv], np.float16).view(np.uint8)
        if dv != 0.0:
            shift[sigma[r]] = -int(np.floor(np.log2(abs(dv) * 8)))
    x = _x_host(rng, k, shift, 32, xdt)
    w = qbn.QTensor("q4_0", n, k, dev(blocks))
    say("gemv q4_0 d edges", k, xdt)
    y = qbn.quantized_gemv(w, x_dev(x))
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    y_ref, s_ref = oracle.gemv_rows(oracle.Q4_0, blocks, None, 1.0, k, x, range(n))
    nz = np.array([dv != 0.0 for dv in dvals])
    assert np.isfinite(y_ref).all() and (y_ref[~nz] == 0).all() and (s_ref[nz] > 2.0 ** -6).all()
    assert (y[~nz] == 0).all()
    assert_within_tolerance(y, y_ref, s_ref, "q4_0 d edges k=%d x=%s" % (k, xdt))


# ------------------------------------------------------------------ NVFP4 in CKE's split-half blocks

@pytest.mark.parametrize("k", [4096, 4160])  # 64 blocks: the row kernel; 65: the generic kernel
@pytest.mark.parametrize("xdt", ["f32", "bf16"])
def test_gemv_cke_every_finite_subscale_byte(k, xdt):
    """Every finite E4M3FN byte as a subscale of CKE's 36-byte blocks ("Why
    4-Bit Quantization Is King", section 5: four subscales, then the split-half
    codes), through the fused GEMV: row r is nonzero only in block sigma[r],
    whose four subscales take the next four bytes of the sweep; every other
    block has zero subscales. The activations over each 16-element subblock
    are scaled to bring its products near 1."""
    rng = np.random.default_rng(k + 17 * (xdt == "bf16"))
    nb = k // 64
    n = nb
    blocks = workloads.cke_blocks(rng, n, k)
    blocks[:, :, 0:4] = 0
    sigma = rng.permutation(nb)
    sweep = E4M3FN_FINITE[rng.permutation(E4M3FN_FINITE.size)]
    shift = np.zeros(4 * nb, np.int64)  # per 16-element subblock
    for r in range(n):
        sub = sweep[(4 * r + np.arange(4)) % sweep.size]
        blocks[r, sigma[r], 0:4] = sub
        mag = np.abs(_e4m3fn_values(sub))
        shift[4 * sigma[r]:4 * sigma[r] + 4] = np.where(mag > 0, -np.floor(np.log2(np.where(mag > 0, mag, 1.0))), 0)
    x = _x_host(rng, k, shift, 16, xdt)
    s2 = float(np.float32(0.37))
    w = qbn.QTensor("nvfp4_cke", n, k, dev(blocks), scale2=s2)
    say("gemv cke subscale sweep", k, xdt)
    y = qbn.quantized_gemv(w, x_dev(x))
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    y_ref, s_ref = oracle.gemv_rows(oracle.NVFP4_CKE, blocks, None, s2, k, x, range(n))
    assert np.isfinite(y_ref).all() and (s_ref > 0.25).all()
    assert_within_tolerance(y, y_ref, s_ref, "cke every subscale byte k=%d x=%s" % (k, xdt))


# ------------------------------------------------------------------ GPTQ / AWQ

@pytest.mark.parametrize("fmt", ["gptq4", "awq4"])
@pytest.mark.parametrize("xdt", ["f32", "bf16"])
def test_gemv_affine_scale_and_zero_edges(fmt, xdt):
    """Group scales across fp16 (every subnormal binade up to 65504, negative
    values) and zero points 0, 8 and 15 ("Bit Packing Architecture", 'Real
    layouts compared': w = s (q - z), so q - z spans -15 .. 15), through the
    fused GPTQ / AWQ GEMV: column n is nonzero only in group gamma[n], and the
    activations over each group are scaled so its products are near 1."""
    K, g = 4096, 32
    ng = K // g
    N = ng  # one group per column
    rng = np.random.default_rng(31 + (fmt == "awq4") * 2 + (xdt == "bf16"))
    svals = [2.0 ** e if e < -14 else float(np.float16(2.0 ** e * (1 + int(rng.integers(0, 1024)) / 1024.0)))
             for e in range(-24, 16)] + [65504.0, -65504.0, -(2.0 ** -24), -0.375]
    if fmt == "gptq4":
        data = rng.integers(0, 2**32, size=(K // 8, N), dtype=np.uint32)
    else:
        data = rng.integers(0, 2**32, size=(K, N // 8), dtype=np.uint32)
    s = np.zeros((ng, N), np.float16)
    z = rng.integers(0, 16, size=(ng, N)).astype(np.uint8)
    gamma = rng.permutation(ng)
    shift = np.zeros(ng, np.int64)
    for col in range(N):
        sv = svals[col % len(svals)]
        s[gamma[col], col] = sv
        z[gamma[col], col] = (0, 15, 8, int(rng.integers(0, 16)))[col % 4]
        shift[gamma[col]] = -int(np.floor(np.log2(abs(sv) * 15)))
    x = _x_host(rng, K, shift, g, xdt)
    w = qbn.QTensor(fmt, N, K, dev(data), dev(s.view(np.uint16)), dev(z), group=g)
    say("gemv affine scale edges", fmt, xdt)
    y = qbn.quantized_gemv(w, x_dev(x))
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    y_ref, s_ref = oracle.int4_gemv(fmt, data, s, z, g, x, range(N))
    assert np.isfinite(y_ref).all() and (s_ref > 2.0 ** -4).all()
    assert_within_tolerance(y, y_ref, s_ref, "%s scale and zero edges x=%s" % (fmt, xdt))


# ------------------------------------------------------------------ W4A8: Q4_K x int8

@pytest.mark.parametrize("k", [4096, 3840])
def test_gemv_q8_q4k_scale_edges(k):
    """The W4A8 route ("Why 4-Bit Quantization Is King", section 7c: per
    256-block d * sum s_j dot_j - dmin * sum m_j bsum_j) on the same
    super-blocks as the Q4_K edge test: fp16 d and dmin from subnormal to
    65504 and negative, sub-scales and mins 0 and 63. The activations are the
    oracle's Q8_K quantization of x scaled per block so the products are near 1."""
    rng = np.random.default_rng(k + 99)
    nb = k // 256
    blocks, mags = _q4k_edge_rows(rng, nb)
    shift = -np.floor(np.log2(mags)).astype(np.int64)
    x = _x_host(rng, k, shift, 256, "f32")
    q, d, bs = oracle.q8_quantize(x)
    w = qbn.QTensor("q4_k", nb, k, dev(blocks), None)
    say("gemv_q8 q4_k scale edges", k)
    y = qbn.quantized_gemv_q8(w, dev(q), dev(d), dev(bs))
    torch.cuda.synchronize()
    y = y.cpu().numpy()
    y_ref, s_ref = oracle.q4k_w4a8_rows(blocks, k, q, d, range(nb))
    assert np.isfinite(y_ref).all() and (s_ref > 2.0 ** -6).all()
    assert_within_tolerance(y, y_ref, s_ref, "gemv_q8 q4_k scale edges k=%d" % k)
