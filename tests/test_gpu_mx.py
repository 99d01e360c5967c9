"""GPU parity of the MX path: qbn_quantize_mx must reproduce the oracle's
OCP MX codes and E8M0 scales bit for bit (MXFP4 and MXFP8);
qbn_quantized_gemm_mx (MXFP4 activations x MXFP4 weights on the
block-scaled matrix cores) must match the oracle's exact sums within
|y - y_ref| <= T = 1e-5 * sum|x_hat w_hat| + 1e-6 (binary32 output), or
inside the round-to-nearest band of that interval (bfloat16 output), on
every entry.

MXFP8 activations (W4A8) are refused by the GEMM. Measured on gfx950
(in-bounds probes, every lane active), v_mfma_scale_f32_32x32x64_f8f6f4 adds
each run of 8 consecutive k aligned to the run's largest product, keeping 13
bits below its exponent and truncating the rest (448 + 2^-5 comes out exact,
448 + 2^-6 as 448). E2M1 x E2M1 products (at most 4 significant bits,
within 2^8 of each other inside a block) never reach the cut, so the W4A4
runs are exact; E4M3 x E2M1 products span 21 binades and do reach it, and
on 37 x 70 x 96 four entries of 2590 missed T. The W4A8 parametrizations
below are skipped for that reason."""
import numpy as np
import pytest
import torch

import bit_block_quantized_nibble_amd as qbn
import oracle
import workloads
from gpu_util import DEV, assert_within_tolerance, dev, host_bits, say

pytestmark = pytest.mark.gpu


def _x_dev(X):
    t = dev(X)
    return t.view(torch.bfloat16) if X.dtype == np.uint16 else t


def _special_rows(rng, m, k):
    X = (rng.standard_normal((m, k)) * np.repeat(10.0 ** rng.uniform(-4, 4, (m, k // 32)), 32, axis=1))
    X = X.astype(np.float32)
    if m > 0 and k >= 32:
        X[0, :32] = 0.0                                   # zero block
    if m > 1 and k >= 64:
        X[1, 32:64] = np.float32(2.0 ** -135)             # scale clamped at 2^-127
        X[1, 40] = np.float32(-2.0 ** -131)
    if m > 2 and k >= 32:
        X[2, :32] = np.float32(0.5) * rng.integers(-12, 13, 32)  # E2M1 ties at scale 1
        X[2, 0] = 6.0
    if m > 3 and k >= 32:
        X[3, :32] = np.float32(3.0e38) * np.sign(rng.standard_normal(32)).astype(np.float32)
    return X


@pytest.mark.parametrize("m,k", [(1, 32), (5, 96), (33, 256), (64, 1024), (7, 8192)])
@pytest.mark.parametrize("xdt", ["f32", "bf16"])
@pytest.mark.parametrize("fmt", ["mxfp4", "mxfp8"])
def test_quantize_mx_bit_exact(m, k, xdt, fmt):
    rng = np.random.default_rng(m * 131 + k)
    X32 = _special_rows(rng, m, k)
    X = X32 if xdt == "f32" else workloads.bf16_bits_from_f32(X32)
    say("quantize_mx", fmt, m, k, xdt)
    codes, scales = qbn.quantize_mx(_x_dev(X), fmt)
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.mx_quantize(X, oracle.MXFP4 if fmt == "mxfp4" else oracle.MXFP8)
    assert np.array_equal(scales.cpu().numpy(), s_ref), "scales differ"
    got = codes.cpu().numpy()
    bad = np.argwhere(got != c_ref)
    assert bad.size == 0, "%d code bytes differ, first at %s: got 0x%02x want 0x%02x" % (
        len(bad), tuple(bad[0]), got[tuple(bad[0])], c_ref[tuple(bad[0])])


def test_quantize_mx_strided_rows():
    rng = np.random.default_rng(4)
    m, k, ld = 9, 256, 320
    X = rng.standard_normal((m, ld)).astype(np.float32)
    say("quantize_mx strided")
    codes, scales = qbn.quantize_mx(dev(X)[:, :k], "mxfp4")
    torch.cuda.synchronize()
    c_ref, s_ref = oracle.mx_quantize(np.ascontiguousarray(X[:, :k]), oracle.MXFP4)
    assert np.array_equal(codes.cpu().numpy(), c_ref) and np.array_equal(scales.cpu().numpy(), s_ref)


def _bf16_value(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


_OFMT = {"mxfp4": oracle.MXFP4, "mxfp8": oracle.MXFP8}
W4A8_SKIP = pytest.mark.skip(reason="MXFP8 x MXFP4 is refused (QBN_ERR_UNSUPPORTED): the FP8 x FP4 matrix "
                             "instruction truncates each run of 8 products 13 bits below the run's largest, "
                             "which misses 1e-5 * sum|x_hat w_hat| + 1e-6 on some entries")
FMTS = ["mxfp4", pytest.param("mxfp8", marks=W4A8_SKIP)]


def _gemm(wc, ws, xc, xs, m, n, k, ydt, what, fmt="mxfp4"):
    w = qbn.QTensor("mxfp4", n, k, dev(wc), dev(ws))
    y = torch.empty((m, n), dtype=ydt, device=DEV)
    say("gemm_mx", fmt, what, m, n, k, ydt)
    qbn.quantized_gemm_mx(w, dev(xc), dev(xs), fmt, y)
    torch.cuda.synchronize()
    return y


def _check(wc, ws, xc, xs, m, n, k, ms, ns, what, fmt="mxfp4"):
    y_ref, s_ref = oracle.mx_gemm_entries(wc, ws, k, _OFMT[fmt], xc, xs, ms, ns)
    T = 1e-5 * s_ref + 1e-6
    y32 = _gemm(wc, ws, xc, xs, m, n, k, torch.float32, what, fmt).cpu().numpy()
    assert_within_tolerance(y32[ms, ns], y_ref, s_ref, "gemm_mx f32 " + what)
    yb = host_bits(_gemm(wc, ws, xc, xs, m, n, k, torch.bfloat16, what, fmt)).reshape(m, n)
    lo = _bf16_value(oracle.bf16_rne_array((y_ref - T).astype(np.float32)))
    hi = _bf16_value(oracle.bf16_rne_array((y_ref + T).astype(np.float32)))
    got = _bf16_value(yb[ms, ns])
    bad = ~((lo <= got) & (got <= hi))
    assert not bad.any(), "gemm_mx bf16 %s: %d entries outside the band" % (what, int(bad.sum()))


def _inputs(rng, m, n, k, fmt="mxfp4"):
    X = workloads.bf16_bits_from_f32(rng.standard_normal((m, k)).astype(np.float32))
    xc, xs = oracle.mx_quantize(X, _OFMT[fmt])
    wc, ws = workloads.mxfp4_weights(rng, n, k, -6, 2)
    return xc, xs, wc, ws


# Shapes reach the small kernel (m or n below 256, or k not a multiple of the
# tiled kernel's k-stage of 256, including k % 64 == 32) and the 256 x 256
# kernel with full and edge tiles, from one k-stage to many.
@pytest.mark.parametrize("m,n,k", [(1, 32, 32), (37, 70, 96), (130, 200, 1056), (64, 512, 2048), (256, 256, 256),
                                   (300, 520, 1024), (512, 256, 4096), (256, 384, 768), (512, 512, 8192),
                                   (256, 256, 128), (260, 512, 640), (384, 300, 1280), (256, 256, 352)])
@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_mx_all_entries(m, n, k, fmt):
    rng = np.random.default_rng(m + 7 * n + k)
    xc, xs, wc, ws = _inputs(rng, m, n, k, fmt)
    ms, ns = np.meshgrid(np.arange(m), np.arange(n), indexing="ij")
    _check(wc, ws, xc, xs, m, n, k, ms.ravel(), ns.ravel(), "%dx%dx%d" % (m, n, k), fmt)


@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_mx_exact_small_integers(fmt):
    """Activations and weights whose products and partial sums are all exact
    in binary32 must come out exactly."""
    rng = np.random.default_rng(8)
    m, n, k = 256, 256, 512
    X = rng.integers(-6, 7, (m, k)).astype(np.float32)
    X[:, ::32] = 6.0  # every block's maximum 6: scale 1 (E2M1) or 2^-6 (E4M3)
    xc, xs = oracle.mx_quantize(X, _OFMT[fmt])
    wc = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    ws = np.full((n, k // 32), 127, np.uint8)
    y = _gemm(wc, ws, xc, xs, m, n, k, torch.float32, "exact", fmt).cpu().numpy()
    ms, ns = np.meshgrid(np.arange(m), np.arange(n), indexing="ij")
    y_ref, _ = oracle.mx_gemm_entries(wc, ws, k, _OFMT[fmt], xc, xs, ms.ravel(), ns.ravel())
    assert np.array_equal(y.ravel().astype(np.float64), y_ref)


@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_mx_workload_end_to_end_sampled(fmt):
    """The GEMM workload's shape (W 8192 x 8192 MXFP4, X 2048 x 8192 bf16):
    device quantizer checked row by row against the oracle on sampled rows,
    then sampled entries of Y against the oracle's exact sums."""
    inp = workloads.workload(4)
    m, n, k = inp["m"], inp["n"], inp["k"]
    say("gemm_mx full workload", fmt, m, n, k)
    Xd = dev(inp["X"]).view(torch.bfloat16)
    xc_d, xs_d = qbn.quantize_mx(Xd, fmt)
    w = qbn.QTensor("mxfp4", n, k, dev(inp["data"]), dev(inp["scales"]))
    Y = qbn.quantized_gemm_mx(w, xc_d, xs_d, fmt)
    torch.cuda.synchronize()
    rng = np.random.default_rng(44)
    rows = np.unique(np.concatenate([rng.integers(0, m, 40), [0, m - 1]]))
    c_ref, s_ref = oracle.mx_quantize(inp["X"][rows], _OFMT[fmt])
    xc = xc_d.cpu().numpy()
    xs = xs_d.cpu().numpy()
    assert np.array_equal(xc[rows], c_ref) and np.array_equal(xs[rows], s_ref)
    ms = np.concatenate([rng.integers(0, m, 1500), np.full(64, m - 1)])
    ns = np.concatenate([rng.integers(0, n, 1500), np.arange(n - 64, n)])
    y_ref, sa = oracle.mx_gemm_entries(inp["data"], inp["scales"], k, _OFMT[fmt], xc, xs, ms, ns)
    T = 1e-5 * sa + 1e-6
    lo = _bf16_value(oracle.bf16_rne_array((y_ref - T).astype(np.float32)))
    hi = _bf16_value(oracle.bf16_rne_array((y_ref + T).astype(np.float32)))
    got = _bf16_value(host_bits(Y).reshape(m, n)[ms, ns])
    assert ((lo <= got) & (got <= hi)).all()


def test_gemm_mx_strided_output_and_empty():
    rng = np.random.default_rng(3)
    m, n, k = 300, 260, 512
    xc, xs, wc, ws = _inputs(rng, m, n, k)
    w = qbn.QTensor("mxfp4", n, k, dev(wc), dev(ws))
    a = _gemm(wc, ws, xc, xs, m, n, k, torch.bfloat16, "plain")
    Yp = torch.zeros((m, n + 8), dtype=torch.bfloat16, device=DEV)
    say("gemm_mx strided")
    qbn.quantized_gemm_mx(w, dev(xc), dev(xs), "mxfp4", Yp[:, :n])
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(Yp[:, :n].contiguous()), host_bits(a))
    assert (host_bits(Yp[:, n:].contiguous()) == 0).all()
    say("gemm_mx k = 0")
    w0 = qbn.QTensor("mxfp4", 24, 0, torch.empty(24, 0, dtype=torch.uint8, device=DEV),
                     torch.empty(24, 0, dtype=torch.uint8, device=DEV))
    y0 = torch.full((5, 24), 3.0, dtype=torch.float32, device=DEV)
    e = torch.empty((5, 0), dtype=torch.uint8, device=DEV)
    qbn.quantized_gemm_mx(w0, e, e, "mxfp4", y0)
    torch.cuda.synchronize()
    assert (y0.cpu() == 0).all()


def test_gemm_mx_refuses_mxfp8_activations():
    """W4A8 on the FP8 x FP4 instruction is refused before any launch, and
    the output is left as it was."""
    rng = np.random.default_rng(12)
    m, n, k = 64, 64, 256
    X = workloads.bf16_bits_from_f32(rng.standard_normal((m, k)).astype(np.float32))
    xc, xs = oracle.mx_quantize(X, oracle.MXFP8)
    wc, ws = workloads.mxfp4_weights(rng, n, k, -6, 2)
    w = qbn.QTensor("mxfp4", n, k, dev(wc), dev(ws))
    y = torch.full((m, n), 7.0, dtype=torch.float32, device=DEV)
    say("gemm_mx mxfp8 refused")
    with pytest.raises(qbn.QbnError) as e:
        qbn.quantized_gemm_mx(w, dev(xc), dev(xs), "mxfp8", y)
    assert e.value.status == 3  # QBN_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    assert (y.cpu() == 7.0).all()


@pytest.mark.parametrize("m,n,k", [(256, 256, 8192), (64, 255, 8160)])  # tiled kernel; small kernel
def test_gemm_mx_every_e8m0_byte_on_both_operands(m, n, k):
    """Every E8M0 byte 0..254 as a weight block scale and as an activation
    block scale, inside the block-scaled matrix core (both bytes go to the
    instruction): weight row r is nonzero only in block column sigma[r], whose
    weight byte b_r sweeps 0..254, and every activation row takes byte 254 - b_r
    in that column, so the product scale is 2^0 and each entry is one block's
    32 exact products. The f32 output within T and the bf16 output within the
    band, for every entry."""
    rng = np.random.default_rng(m + n + k)
    nb = k // 32
    sigma = rng.permutation(nb)[:n]
    wbyte = (np.arange(n) % 255).astype(np.uint8)
    wc = np.zeros((n, k // 2), np.uint8)
    ws = rng.integers(0, 255, (n, nb)).astype(np.uint8)
    for r in range(n):
        wc[r, 16 * sigma[r]:16 * sigma[r] + 16] = rng.integers(0, 256, 16)
        ws[r, sigma[r]] = wbyte[r]
    xc = rng.integers(0, 256, (m, k // 2)).astype(np.uint8)
    xs = rng.integers(100, 155, (m, nb)).astype(np.uint8)
    for r in range(n):
        xs[:, sigma[r]] = 254 - int(wbyte[r])
    ms, ns = np.meshgrid(np.arange(m), np.arange(n), indexing="ij")
    _check(wc, ws, xc, xs, m, n, k, ms.ravel(), ns.ravel(), "every E8M0 byte %dx%dx%d" % (m, n, k))
