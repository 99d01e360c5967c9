"""GPU parity of the W4A8 route: qbn_quantize_q8 must reproduce the oracle's
int8 codes, block scales and code sums bit for bit; qbn_quantized_gemv_q8
must match the oracle's binary64 Q4_K x int8 dot within
|y - y_ref| <= 1e-5 * sum|w x_hat| + 1e-6, row by row."""
import numpy as np
import pytest
import torch

import bit_block_quantized_nibble_amd as qbn
import oracle
import workloads
from gpu_util import DEV, assert_within_tolerance, dev, host_bits, qtensor, say, x_dev

pytestmark = pytest.mark.gpu


def _quantize(x_host, what):
    say("quantize_q8", what, x_host.size, x_host.dtype)
    q, d, bs = qbn.quantize_q8(x_dev(x_host))
    torch.cuda.synchronize()
    return q.cpu().numpy(), host_bits(d), bs.cpu().numpy()


def _check_quantize(x_host, what):
    q, d_bits, bs = _quantize(x_host, what)
    q_ref, d_ref, bs_ref = oracle.q8_quantize(x_host)
    assert np.array_equal(d_bits, d_ref.view(np.uint32)), "%s: block scales differ" % what
    bad = np.flatnonzero(q != q_ref)
    assert bad.size == 0, "%s: %d codes differ, first at %d: got %d want %d" % (
        what, bad.size, bad[0], q[bad[0]], q_ref[bad[0]])
    assert np.array_equal(bs, bs_ref), "%s: code sums differ" % what
    return q_ref, d_ref, bs_ref


def _special_x(k, rng):
    """N(0,1) blocks interleaved with the quantizer's corner cases."""
    x = (rng.standard_normal(k) * np.repeat(rng.uniform(1e-3, 50, k // 256), 256)).astype(np.float32)
    nb = k // 256
    cases = [
        lambda b: b.fill(0.0),                                               # zero block
        lambda b: b.__imul__(np.float32(1e-39)),                             # amax far below 2^-118
        lambda b: (b.fill(0.0), b.__setitem__(9, np.float32(2.0 ** -118))),  # exactly at the threshold
        lambda b: (b.fill(0.0), b.__setitem__(200, np.float32(-2.0 ** -118) * np.float32(1 - 2.0 ** -24))),
        lambda b: (b.__setitem__(slice(None), np.float32(0.5) * rng.integers(-254, 255, 256)),
                   b.__setitem__(3, -127.0)),                                # ties at scale 1
        lambda b: b.fill(np.float32(-3e38)),                                 # huge, negative, constant
        lambda b: b.__setitem__(slice(None), np.float32(1e-30) * rng.standard_normal(256)),  # tiny but quantized
    ]
    for i, f in enumerate(cases):
        if i < nb:
            blk = x[256 * i: 256 * (i + 1)]
            f(blk)
    return x


@pytest.mark.parametrize("k", [256, 1024, 4096, 256 * 43, 14336])
@pytest.mark.parametrize("xdt", ["f32", "bf16"])
def test_quantize_q8_bit_exact(k, xdt):
    rng = np.random.default_rng(k + (xdt == "bf16"))
    x32 = _special_x(k, rng)
    x = x32 if xdt == "f32" else workloads.bf16_bits_from_f32(x32)
    _check_quantize(x, "k=%d %s" % (k, xdt))


def _gemv_q8(inp, q, d, bs, what):
    w = qtensor(inp)
    say("gemv_q8", what, inp["n"], inp["k"])
    y = qbn.quantized_gemv_q8(w, dev(q), dev(d), dev(bs))
    torch.cuda.synchronize()
    return y.cpu().numpy()


# k / 256 blocks per row reaches every launch case: 16, 8, 4 and 2 rows per
# wave (1, 2, 3-4 and 5-8 blocks), one wave per row with 1 to 4 blocks per
# lane (with idle slots for 12, 20, 43, 56), and the 64-block chunk loop
# (70 and 130 blocks); row counts leave ragged waves.
SHAPES = [(1, 256), (7, 256), (37, 512), (19, 768), (130, 1024), (33, 1280), (64, 2048), (21, 3072),
          (257, 4096), (29, 5120), (18, 8192), (11, 256 * 43), (9, 14336), (5, 16384), (3, 256 * 70),
          (2, 256 * 130)]


@pytest.mark.parametrize("n,k", SHAPES)
def test_gemv_q8_all_rows(n, k):
    inp = workloads.workload(6, n=n, k=k, seed=5000 + n + k)
    q, d, bs = oracle.q8_quantize(inp["x"])
    y = _gemv_q8(inp, q, d, bs, "shape")
    y_ref, s_ref = oracle.q4k_w4a8_rows(inp["data"], k, q, d, range(n))
    assert_within_tolerance(y, y_ref, s_ref, "gemv_q8 n=%d k=%d" % (n, k))


def test_gemv_q8_workload_full_size_end_to_end():
    """The bench workload at full size through both kernels: the device codes
    must equal the oracle's, then sampled rows of y must meet the bound."""
    inp = workloads.workload(6)
    n, k = inp["n"], inp["k"]
    q, d, bs = _check_quantize(inp["x"], "workload 6")
    w = qtensor(inp)
    say("gemv_q8 full workload 6", n, k)
    qd, dd, bd = qbn.quantize_q8(x_dev(inp["x"]))
    y = qbn.quantized_gemv_q8(w, qd, dd, bd).cpu().numpy()
    rng = np.random.default_rng(6)
    rows = np.unique(np.concatenate([rng.integers(0, n, 1500), np.arange(64), np.arange(n - 64, n)]))
    y_ref, s_ref = oracle.q4k_w4a8_rows(inp["data"], k, q, d, rows)
    assert_within_tolerance(y[rows], y_ref, s_ref, "gemv_q8 workload 6 sampled")


def test_gemv_q8_cancellation_is_exact():
    """Blocks with dmin = d and m_j = s_j * q for their single code q have every
    weight exactly zero (d s_j q - dmin m_j = 0), so y must be exactly zero,
    however large the two cancelling terms are."""
    n, k = 12, 1024
    nb = k // 256
    rng = np.random.default_rng(17)
    blocks = np.zeros((n, nb, 144), np.uint8)
    for r in range(n):
        for b in range(nb):
            qv = int(rng.integers(1, 16))
            s = [int(rng.integers(1, 63 // qv + 1)) for _ in range(8)]
            m = [sj * qv for sj in s]
            d = np.float16(2.0 ** int(rng.integers(-4, 9)))
            blk = blocks[r, b]
            blk[0:2] = np.array([d], np.float16).view(np.uint8)
            blk[2:4] = np.array([d], np.float16).view(np.uint8)
            blk[4:16] = oracle.q4k_pack_scales(s, m)
            blk[16:144] = qv | (qv << 4)
    inp = dict(fmt="q4_k", n=n, k=k, data=blocks, scales=None, scale2=1.0)
    W = oracle.dequant_rows(oracle.Q4_K, blocks, None, 1.0, k, range(n))
    assert (W == 0).all()
    x = (rng.standard_normal(k) * 1e3).astype(np.float32)
    q, d, bs = oracle.q8_quantize(x)
    y = _gemv_q8(inp, q, d, bs, "cancellation")
    assert (y == 0).all()


def test_gemv_q8_deterministic_and_empty():
    inp = workloads.workload(6, n=300, k=4096, seed=8)
    q, d, bs = oracle.q8_quantize(inp["x"])
    a = _gemv_q8(inp, q, d, bs, "run 1")
    b = _gemv_q8(inp, q, d, bs, "run 2")
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    say("gemv_q8 k = 0")
    w0 = qbn.QTensor("q4_k", 5, 0, torch.empty(5, 0, dtype=torch.uint8, device=DEV))
    y = torch.full((5,), 7.0, device=DEV)
    e = torch.empty(0, dtype=torch.int8, device=DEV)
    qbn.quantized_gemv_q8(w0, e, e.float(), e.int(), y)
    torch.cuda.synchronize()
    assert (y.cpu() == 0).all()
