"""GPU parity: qbn_quantized_gemv against the oracle's binary64 dot, element
by element, within |y - y_ref| <= 1e-5 * sum|w x| + 1e-6; exact where every
partial sum is representable; deterministic across runs."""
import numpy as np
import pytest
import torch

import bit_block_quantized_nibble_amd as qbn
import oracle
import workloads
from gpu_util import (DEV, ORACLE_FMT, assert_within_tolerance, dev, host_bits, qtensor, say, x_dev)

pytestmark = pytest.mark.gpu


def _bf16(x32):
    return workloads.bf16_bits_from_f32(x32)


def _run(inp, x_host, what):
    w = qtensor(inp)
    say("gemv", what, inp["fmt"], inp["n"], inp["k"], x_host.dtype)
    y = qbn.quantized_gemv(w, x_dev(x_host))
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _ref(inp, x_host, rows=None):
    rows = range(inp["n"]) if rows is None else rows
    return oracle.gemv_rows(ORACLE_FMT[inp["fmt"]], inp["data"], inp["scales"], inp["scale2"], inp["k"], x_host, rows)


# (workload recipe, n, k): fast paths (every chunk / block split), ragged row
# tails, and the generic kernels (k not a fast-path size)
SHAPES = [
    (1, 1, 32), (1, 67, 64), (1, 37, 1024), (1, 130, 2048), (1, 21, 4096), (1, 19, 8192), (1, 5, 96),
    (1, 3, 2080),
    (2, 41, 4096), (2, 9, 48), (2, 33, 1024), (2, 17, 8192), (2, 7, 16), (2, 70, 512),
    (3, 29, 4096), (3, 8, 256), (3, 31, 512), (3, 17, 1024), (3, 11, 2048), (3, 5, 768), (3, 3, 8192),
    (3, 2, 12288),
]


@pytest.mark.parametrize("c,n,k", SHAPES)
@pytest.mark.parametrize("xdt", ["f32", "bf16"])
def test_gemv_shapes(c, n, k, xdt):
    inp = workloads.workload(c, n=n, k=k, seed=900 + 7 * c + n)
    rng = np.random.default_rng(n * 31 + k)
    x32 = rng.standard_normal(k).astype(np.float32)
    x = x32 if xdt == "f32" else _bf16(x32)
    y = _run(inp, x, "shape")
    y_ref, s_ref = _ref(inp, x)
    assert_within_tolerance(y, y_ref, s_ref, "gemv %s n=%d k=%d x=%s" % (inp["fmt"], n, k, xdt))


@pytest.mark.parametrize("c", [1, 2, 3])
def test_gemv_workload_full_size(c):
    inp = workloads.workload(c)
    x = inp["x"]
    y = _run(inp, x, "full workload %d" % c)
    y_ref, s_ref = _ref(inp, x)
    worst = assert_within_tolerance(y, y_ref, s_ref, "workload %d" % c)
    say("workload %d worst error / bound = %.3g" % (c, worst))


@pytest.mark.parametrize("c", [1, 2, 3])
def test_gemv_deterministic(c):
    inp = workloads.workload(c, n=257, k=4096 if c != 1 else 1024, seed=77)
    w = qtensor(inp)
    xd = x_dev(inp["x"])
    say("gemv determinism", c)
    a = qbn.quantized_gemv(w, xd)
    b = qbn.quantized_gemv(w, xd)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(a), host_bits(b))


def test_gemv_mxfp4_dyadic_exact():
    # small-integer x and scales in [2^-4, 2^2]: every partial sum is exact in
    # binary32, so the GPU must equal the exact dot bit for bit
    rng = np.random.default_rng(12)
    for n, k in ((64, 1024), (33, 4096), (5, 160)):
        codes = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
        scales = (127 + rng.integers(-4, 3, (n, k // 32))).astype(np.uint8)
        x = rng.integers(-8, 9, k).astype(np.float32)
        inp = dict(fmt="mxfp4", n=n, k=k, data=codes, scales=scales, scale2=1.0)
        y = _run(inp, x, "dyadic")
        y_ref, _ = _ref(inp, x)
        assert np.array_equal(y.astype(np.float64), y_ref)


def test_gemv_page_dot_facts():
    # Four Bits, Three Contracts, section 2: the 4-weight row at scales 0.5 and
    # 0.125 gives -2 and -1.625, embedded in a full 32-block with x = 0 elsewhere
    w_row = [-1.0, 0.3, 0.9, 1.7]
    x = np.zeros(32, np.float32)
    x[:4] = [2.0, 1.0, -1.0, 0.5]
    for scale, e8, want in ((0.5, 126, -2.0), (0.125, 124, -1.625)):
        codes = [oracle.e2m1_nearest(v, scale) for v in w_row] + [0] * 28
        packed = np.array([[codes[2 * i] | (codes[2 * i + 1] << 4) for i in range(16)]], np.uint8)
        inp = dict(fmt="mxfp4", n=1, k=32, data=packed, scales=np.array([[e8]], np.uint8), scale2=1.0)
        assert _run(inp, x, "page fact")[0] == want
        assert _run(inp, _bf16(x), "page fact bf16")[0] == want


def test_gemv_q4k_cancelling_subblocks():
    # Sub-blocks whose every weight is exactly zero because gain*q == offset
    # (d = 1/64, s = 8, q = 8; dmin = 1/32, m = 32): the tolerance is then
    # relative to the remaining terms only, which a kernel that factors the
    # offset out of the sum cannot meet.
    rng = np.random.default_rng(14)
    n, k = 16, 4096
    nb = k // 256
    blocks = workloads.q4k_weights(rng, n, k)
    sc = oracle.q4k_pack_scales([8] * 8, [32] * 8)
    for r in range(n):
        for b in range(nb):
            if (r + b) % 3:
                blk = blocks[r, b]
                blk[0:2] = np.array([1 / 64], np.float16).view(np.uint8)
                blk[2:4] = np.array([1 / 32], np.float16).view(np.uint8)
                blk[4:16] = sc
                blk[16:144] = 0x88
    inp = dict(fmt="q4_k", n=n, k=k, data=blocks, scales=None, scale2=1.0)
    x = (rng.standard_normal(k) * 100).astype(np.float32)
    y = _run(inp, x, "q4k cancel")
    y_ref, s_ref = _ref(inp, x)
    assert_within_tolerance(y, y_ref, s_ref, "q4k cancelling sub-blocks")


def test_gemv_empty_and_zero_k():
    w = qbn.QTensor("mxfp4", 0, 64, torch.empty(0, 32, dtype=torch.uint8, device=DEV),
                    torch.empty(0, 2, dtype=torch.uint8, device=DEV))
    y = qbn.quantized_gemv(w, torch.zeros(64, device=DEV))
    assert y.numel() == 0
    w = qbn.QTensor("nvfp4", 5, 0, torch.empty(5, 0, dtype=torch.uint8, device=DEV),
                    torch.empty(5, 0, dtype=torch.uint8, device=DEV), scale2=1.0)
    y = torch.full((5,), 7.0, device=DEV)
    say("gemv k = 0")
    qbn.quantized_gemv(w, torch.zeros(16, device=DEV), y)
    torch.cuda.synchronize()
    assert (y.cpu() == 0).all()
