"""GPU parity of the decode GEMV over the integer int4 layouts (Q4_0, GPTQ4,
AWQ4) through qbn_quantized_gemv: every output within |y - y_ref| <= 1e-5 *
sum|w x| + 1e-6 of the oracle's compensated binary64 dot of the dequantized
weights, at shapes that reach the vector and element paths, ragged column
counts, several group sizes, and the full 4096 x 11008 layer."""
import numpy as np
import pytest
import torch

import bit_block_quantized_nibble_amd as qbn
import oracle
import workloads
from gpu_util import DEV, assert_within_tolerance, dev, host_bits, say, x_dev

pytestmark = pytest.mark.gpu


def _affine(rng, fmt, K, N, g):
    if fmt == "gptq4":
        data = rng.integers(0, 2**32, size=(K // 8, N), dtype=np.uint32)
    else:
        data = rng.integers(0, 2**32, size=(K, N // 8), dtype=np.uint32)
    s = rng.uniform(1e-3, 1e-2, size=(K // g, N)).astype(np.float16)
    z = rng.integers(0, 16, size=(K // g, N)).astype(np.uint8)
    return data, s, z


def _run_affine(fmt, data, s, z, K, N, g, x, offset=False):
    if offset:  # misaligned views: the element-load path
        dd = torch.zeros(data.size + 1, dtype=torch.int32, device=DEV)
        dd[1:] = dev(data).flatten()
        sd = torch.zeros(s.size + 1, dtype=torch.int16, device=DEV)
        sd[1:] = dev(s.view(np.uint16)).flatten()
        zd = torch.zeros(z.size + 1, dtype=torch.uint8, device=DEV)
        zd[1:] = dev(z).flatten()
        w = qbn.QTensor(fmt, N, K, dd[1:], sd[1:], zd[1:], group=g)
    else:
        w = qbn.QTensor(fmt, N, K, dev(data), dev(s.view(np.uint16)), dev(z), group=g)
    say("gemv", fmt, "K", K, "N", N, "g", g, "x", x.dtype, "offset" if offset else "")
    y = qbn.quantized_gemv(w, x_dev(x))
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("fmt", ["gptq4", "awq4"])
@pytest.mark.parametrize("K,N,g", [(256, 64, 128), (512, 40, 32), (1024, 264, 64), (128, 8, 128),
                                   (4096, 1000, 128), (2048, 96, 1024), (8, 16, 8)])
@pytest.mark.parametrize("xdt", ["f32", "bf16"])
def test_affine_gemv_shapes(fmt, K, N, g, xdt):
    if fmt == "awq4" and N % 8:
        pytest.skip("AWQ packs eight columns per word: n % 8 == 0")
    rng = np.random.default_rng(K + 3 * N + g)
    data, s, z = _affine(rng, fmt, K, N, g)
    x32 = workloads.x_f32(rng, K)
    x = x32 if xdt == "f32" else workloads.bf16_bits_from_f32(x32)
    y = _run_affine(fmt, data, s, z, K, N, g, x)
    y_ref, s_ref = oracle.int4_gemv(fmt, data, s, z, g, x, range(N))
    assert_within_tolerance(y, y_ref, s_ref, "%s K=%d N=%d g=%d %s" % (fmt, K, N, g, xdt))


# GPTQ in the vector layout deals its n / 8 column groups over up to 256
# workgroups: 257 groups (one workgroup takes two), 513 (two or three each),
# 2050 (more than 8 per workgroup would be needed: 257 workgroups of 7 or 8),
# groups of 8 (rounds of one 8-row step) and k shorter than one round per
# slice.
@pytest.mark.parametrize("K,N,g", [(256, 2056, 64), (1024, 4104, 128), (512, 16400, 128), (64, 2064, 8),
                                   (4096, 3000, 4096), (96, 2048, 32)])
@pytest.mark.parametrize("xdt", ["f32", "bf16"])
def test_gptq_gemv_column_groups_per_workgroup(K, N, g, xdt):
    rng = np.random.default_rng(K + 7 * N + g)
    data, s, z = _affine(rng, "gptq4", K, N, g)
    x32 = workloads.x_f32(rng, K)
    x = x32 if xdt == "f32" else workloads.bf16_bits_from_f32(x32)
    y = _run_affine("gptq4", data, s, z, K, N, g, x)
    y_ref, s_ref = oracle.int4_gemv("gptq4", data, s, z, g, x, range(N))
    assert_within_tolerance(y, y_ref, s_ref, "gptq4 K=%d N=%d g=%d %s" % (K, N, g, xdt))


@pytest.mark.parametrize("fmt", ["gptq4", "awq4"])
def test_affine_gemv_misaligned_buffers(fmt):
    rng = np.random.default_rng(5)
    K, N, g = 512, 48, 64
    data, s, z = _affine(rng, fmt, K, N, g)
    x = workloads.x_f32(rng, K)
    a = _run_affine(fmt, data, s, z, K, N, g, x)
    b = _run_affine(fmt, data, s, z, K, N, g, x, offset=True)
    y_ref, s_ref = oracle.int4_gemv(fmt, data, s, z, g, x, range(N))
    assert_within_tolerance(b, y_ref, s_ref, fmt + " element loads")
    assert_within_tolerance(a, y_ref, s_ref, fmt + " vector loads")


# k = 32 * 500: past the activation staging buffer (activations read from global memory)
@pytest.mark.parametrize("n,k", [(1, 32), (7, 96), (33, 4096), (9, 160), (130, 1024), (5, 32 * 200), (11, 32 * 500)])
@pytest.mark.parametrize("xdt", ["f32", "bf16"])
def test_q4_0_gemv_shapes(n, k, xdt):
    rng = np.random.default_rng(n * 5 + k)
    blocks = workloads.q4_0_blocks(rng, n, k)
    x32 = workloads.x_f32(rng, k)
    x = x32 if xdt == "f32" else workloads.bf16_bits_from_f32(x32)
    w = qbn.QTensor("q4_0", n, k, dev(blocks))
    say("gemv q4_0", n, k, xdt)
    y = qbn.quantized_gemv(w, x_dev(x))
    torch.cuda.synchronize()
    y_ref, s_ref = oracle.gemv_rows(oracle.Q4_0, blocks, None, 1.0, k, x, range(n))
    assert_within_tolerance(y.cpu().numpy(), y_ref, s_ref, "q4_0 n=%d k=%d %s" % (n, k, xdt))


@pytest.mark.parametrize("fmt", ["gptq4", "awq4", "q4_0"])
def test_int4_gemv_workload_full_size(fmt):
    """The 4096 x 11008 layer, every output."""
    inp = workloads.workload(7)
    K, N, g = inp["K"], inp["N"], inp["group"]
    x = inp["x"]
    if fmt == "q4_0":
        w = qbn.QTensor("q4_0", N, K, dev(inp["q4_0"]))
        say("gemv q4_0 full", N, K)
        y = qbn.quantized_gemv(w, x_dev(x))
        torch.cuda.synchronize()
        y_ref, s_ref = oracle.gemv_rows(oracle.Q4_0, inp["q4_0"], None, 1.0, K, x, range(N))
    else:
        data = inp["gptq"] if fmt == "gptq4" else inp["awq"]
        y = torch.from_numpy(_run_affine(fmt, data, inp["scales"], inp["zeros"], K, N, g, x))
        y_ref, s_ref = oracle.int4_gemv(fmt, data, inp["scales"], inp["zeros"], g, x, range(N))
    assert_within_tolerance(y.cpu().numpy() if torch.is_tensor(y) else y, y_ref, s_ref, fmt + " full layer")


def test_int4_gemv_deterministic_and_empty():
    rng = np.random.default_rng(9)
    K, N, g = 1024, 256, 128
    data, s, z = _affine(rng, "gptq4", K, N, g)
    x = workloads.x_f32(rng, K)
    a = _run_affine("gptq4", data, s, z, K, N, g, x)
    b = _run_affine("gptq4", data, s, z, K, N, g, x)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    say("gemv gptq4 k = 0")
    w0 = qbn.QTensor("gptq4", 16, 0, torch.empty(0, 16, dtype=torch.int32, device=DEV),
                     torch.empty(0, 16, dtype=torch.int16, device=DEV), torch.empty(0, 16, dtype=torch.uint8,
                                                                                     device=DEV), group=128)
    y = torch.full((16,), 5.0, dtype=torch.float32, device=DEV)
    qbn.quantized_gemv(w0, torch.empty(0, dtype=torch.float32, device=DEV), y)
    torch.cuda.synchronize()
    assert (y.cpu() == 0).all()
