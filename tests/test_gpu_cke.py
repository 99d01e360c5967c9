"""GPU parity of NVFP4 in CKE's split-half blocks (qbn format nvfp4_cke):
bulk dequantization bit-exact with the oracle (binary32 and bfloat16, both
output layouts), the decode GEMV within |y - y_ref| <= 1e-5 * sum|w x| + 1e-6
of the oracle's binary64 dot, the repack to and from plain NVFP4 bit-exact
with the oracle's packer, and the load-time NaN-subscale scan."""
import numpy as np
import pytest
import torch

import bit_block_quantized_nibble_amd as qbn
import oracle
import workloads
from gpu_util import (DEV, assert_bf16_bits_equal, assert_f32_bits_equal, assert_within_tolerance, dev, host_bits,
                      say, x_dev)

pytestmark = pytest.mark.gpu

SCALE2 = float(np.float32(0.01))


def _cke(rng, n, k, every_byte=False):
    blocks = workloads.cke_blocks(rng, n, k)
    if every_byte:  # subscales over every finite byte, zero and negative ones included
        sub = rng.integers(0, 256, size=(n, k // 64, 4)).astype(np.uint8)
        sub[(sub & 0x7F) == 0x7F] = 0x38
        blocks[:, :, :4] = sub
    return blocks


def _qt(blocks, n, k, scale2=SCALE2):
    return qbn.QTensor("nvfp4_cke", n, k, dev(blocks), scale2=scale2)


SHAPES = [(1, 64), (7, 192), (33, 4096), (130, 1024), (5, 64 * 200), (3, 8192), (9, 128), (17, 2048)]


@pytest.mark.parametrize("n,k", SHAPES)
def test_dequant_f32_bf16_both_layouts(n, k):
    rng = np.random.default_rng(n * 7 + k)
    blocks = _cke(rng, n, k, every_byte=True)
    want = oracle.dequant_rows(oracle.NVFP4_CKE, blocks, None, SCALE2, k, range(n))
    w = _qt(blocks, n, k)
    say("cke dequant", n, k)
    got = qbn.dequantize(w, dtype=torch.float32)
    got_kn = qbn.dequantize(w, dtype=torch.float32, layout="kn")
    got_bf = qbn.dequantize(w, dtype=torch.bfloat16)
    got_bf_kn = qbn.dequantize(w, dtype=torch.bfloat16, layout="kn")
    torch.cuda.synchronize()
    assert_f32_bits_equal(host_bits(got), want, "cke f32 nk")
    assert_f32_bits_equal(host_bits(got_kn), want.T, "cke f32 kn")
    assert_bf16_bits_equal(host_bits(got_bf), want, "cke bf16 nk")
    assert_bf16_bits_equal(host_bits(got_bf_kn), want.T, "cke bf16 kn")


@pytest.mark.parametrize("n,k", SHAPES)
@pytest.mark.parametrize("xdt", ["f32", "bf16"])
def test_gemv_shapes(n, k, xdt):
    rng = np.random.default_rng(n * 11 + k + (xdt == "bf16"))
    blocks = _cke(rng, n, k)
    x32 = workloads.x_f32(rng, k)
    x = x32 if xdt == "f32" else workloads.bf16_bits_from_f32(x32)
    say("cke gemv", n, k, xdt)
    y = qbn.quantized_gemv(_qt(blocks, n, k), x_dev(x))
    torch.cuda.synchronize()
    y_ref, s_ref = oracle.gemv_rows(oracle.NVFP4_CKE, blocks, None, SCALE2, k, x, range(n))
    assert_within_tolerance(y.cpu().numpy(), y_ref, s_ref, "cke n=%d k=%d %s" % (n, k, xdt))


def test_gemv_workload_full_size():
    """Workload 8 (4096 x 4096, bf16 activations), every output."""
    inp = workloads.workload(8)
    n, k = inp["n"], inp["k"]
    say("cke gemv full", n, k)
    y = qbn.quantized_gemv(_qt(inp["data"], n, k, inp["scale2"]), x_dev(inp["x"]))
    torch.cuda.synchronize()
    y_ref, s_ref = oracle.gemv_rows(oracle.NVFP4_CKE, inp["data"], None, inp["scale2"], k, inp["x"], range(n))
    assert_within_tolerance(y.cpu().numpy(), y_ref, s_ref, "cke full")


def test_gemv_deterministic_and_empty():
    rng = np.random.default_rng(3)
    n, k = 300, 4096
    blocks = _cke(rng, n, k)
    x = x_dev(workloads.x_bf16(rng, k))
    w = _qt(blocks, n, k)
    say("cke gemv twice")
    a = qbn.quantized_gemv(w, x)
    b = qbn.quantized_gemv(w, x)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    say("cke gemv k = 0")
    w0 = qbn.QTensor("nvfp4_cke", 16, 0, torch.empty(0, dtype=torch.uint8, device=DEV), scale2=SCALE2)
    y = torch.full((16,), 5.0, dtype=torch.float32, device=DEV)
    qbn.quantized_gemv(w0, torch.empty(0, dtype=torch.float32, device=DEV), y)
    torch.cuda.synchronize()
    assert (y.cpu() == 0).all()


def _adjacent(codes):
    return np.ascontiguousarray((codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8))


@pytest.mark.parametrize("n,k", [(1, 64), (5, 320), (64, 4096), (4096, 4096)])
def test_repack_both_directions(n, k):
    rng = np.random.default_rng(n + k)
    codes = rng.integers(0, 16, (n, k)).astype(np.uint8)
    scales = rng.integers(0, 256, (n, k // 16)).astype(np.uint8)
    want_blocks = oracle.cke_pack(codes, scales)
    src = qbn.QTensor("nvfp4", n, k, dev(_adjacent(codes)), dev(scales), scale2=SCALE2)
    say("cke repack", n, k)
    cke = qbn.repack(src, "nvfp4_cke")
    back = qbn.repack(cke, "nvfp4")
    torch.cuda.synchronize()
    assert np.array_equal(cke.data.cpu().numpy().reshape(want_blocks.shape), want_blocks)
    assert np.array_equal(back.data.cpu().numpy(), _adjacent(codes))
    assert np.array_equal(back.scales.cpu().numpy(), scales)
    assert cke.scale2 == SCALE2 and back.scale2 == SCALE2


def test_repack_then_gemv_matches_the_nvfp4_oracle():
    inp = workloads.workload(2, n=256, k=4096)
    n, k = inp["n"], inp["k"]
    src = qbn.QTensor("nvfp4", n, k, dev(inp["data"]), dev(inp["scales"]), scale2=inp["scale2"])
    say("cke repack + gemv", n, k)
    y = qbn.quantized_gemv(qbn.repack(src, "nvfp4_cke"), x_dev(inp["x"]))
    torch.cuda.synchronize()
    y_ref, s_ref = oracle.gemv_rows(oracle.NVFP4, inp["data"], inp["scales"], inp["scale2"], k, inp["x"], range(n))
    assert_within_tolerance(y.cpu().numpy(), y_ref, s_ref, "nvfp4 -> cke gemv")


@pytest.mark.parametrize("bad", [0x7F, 0xFF])
def test_validate_nan_subscale(bad):
    rng = np.random.default_rng(bad)
    n, k = 6, 256
    blocks = _cke(rng, n, k)
    say("cke validate clean")
    assert qbn.validate(_qt(blocks, n, k)) == -1
    # subscale j of block b of row r is logical index r * (k/16) + 4b + j
    for (r, b, j) in [(5, 3, 3), (2, 1, 0), (0, 0, 2)]:
        blocks[r, b, j] = bad
        say("cke validate", r, b, j)
        assert qbn.validate(_qt(blocks, n, k)) == r * (k // 16) + 4 * b + j
