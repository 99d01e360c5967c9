"""GPU parity: qbn_dequantize is bit-exact with the oracle for all six
formats, both output dtypes and both layouts, including exhaustive sweeps of
every code and scale encoding."""
import numpy as np
import pytest
import torch

import bit_block_quantized_nibble_amd as qbn
import oracle
import workloads
from gpu_util import (DEV, ORACLE_FMT, assert_bf16_bits_equal, assert_f32_bits_equal, dev, host_bits, qtensor,
                      say)

pytestmark = pytest.mark.gpu

LAYOUTS = ["nk", "kn"]
DTYPES = [torch.float32, torch.bfloat16]


def _check_all(w: qbn.QTensor, ref_nk: np.ndarray, what: str):
    for layout in LAYOUTS:
        for dt in DTYPES:
            say("dequant", what, layout, dt)
            out = qbn.dequantize(w, dtype=dt, layout=layout)
            torch.cuda.synchronize()
            ref = ref_nk if layout == "nk" else np.ascontiguousarray(ref_nk.T)
            if dt == torch.float32:
                assert_f32_bits_equal(host_bits(out), ref, "%s %s f32" % (what, layout))
            else:
                assert_bf16_bits_equal(host_bits(out), ref, "%s %s bf16" % (what, layout))


def _pack_low_even(codes):
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def test_mxfp4_every_code_and_scale_byte():
    n, k = 256, 64
    codes = _pack_low_even(np.tile(np.arange(16, dtype=np.uint8), (n, k // 16)))
    scales = np.repeat(np.arange(256, dtype=np.uint8)[:, None], k // 32, axis=1)
    scales[:, 1] = scales[::-1, 0]
    w = qbn.QTensor("mxfp4", n, k, dev(codes), dev(scales))
    ref = oracle.dequant_rows(oracle.MXFP4, codes, scales, 1.0, k, range(n))
    _check_all(w, ref, "mxfp4 sweep")


@pytest.mark.parametrize("scale2", [0.01, 0.25, 3.0e-39, 1.0e30])
def test_nvfp4_every_scale_byte_and_code(scale2):
    # all 256 E4M3FN bytes (0x7F / 0xFF decode to NaN) x all 16 codes
    n, k = 256, 32
    codes = _pack_low_even(np.tile(np.arange(16, dtype=np.uint8), (n, 2)))
    scales = np.stack([np.arange(256, dtype=np.uint8), np.arange(256, dtype=np.uint8)[::-1]], axis=1)
    s2 = float(np.float32(scale2))
    w = qbn.QTensor("nvfp4", n, k, dev(codes), dev(np.ascontiguousarray(scales)), scale2=s2)
    ref = oracle.dequant_rows(oracle.NVFP4, codes, scales, s2, k, range(n))
    _check_all(w, ref, "nvfp4 sweep scale2=%g" % s2)


def _q4k_blocks_wide_range(rng, n, nb):
    blocks = np.zeros((n, nb, 144), np.uint8)
    d = (rng.uniform(-1, 1, (n, nb)) * 2.0 ** rng.integers(-24, 14, (n, nb))).astype(np.float16)
    dmin = (rng.uniform(-1, 1, (n, nb)) * 2.0 ** rng.integers(-24, 14, (n, nb))).astype(np.float16)
    blocks[..., 0:2] = d.view(np.uint8).reshape(n, nb, 2)
    blocks[..., 2:4] = dmin.view(np.uint8).reshape(n, nb, 2)
    blocks[..., 4:144] = rng.integers(0, 256, (n, nb, 140), dtype=np.uint8)
    return blocks


def test_q4k_wide_range_blocks():
    rng = np.random.default_rng(31)
    n, k = 24, 1024
    blocks = _q4k_blocks_wide_range(rng, n, k // 256)
    w = qbn.QTensor("q4_k", n, k, dev(blocks))
    ref = oracle.dequant_rows(oracle.Q4_K, blocks, None, 1.0, k, range(n))
    _check_all(w, ref, "q4_k wide")


def test_q4_0_every_d_value():
    rng = np.random.default_rng(32)
    n, k = 512, 4096  # 65536 blocks, one per fp16 bit pattern
    blocks = np.zeros((n * (k // 32), 18), np.uint8)
    blocks[:, 0:2] = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.uint8).reshape(-1, 2)
    blocks[:, 2:] = rng.integers(0, 256, (blocks.shape[0], 16), dtype=np.uint8)
    blocks = blocks.reshape(n, k // 32, 18)
    w = qbn.QTensor("q4_0", n, k, dev(blocks))
    ref = oracle.dequant_rows(oracle.Q4_0, blocks, None, 1.0, k, range(n))
    _check_all(w, ref, "q4_0 all d")


@pytest.mark.parametrize("c,n,k", [(1, 37, 1024), (2, 41, 4096), (2, 9, 48), (3, 13, 2048)])
def test_workload_recipes_small(c, n, k):
    inp = workloads.workload(c, n=n, k=k, seed=500 + c)
    w = qtensor(inp)
    ref = oracle.dequant_rows(ORACLE_FMT[inp["fmt"]], inp["data"], inp["scales"], inp["scale2"], k, range(n))
    _check_all(w, ref, "workload %d small" % c)


@pytest.mark.parametrize("c", [1, 2, 3])
def test_workload_full_size_f32(c):
    inp = workloads.workload(c)
    n, k = inp["n"], inp["k"]
    w = qtensor(inp)
    say("dequant full workload", c, n, k)
    out = qbn.dequantize(w, dtype=torch.float32, layout="nk")
    torch.cuda.synchronize()
    rows = np.arange(n) if c != 3 else np.unique(np.concatenate([np.arange(0, n, 37), [n - 1]]))
    ref = oracle.dequant_rows(ORACLE_FMT[inp["fmt"]], inp["data"], inp["scales"], inp["scale2"], k, rows)
    assert_f32_bits_equal(host_bits(out).reshape(n, k)[rows], ref, "workload %d full" % c)


def _affine_ref(q, scales, zeros, group):
    return oracle.affine_dequant(q, scales.view(np.uint16), zeros, group)  # [K][N]


@pytest.mark.parametrize("K,N,g", [(256, 96, 64), (128, 40, 128), (64, 8, 8)])
def test_gptq_awq_random(K, N, g):
    rng = np.random.default_rng(K + N + g)
    q = rng.integers(0, 16, (K, N)).astype(np.uint8)
    scales = rng.uniform(-0.02, 0.02, (K // g, N)).astype(np.float16)
    zeros = rng.integers(0, 16, (K // g, N)).astype(np.uint8)
    ref_kn = _affine_ref(q, scales, zeros, g)
    gp = qbn.QTensor("gptq4", N, K, dev(oracle.gptq_pack(q)), dev(scales.view(np.uint16)), dev(zeros), group=g)
    _check_all(gp, np.ascontiguousarray(ref_kn.T), "gptq %dx%d g%d" % (K, N, g))
    if N % 8 == 0:
        aw = qbn.QTensor("awq4", N, K, dev(oracle.awq_pack(q)), dev(scales.view(np.uint16)), dev(zeros), group=g)
        _check_all(aw, np.ascontiguousarray(ref_kn.T), "awq %dx%d g%d" % (K, N, g))


def test_gptq_awq_probes():
    K, N, g = 256, 256, 128
    pat, rand, full = workloads.layout_probes(K, N)
    scales = np.full((K // g, N), 1.0, np.float16)
    zeros = np.zeros((K // g, N), np.uint8)
    for name, probe in (("patterned", pat), ("random", rand), ("all-15", full)):
        ref = np.ascontiguousarray(_affine_ref(probe, scales, zeros, g).T)
        gp = qbn.QTensor("gptq4", N, K, dev(oracle.gptq_pack(probe)), dev(scales.view(np.uint16)), dev(zeros),
                         group=g)
        aw = qbn.QTensor("awq4", N, K, dev(oracle.awq_pack(probe)), dev(scales.view(np.uint16)), dev(zeros), group=g)
        _check_all(gp, ref, "gptq probe " + name)
        _check_all(aw, ref, "awq probe " + name)


def test_workload5_gptq_to_bf16_full():
    inp = workloads.workload(5)
    K, N, g = inp["K"], inp["N"], inp["group"]
    w = qtensor(inp)
    say("dequant workload 5 gptq -> bf16 [K][N]")
    out = qbn.dequantize(w, dtype=torch.bfloat16, layout="kn")
    torch.cuda.synchronize()
    q = oracle.gptq_unpack(inp["qweight"])
    ref = _affine_ref(q, inp["scales"], inp["zeros"], g)
    assert_bf16_bits_equal(host_bits(out), ref, "workload 5 dequant")
