"""GPU parity of the prefill GEMM straight from the int4 layouts
(qbn_quantized_gemm with GPTQ4, AWQ4 or Q4_0 weights, bf16 activations)
against the oracle's binary64 entries: a float32 output within
|y - y_ref| <= 1e-5 * sum|w x| + 1e-6, a bf16 output inside
[RNE(y_ref - T), RNE(y_ref + T)] (rounding to nearest is monotone). Shapes
cover one and several 128 x 128 tiles, ragged m and n, k with a half k-tile
tail, groups of 32 up to all of k, the 256 x 128 kernel's cases, and
the 2048 x 11008 x 4096 layer."""
import numpy as np
import pytest
import torch

import bit_block_quantized_nibble_amd as qbn
import oracle
import workloads
from gpu_util import DEV, dev, host_bits, say

pytestmark = pytest.mark.gpu


def _bf16_value(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32).astype(np.float64)


def _qt(fmt, inp, K, N, g):
    if fmt == "q4_0":
        return qbn.QTensor("q4_0", N, K, dev(inp["q4_0"]))
    data = inp["gptq"] if fmt == "gptq4" else inp["awq"]
    return qbn.QTensor(fmt, N, K, dev(data), dev(inp["scales"].view(np.uint16)), dev(inp["zeros"]), group=g)


def _ref(fmt, inp, g, ms, ns):
    data = inp["q4_0"] if fmt == "q4_0" else (inp["gptq"] if fmt == "gptq4" else inp["awq"])
    return oracle.int4_gemm_entries(fmt, data, inp["scales"], inp["zeros"], g, inp["X"], ms, ns)


def _check(Y, y_ref, s_ref, ms, ns, what):
    T = 1e-5 * s_ref + 1e-6
    if Y.dtype == torch.float32:
        got = Y.cpu().numpy().astype(np.float64)[ms, ns]
        bad = ~(np.abs(got - y_ref) <= T)
        lo = hi = None
    else:
        got = _bf16_value(host_bits(Y).reshape(Y.shape)[ms, ns])
        lo = _bf16_value(oracle.bf16_rne_array((y_ref - T).astype(np.float32)))
        hi = _bf16_value(oracle.bf16_rne_array((y_ref + T).astype(np.float32)))
        bad = ~((lo <= got) & (got <= hi))
    if bad.any():
        i = int(np.argwhere(bad)[0][0])
        raise AssertionError("%s: %d of %d entries out of tolerance; first (m=%d, n=%d): got %r ref %r" % (
            what, int(bad.sum()), bad.size, ms[i], ns[i], got[i], y_ref[i]))


def _inputs(seed, M, N, K, g):
    """Workload 9's recipe at a small shape, with the group size overridden."""
    rng = np.random.default_rng(seed)
    inp = dict(gptq=rng.integers(0, 2**32, size=(K // 8, N), dtype=np.uint32),
               awq=rng.integers(0, 2**32, size=(K, N // 8 if N % 8 == 0 else 1), dtype=np.uint32),
               scales=rng.uniform(1e-3, 1e-2, size=(K // g, N)).astype(np.float16),
               zeros=rng.integers(0, 16, size=(K // g, N)).astype(np.uint8),
               q4_0=workloads.q4_0_blocks(rng, N, K))
    inp["X"] = workloads.bf16_bits_from_f32(rng.standard_normal((M, K)).astype(np.float32))
    return inp


# n % 8 != 0 (70, 130) takes the element-load path for GPTQ; groups of 32, 96
# and 160 the per-32-k rescale; a group that is a multiple of 64 the
# per-group rescale (one, three and five k-tiles in three shapes). With
# k % 64 == 0 and n % 8 == 0, groups of 32, 96 and 160 take GPTQ's buffer
# path, where a k-tile may span two groups and the lanes in the second add
# one group row.
SHAPES = [(1, 40, 96, 32), (37, 72, 128, 64), (130, 264, 256, 128), (256, 256, 1024, 128), (5, 136, 4096, 4096),
          (129, 128, 160, 32), (64, 8, 2048, 256), (200, 520, 512, 512), (33, 70, 128, 32), (20, 64, 192, 96),
          (140, 130, 384, 128), (3, 96, 576, 96), (9, 128, 64, 64), (24, 64, 192, 64), (70, 200, 320, 64),
          (48, 136, 256, 32), (70, 200, 640, 160)]


@pytest.mark.parametrize("fmt", ["gptq4", "awq4", "q4_0"])
@pytest.mark.parametrize("M,N,K,g", SHAPES)
@pytest.mark.parametrize("ydt", ["bf16", "f32"])
def test_int4_gemm_all_entries(fmt, M, N, K, g, ydt):
    if fmt == "awq4" and N % 8:
        pytest.skip("AWQ packs eight columns per word: n % 8 == 0")
    inp = _inputs(M * 7 + N + K + g, M, N, K, g)
    w = _qt(fmt, inp, K, N, g)
    X = dev(inp["X"]).view(torch.bfloat16)
    Y = torch.empty((M, N), dtype=torch.bfloat16 if ydt == "bf16" else torch.float32, device=DEV)
    say("int4 gemm", fmt, M, N, K, g, ydt)
    qbn.quantized_gemm(w, X, Y)
    torch.cuda.synchronize()
    ms, ns = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    ms, ns = ms.ravel(), ns.ravel()
    y_ref, s_ref = _ref(fmt, inp, g, ms, ns)
    _check(Y, y_ref, s_ref, ms, ns, "%s %dx%dx%d g=%d %s" % (fmt, M, N, K, g, ydt))


# m >= 256, n >= 128 and k % 64 == 0 (GPTQ / AWQ: a group that is a multiple
# of 64; GPTQ: n even) run the 256 x 128 kernel: one k-tile (k = 64); an odd
# number of k-tiles (the two-tile unrolled loop's tail) with one group per
# k-tile; groups of two k-tiles; group sizes known only at run time (192,
# 256, all of k); m just past one row tile; n even but not a multiple of 8
# (the last column tile reads column n - 1 in place of the missing ones);
# groups that are odd multiples of 32 (32, 96, 160: each 32-k half of a
# k-tile scaled on its own, a k-tile spanning two groups). Q4_0 ignores the
# group size (its blocks are 32 long).
SHAPES_256 = [(256, 128, 64, 64), (300, 264, 512, 128), (520, 200, 192, 64), (777, 130, 384, 192),
              (257, 1000, 1024, 256), (512, 136, 4096, 4096), (256, 136, 320, 64), (384, 250, 1152, 128),
              (300, 264, 512, 32), (520, 200, 384, 96), (256, 136, 640, 160), (777, 130, 192, 32)]


@pytest.mark.parametrize("fmt", ["gptq4", "awq4", "q4_0"])
@pytest.mark.parametrize("M,N,K,g", SHAPES_256)
@pytest.mark.parametrize("ydt", ["bf16", "f32"])
def test_int4_gemm_256_row_tiles(fmt, M, N, K, g, ydt):
    if fmt == "awq4" and N % 8:
        pytest.skip("AWQ packs eight columns per word: n % 8 == 0")
    inp = _inputs(M * 5 + N * 3 + K + g, M, N, K, g)
    w = _qt(fmt, inp, K, N, g)
    X = dev(inp["X"]).view(torch.bfloat16)
    Y = torch.empty((M, N), dtype=torch.bfloat16 if ydt == "bf16" else torch.float32, device=DEV)
    say("int4 gemm 256-row tiles", fmt, M, N, K, g, ydt)
    qbn.quantized_gemm(w, X, Y)
    torch.cuda.synchronize()
    ms, ns = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    ms, ns = ms.ravel(), ns.ravel()
    y_ref, s_ref = _ref(fmt, inp, g, ms, ns)
    _check(Y, y_ref, s_ref, ms, ns, "%s %dx%dx%d g=%d %s" % (fmt, M, N, K, g, ydt))


@pytest.mark.parametrize("fmt", ["gptq4", "awq4", "q4_0"])
def test_int4_gemm_256_row_tiles_strided(fmt):
    """The 256 x 128 kernel with ldx > k and ldy > n."""
    M, N, K, g = 300, 136, 256, 128
    inp = _inputs(41, M, N, K, g)
    w = _qt(fmt, inp, K, N, g)
    Xp = torch.zeros((M, K + 40), dtype=torch.bfloat16, device=DEV)
    Xp[:, :K] = dev(inp["X"]).view(torch.bfloat16)
    Yp = torch.full((M, N + 6), 7.0, dtype=torch.float32, device=DEV)
    say("int4 gemm 256-row tiles strided", fmt)
    qbn.quantized_gemm(w, Xp[:, :K], Yp[:, :N])
    torch.cuda.synchronize()
    ms, ns = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    ms, ns = ms.ravel(), ns.ravel()
    y_ref, s_ref = _ref(fmt, inp, g, ms, ns)
    _check(Yp[:, :N], y_ref, s_ref, ms, ns, fmt + " 256-row strided")
    assert (Yp[:, N:].cpu() == 7.0).all()


@pytest.mark.parametrize("fmt", ["gptq4", "awq4"])
@pytest.mark.parametrize("M,zofs", [(40, 1), (300, 1), (300, 2)])
def test_int4_gemm_misaligned_codes_and_zeros(fmt, M, zofs):
    """Codes 4 bytes past a 16-byte boundary and zero points 1 or 2 bytes past
    an 8-byte one: the element-load path (m = 40), and the 256 x 128 kernel,
    which takes dword-aligned codes and (AWQ) 2-byte aligned zero points
    (m = 300; AWQ with zofs = 1 goes to the element-load path)."""
    N, K, g = 136, 256, 64
    inp = _inputs(17 + M + zofs, M, N, K, g)
    data = inp["gptq"] if fmt == "gptq4" else inp["awq"]
    dd = torch.zeros(data.size + 1, dtype=torch.int32, device=DEV)
    dd[1:] = dev(data).flatten()
    zd = torch.zeros(inp["zeros"].size + zofs, dtype=torch.uint8, device=DEV)
    zd[zofs:] = dev(inp["zeros"]).flatten()
    w = qbn.QTensor(fmt, N, K, dd[1:], dev(inp["scales"].view(np.uint16)), zd[zofs:], group=g)
    X = dev(inp["X"]).view(torch.bfloat16)
    say("int4 gemm misaligned", fmt, M, zofs)
    Y = torch.empty((M, N), dtype=torch.float32, device=DEV)
    qbn.quantized_gemm(w, X, Y)
    torch.cuda.synchronize()
    ms, ns = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    ms, ns = ms.ravel(), ns.ravel()
    y_ref, s_ref = _ref(fmt, inp, g, ms, ns)
    _check(Y, y_ref, s_ref, ms, ns, "%s misaligned m=%d zofs=%d" % (fmt, M, zofs))


def test_int4_gemm_strided_activations_and_output():
    """ldx > k and ldy > n: rows are read and written at their strides; the
    padding columns of Y are left untouched."""
    M, N, K, g = 70, 96, 256, 64
    inp = _inputs(5, M, N, K, g)
    w = _qt("gptq4", inp, K, N, g)
    Xp = torch.zeros((M, K + 24), dtype=torch.bfloat16, device=DEV)
    Xp[:, :K] = dev(inp["X"]).view(torch.bfloat16)
    Yp = torch.full((M, N + 10), 7.0, dtype=torch.float32, device=DEV)
    say("int4 gemm strided")
    qbn.quantized_gemm(w, Xp[:, :K], Yp[:, :N])
    torch.cuda.synchronize()
    ms, ns = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    ms, ns = ms.ravel(), ns.ravel()
    y_ref, s_ref = _ref("gptq4", inp, g, ms, ns)
    _check(Yp[:, :N], y_ref, s_ref, ms, ns, "strided")
    assert (Yp[:, N:].cpu() == 7.0).all()


@pytest.mark.parametrize("fmt", ["gptq4", "awq4", "q4_0"])
def test_int4_gemm_workload_full_size(fmt):
    """Workload 9 (X 2048 x 4096 bf16, the 4096 x 11008 layer): every entry of
    four whole rows and four whole columns, and 4000 random entries."""
    inp = workloads.workload(9)
    M, N, K, g = inp["M"], inp["N"], inp["K"], inp["group"]
    w = _qt(fmt, inp, K, N, g)
    X = dev(inp["X"]).view(torch.bfloat16)
    say("int4 gemm full", fmt, M, N, K)
    Y = qbn.quantized_gemm(w, X)
    torch.cuda.synchronize()
    rng = np.random.default_rng(99)
    rows = [0, 1, 1027, M - 1]
    cols = [0, 127, 5000, N - 1]
    ms = np.concatenate([np.repeat(rows, N), np.tile(np.arange(M), len(cols)), rng.integers(0, M, 4000)])
    ns = np.concatenate([np.tile(np.arange(N), len(rows)), np.repeat(cols, M), rng.integers(0, N, 4000)])
    y_ref, s_ref = _ref(fmt, inp, g, ms, ns)
    _check(Y, y_ref, s_ref, ms, ns, fmt + " full")


def test_int4_gemm_deterministic_and_empty():
    M, N, K, g = 150, 136, 512, 128
    inp = _inputs(3, M, N, K, g)
    w = _qt("awq4", inp, K, N, g)
    X = dev(inp["X"]).view(torch.bfloat16)
    say("int4 gemm twice")
    a = qbn.quantized_gemm(w, X)
    b = qbn.quantized_gemm(w, X)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    say("int4 gemm k = 0")
    w0 = qbn.QTensor("gptq4", 16, 0, torch.empty(0, 16, dtype=torch.int32, device=DEV),
                     torch.empty(0, 16, dtype=torch.int16, device=DEV), torch.empty(0, 16, dtype=torch.uint8,
                                                                                     device=DEV), group=128)
    Y = torch.full((4, 16), 3.0, dtype=torch.float32, device=DEV)
    qbn.quantized_gemm(w0, torch.empty((4, 0), dtype=torch.bfloat16, device=DEV), Y)
    torch.cuda.synchronize()
    assert (Y.cpu() == 0).all()
