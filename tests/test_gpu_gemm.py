"""GPU parity: qbn_quantized_gemm (MXFP4 weights, bf16 activations and
output) against the oracle's binary64 entries. A bf16 output y passes when
RNE_bf16(y_ref - T) <= y <= RNE_bf16(y_ref + T), T = 1e-5 * sum|w x| + 1e-6:
rounding to nearest is monotone, so any binary32 result within T of the exact
value rounds into this band. Inputs whose partial sums are all exact must
match bit for bit."""
import os
from concurrent.futures import ThreadPoolExecutor

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


def _band(y_ref, s_ref):
    T = 1e-5 * s_ref + 1e-6
    lo = oracle.bf16_rne_array((y_ref - T).astype(np.float32))
    hi = oracle.bf16_rne_array((y_ref + T).astype(np.float32))
    return _bf16_value(lo), _bf16_value(hi)


def _run(inp, what):
    n, k, m = inp["n"], inp["k"], inp["m"]
    w = qbn.QTensor("mxfp4", n, k, dev(inp["data"]), dev(inp["scales"]))
    X = dev(inp["X"]).view(torch.bfloat16)
    say("gemm", what, m, n, k)
    Y = qbn.quantized_gemm(w, X)
    torch.cuda.synchronize()
    return host_bits(Y).reshape(m, n)


def _oracle_entries(inp, ms, ns):
    """The oracle's entries, split over the host's cores (each call releases
    the interpreter lock while the C oracle runs)."""
    ms, ns = np.asarray(ms), np.asarray(ns)
    workers = max(1, min(16, os.cpu_count() or 1))
    parts = [p for p in np.array_split(np.arange(ms.size), 4 * workers) if p.size]
    with ThreadPoolExecutor(workers) as ex:
        res = list(ex.map(lambda p: oracle.gemm_entries(oracle.MXFP4, inp["data"], inp["scales"], 1.0, inp["k"],
                                                        inp["X"], ms[p], ns[p]), parts))
    return np.concatenate([r[0] for r in res]), np.concatenate([r[1] for r in res])


def _check_entries(inp, Ybits, ms, ns, what):
    y_ref, s_ref = _oracle_entries(inp, ms, ns)
    got = _bf16_value(Ybits[ms, ns])
    lo, hi = _band(y_ref, s_ref)
    bad = ~((lo <= got) & (got <= hi))
    if bad.any():
        i = int(np.argwhere(bad)[0][0])
        raise AssertionError("%s: %d of %d entries outside the band; first (m=%d, n=%d): got %r, ref %r, band [%r, %r]"
                             % (what, int(bad.sum()), bad.size, ms[i], ns[i], got[i], y_ref[i], lo[i], hi[i]))


# Shapes reach every path: the 128 x 128 kernel (m or n below 256), the
# 256 x 256 kernel's edge tiles (ragged m / n, or k not a multiple of 64),
# its per-k-tile interior path (k a multiple of 64 but not of 512) and its
# chunked interior path (k a multiple of 512).
@pytest.mark.parametrize("m,n,k", [(128, 128, 64), (37, 200, 512), (1, 64, 32), (130, 70, 96), (256, 384, 4096),
                                   (300, 520, 1056), (512, 256, 2048), (256, 256, 576), (512, 512, 1536),
                                   (64, 130, 1056)])
def test_gemm_all_entries(m, n, k):
    inp = workloads.workload(4, n=n, k=k, m=m, seed=m * 1000 + n + k)
    Y = _run(inp, "all entries")
    ms, ns = np.meshgrid(np.arange(m), np.arange(n), indexing="ij")
    _check_entries(inp, Y, ms.ravel(), ns.ravel(), "gemm %dx%dx%d" % (m, n, k))


def test_gemm_dyadic_exact():
    rng = np.random.default_rng(21)
    m, n, k = 96, 160, 512
    codes = rng.integers(0, 256, (n, k // 2), dtype=np.uint8)
    scales = (127 + rng.integers(-4, 3, (n, k // 32))).astype(np.uint8)
    X = workloads.bf16_bits_from_f32(rng.integers(-8, 9, (m, k)).astype(np.float32))
    inp = dict(n=n, k=k, m=m, data=codes, scales=scales, X=X)
    Y = _run(inp, "dyadic")
    ms, ns = np.meshgrid(np.arange(m), np.arange(n), indexing="ij")
    y_ref, _ = oracle.gemm_entries(oracle.MXFP4, codes, scales, 1.0, k, X, ms.ravel(), ns.ravel())
    want = oracle.bf16_rne_array(y_ref.astype(np.float32))
    assert np.array_equal(Y.ravel(), want)


def test_gemm_workload_full_size_sampled():
    inp = workloads.workload(4)
    m, n = inp["m"], inp["n"]
    Y = _run(inp, "full workload 4")
    rng = np.random.default_rng(99)
    ms = np.concatenate([rng.integers(0, m, 1500), np.full(64, m - 1), np.arange(64)])
    ns = np.concatenate([rng.integers(0, n, 1500), np.arange(n - 64, n), np.full(64, 0)])
    _check_entries(inp, Y, ms, ns, "workload 4 sampled")


def test_gemm_workload_full_width_rows():
    """64 full rows of the 2048 x 8192 x 8192 product: every column tile,
    so every workgroup position of the XCD-banded order, 8 rows in each of
    the 8 row tiles (first, last and inside)."""
    inp = workloads.workload(4)
    m, n = inp["m"], inp["n"]
    Y = _run(inp, "full workload 4, 64 full rows")
    rng = np.random.default_rng(64)
    rows = np.concatenate([[256 * t, 256 * t + 255] + list(256 * t + rng.choice(np.arange(1, 255), 6, replace=False))
                           for t in range(m // 256)])
    assert rows.size == 64 and np.unique(rows).size == 64
    ms, ns = np.meshgrid(rows, np.arange(n), indexing="ij")
    _check_entries(inp, Y, ms.ravel(), ns.ravel(), "workload 4, 64 full rows")


@pytest.mark.parametrize("k,x_binades", [(8192, 1), (8192, 13), (65536, 13)])
def test_gemm_one_sign_long_k(k, x_binades):
    """Positive weights and activations: nothing cancels, the accumulator
    grows to the full sum, and every product is added far below it, which is
    where the matrix core's alignment of the addends to the largest one drops
    low bits. The band must still hold over 64 rows x 256 columns."""
    rng = np.random.default_rng(k + x_binades)
    m, n = 256, 256
    nib = rng.integers(1, 8, (n, k)).astype(np.uint8)
    data = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    scales = rng.integers(112, 128, (n, k // 32)).astype(np.uint8)
    x = rng.uniform(1.0, 2.0, (m, k)) * np.exp2(-rng.integers(0, x_binades, (m, k)))
    inp = dict(n=n, k=k, m=m, data=data, scales=scales, X=workloads.bf16_bits_from_f32(x.astype(np.float32)))
    Y = _run(inp, "one sign")
    ms, ns = np.meshgrid(np.arange(0, m, 4), np.arange(n), indexing="ij")
    _check_entries(inp, Y, ms.ravel(), ns.ravel(), "one-sign %d x %d x %d" % (m, n, k))


def test_gemm_deterministic_and_strided():
    inp = workloads.workload(4, n=192, k=1024, m=80, seed=5)
    w = qbn.QTensor("mxfp4", 192, 1024, dev(inp["data"]), dev(inp["scales"]))
    X = dev(inp["X"]).view(torch.bfloat16)
    a = qbn.quantized_gemm(w, X)
    b = qbn.quantized_gemm(w, X)
    # the same product through padded leading dimensions
    Xp = torch.zeros((80, 1024 + 64), dtype=torch.bfloat16, device=DEV)
    Xp[:, :1024] = X
    Yp = torch.zeros((80, 192 + 8), dtype=torch.bfloat16, device=DEV)
    say("gemm strided")
    qbn.quantized_gemm(w, Xp[:, :1024], Yp[:, :192])
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(a), host_bits(b))
    assert np.array_equal(host_bits(Yp[:, :192].contiguous()), host_bits(a))
    assert (host_bits(Yp[:, 192:].contiguous()) == 0).all()


def test_gemm_zero_k_fills_only_the_logical_output():
    w = qbn.QTensor("mxfp4", 24, 0, torch.empty(24, 0, dtype=torch.uint8, device=DEV),
                    torch.empty(24, 0, dtype=torch.uint8, device=DEV))
    Yp = torch.full((5, 32), 3.0, dtype=torch.bfloat16, device=DEV)
    X = torch.empty((5, 8), dtype=torch.bfloat16, device=DEV)
    say("gemm k = 0")
    qbn.quantized_gemm(w, X[:, :0], Yp[:, :24])
    torch.cuda.synchronize()
    assert (Yp[:, :24].float().cpu() == 0).all()
    assert (Yp[:, 24:].float().cpu() == 3).all()


@pytest.mark.parametrize("offset", [2, 1])
def test_gemm_unaligned_scales(offset):
    """Scale bytes at a 2-byte (per-k-tile interior path) or odd (edge path)
    address must give the same product as aligned ones."""
    m, n, k = 256, 256, 1024
    inp = workloads.workload(4, n=n, k=k, m=m, seed=77 + offset)
    base = dev(inp["data"])
    sc = torch.zeros(inp["scales"].size + 16, dtype=torch.uint8, device=DEV)
    sc[offset:offset + inp["scales"].size] = dev(inp["scales"]).reshape(-1)
    w = qbn.QTensor("mxfp4", n, k, base, sc[offset:offset + inp["scales"].size].view(n, k // 32))
    X = dev(inp["X"]).view(torch.bfloat16)
    say("gemm scales offset", offset)
    Y = host_bits(qbn.quantized_gemm(w, X)).reshape(m, n)
    Y0 = _run(inp, "aligned scales")
    assert np.array_equal(Y, Y0)
    ms, ns = np.meshgrid(np.arange(0, m, 7), np.arange(0, n, 5), indexing="ij")
    _check_entries(inp, Y, ms.ravel(), ns.ravel(), "unaligned scales")
