"""GPU: every hot-path entry point captured in a HIP graph (torch.cuda.graph,
as bench.py times them) and replayed three times. Before the eager run and
before every replay the outputs are overwritten with one sentinel byte by an
eager fill on the same stream, with a synchronization between; every replay
must reproduce the eager run's output bytes exactly. A launch path that
recorded a memset node, allocated, synchronized or read back on the host
during capture would fail here (capture errors, or a replay that leaves the
sentinel or stale bytes). The kernels reduce in fixed orders, so the eager
and replayed results are bit-identical."""
import ctypes

import numpy as np
import pytest
import torch

import bit_block_quantized_nibble_amd as qbn
import workloads
from gpu_util import DEV, dev, say, x_dev

pytestmark = pytest.mark.gpu

SENTINEL = 0xA5


def _bytes(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.uint8).cpu().numpy().copy()


def _fill(outs):
    for o in outs:
        o.view(torch.uint8).fill_(SENTINEL)


def _replays_match(step, outs, what, replays=3):
    _fill(outs)
    torch.cuda.synchronize()
    step()
    torch.cuda.synchronize()
    want = [_bytes(o) for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(replays):
        _fill(outs)
        torch.cuda.synchronize()
        say("graph replay", what, rep)
        g.replay()
        torch.cuda.synchronize()
        for i, (o, w) in enumerate(zip(outs, want)):
            got = _bytes(o)
            assert np.array_equal(got, w), "%s: replay %d, output %d differs from the eager run in %d bytes" % (
                what, rep, i, int((got != w).sum()))
    del g


def _seq(*calls):
    def run():
        for c in calls:
            c()
    return run


def _qt(inp):
    return qbn.QTensor(inp["fmt"], inp["n"], inp["k"], dev(inp["data"]),
                       None if inp.get("scales") is None else dev(inp["scales"]), scale2=inp.get("scale2", 1.0))


# (workload, n, k): the rows kernels of MXFP4 and NVFP4, the Q4_K row loop
# (x staged in LDS), the CKE split-half kernel
@pytest.mark.parametrize("c,n,k", [(1, 256, 1024), (2, 96, 4096), (3, 80, 4096), (8, 64, 4096)])
def test_graph_gemv(c, n, k):
    inp = workloads.workload(c, n=n, k=k, seed=7100 + c)
    w = _qt(inp)
    x = x_dev(inp["x"])
    y = torch.empty(n, dtype=torch.float32, device=DEV)
    _replays_match(qbn.prepare_gemv(w, x, y), [y], "gemv %s %dx%d" % (inp["fmt"], n, k))


@pytest.mark.parametrize("fmt", ["gptq4", "awq4", "q4_0"])
def test_graph_gemv_int4(fmt):
    inp = workloads.workload(7, n=1024, k=4096, seed=7107)
    N, K, g = inp["N"], inp["K"], inp["group"]
    if fmt == "q4_0":
        w = qbn.QTensor("q4_0", N, K, dev(inp["q4_0"]))
    else:
        w = qbn.QTensor(fmt, N, K, dev(inp["gptq"] if fmt == "gptq4" else inp["awq"]),
                        dev(inp["scales"].view(np.uint16)), dev(inp["zeros"]), group=g)
    x = x_dev(inp["x"])
    y = torch.empty(N, dtype=torch.float32, device=DEV)
    _replays_match(qbn.prepare_gemv(w, x, y), [y], "gemv %s %dx%d" % (fmt, N, K))


def test_graph_gemm_mxfp4():
    # 256 x 256 tiles with whole 8-k-tile scale chunks (k % 512 == 0)
    inp = workloads.workload(4, n=512, k=1024, m=256, seed=7104)
    w = _qt(inp)
    X = x_dev(inp["X"])
    Y = torch.empty((256, 512), dtype=torch.bfloat16, device=DEV)
    _replays_match(qbn.prepare_gemm(w, X, Y), [Y], "gemm mxfp4 256x512x1024")


@pytest.mark.parametrize("fmt", ["gptq4", "awq4", "q4_0"])
def test_graph_gemm_int4(fmt):
    # the 256 x 128 workgroup tile (m >= 256)
    inp = workloads.workload(9, n=256, k=512, m=256, seed=7109)
    N, K, M, g = inp["N"], inp["K"], inp["M"], inp["group"]
    if fmt == "q4_0":
        w = qbn.QTensor("q4_0", N, K, dev(inp["q4_0"]))
    else:
        w = qbn.QTensor(fmt, N, K, dev(inp["gptq"] if fmt == "gptq4" else inp["awq"]),
                        dev(inp["scales"].view(np.uint16)), dev(inp["zeros"]), group=g)
    X = x_dev(inp["X"])
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    _replays_match(qbn.prepare_gemm(w, X, Y), [Y], "gemm %s %dx%dx%d" % (fmt, M, N, K))


@pytest.mark.parametrize("c", [3, 2])  # Q4_K x Q8_K (float32 y); NVFP4 x Q8_K, integer-exact (float16 y)
def test_graph_quantize_q8_then_gemv_q8(c):
    inp = workloads.workload(c, n=64, k=4096, seed=7200 + c)
    w = _qt(inp)
    x = x_dev(inp["x"])
    k = inp["k"]
    q = torch.empty(k, dtype=torch.int8, device=DEV)
    d = torch.empty(k // 256, dtype=torch.float32, device=DEV)
    bs = torch.empty(k // 32, dtype=torch.int32, device=DEV)
    y = torch.empty(64, dtype=torch.float32 if c == 3 else torch.float16, device=DEV)
    step = _seq(qbn.prepare_quantize_q8(x, q, d, bs), qbn.prepare_gemv_q8(w, q, d, bs, y))
    _replays_match(step, [q, d, bs, y], "quantize_q8 + gemv_q8 %s" % inp["fmt"])


def test_graph_quantize_mx_then_gemm_mx():
    inp = workloads.workload(4, n=256, k=512, m=128, seed=7300)
    w = _qt(inp)
    X = x_dev(inp["X"])
    xc = torch.empty((128, 256), dtype=torch.uint8, device=DEV)
    xs = torch.empty((128, 16), dtype=torch.uint8, device=DEV)
    Y = torch.empty((128, 256), dtype=torch.bfloat16, device=DEV)
    step = _seq(qbn.prepare_quantize_mx(X, xc, xs), qbn.prepare_gemm_mx(w, xc, xs, Y))
    _replays_match(step, [xc, xs, Y], "quantize_mx + gemm_mx 128x256x512")


def test_graph_quantize_nvfp4():
    rng = np.random.default_rng(7400)
    X = x_dev(workloads.bf16_bits_from_f32(rng.standard_normal((64, 4096)).astype(np.float32)))
    codes = torch.empty((64, 2048), dtype=torch.uint8, device=DEV)
    scales = torch.empty((64, 256), dtype=torch.uint8, device=DEV)
    _replays_match(qbn.prepare_quantize_nvfp4(X, 0.01, 0, codes, scales), [codes, scales], "quantize_nvfp4 64x4096")


def _gptq_src(K, N, g, zeros8, seed):
    inp = workloads.workload(5, n=N, k=K, seed=seed)
    zeros = np.full_like(inp["zeros"], 8) if zeros8 else inp["zeros"]
    return qbn.QTensor("gptq4", N, K, dev(inp["qweight"]), dev(inp["scales"].view(np.uint16)), dev(zeros), group=g)


@pytest.mark.parametrize("dst_fmt,zeros8", [("awq4", False), ("q4_0", True), ("q4_0", False)])
def test_graph_repack(dst_fmt, zeros8):
    # GPTQ -> AWQ; GPTQ -> Q4_0 accepted (every zero point 8) and refused
    # (random zero points: the status word gets the first index, dst untouched)
    K, N, g = 512, 1024, 128
    src = _gptq_src(K, N, g, zeros8, 7500)
    dst = qbn.repack_target(src, dst_fmt, None)
    status = torch.empty(qbn.REPACK_STATUS_WORDS, dtype=torch.int64, device=DEV)
    outs = [dst.data, status[:1]]
    if dst_fmt == "awq4":
        outs = [dst.data, dst.scales, dst.zeros, status[:1]]
    _replays_match(qbn.prepare_repack(src, dst, status), outs, "repack gptq4 -> %s zeros8=%s" % (dst_fmt, zeros8))
    if dst_fmt == "q4_0":
        r = int(status[0].item())
        assert (r == -1) if zeros8 else (r >= 0), r


@pytest.mark.parametrize("zeros8", [True, False])
def test_graph_repack_noalloc(zeros8):
    K, N, g = 512, 1024, 128
    src = _gptq_src(K, N, g, zeros8, 7600)
    dst = qbn.repack_target(src, "q4_0", None)
    result = torch.empty(1, dtype=torch.int64, device=DEV)
    lib = qbn._load()
    cs, cd = src._c(), dst._c()

    def step():
        st = lib.qbn_repack_noalloc(ctypes.byref(cs), ctypes.byref(cd), ctypes.c_void_p(result.data_ptr()),
                                    ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        assert st == 0, st

    _replays_match(step, [dst.data, result], "repack_noalloc gptq4 -> q4_0 zeros8=%s" % zeros8)


@pytest.mark.parametrize("layout", ["nk", "kn"])
def test_graph_dequantize(layout):
    src = _gptq_src(512, 1024, 128, False, 7700)
    out = torch.empty((1024, 512) if layout == "nk" else (512, 1024), dtype=torch.bfloat16, device=DEV)
    _replays_match(qbn.prepare_dequantize(src, out, layout=layout), [out], "dequantize gptq4 %s" % layout)


def _prepared(fn, args, what, keep):
    return qbn.Prepared(fn, args, what, torch.device(DEV), keep)


@pytest.mark.parametrize("g", [128, 24])
def test_graph_quantize_int4_sym(g):
    # group 128: the grid-stride lane kernel; 24: one thread per group
    rng = np.random.default_rng(7800 + g)
    m, k = 96, 1536
    W = x_dev(workloads.bf16_bits_from_f32(rng.standard_normal((m, k)).astype(np.float32)))
    codes = torch.empty((m, k // 2), dtype=torch.uint8, device=DEV)
    scales = torch.empty((m, k // g), dtype=torch.float32, device=DEV)
    lib = qbn._load()
    step = _prepared(lib.qbn_quantize_int4_sym, (qbn._ptr(W, "w"), qbn._DTYPES[torch.bfloat16], m, k, k, g,
                                                 qbn._ptr(codes, "codes"), qbn._ptr(scales, "scales")),
                     "qbn_quantize_int4_sym", (W, codes, scales))
    _replays_match(step, [codes, scales], "quantize_int4_sym %dx%d group %d" % (m, k, g))


def test_graph_pack_bits_planes():
    rng = np.random.default_rng(7900)
    count, bits, lo = 100003, 6, 4
    v = dev(rng.integers(0, 1 << bits, count).astype(np.uint8))
    w_lo = torch.empty((count * lo + 31) // 32, dtype=torch.int32, device=DEV)
    w_hi = torch.empty((count * (bits - lo) + 31) // 32, dtype=torch.int32, device=DEV)
    lib = qbn._load()
    step = _prepared(lib.qbn_pack_bits, (qbn._ptr(v, "values"), count, bits, lo, qbn._ptr(w_lo, "lo"),
                                         qbn._ptr(w_hi, "hi")), "qbn_pack_bits", (v, w_lo, w_hi))
    _replays_match(step, [w_lo, w_hi], "pack_bits %d values, 6 bits as 4 + 2" % count)


@pytest.mark.parametrize("K,g", [(4096, 128), (8192, 8)])
def test_graph_resolve_g_idx(K, g):
    # 32 groups (per-wave prefix) and 1024 groups (waves taking turns)
    rng = np.random.default_rng(8000 + K)
    N = 264
    qw = dev(rng.integers(0, 2**32, (K // 8, N), dtype=np.uint32))
    gi = dev(rng.permutation(np.arange(K) // g).astype(np.int32))
    out = torch.empty_like(qw)
    perm = torch.empty(K, dtype=torch.int32, device=DEV)
    status = torch.empty(1, dtype=torch.int32, device=DEV)
    lib = qbn._load()
    step = _prepared(lib.qbn_gptq_resolve_g_idx, (qbn._ptr(qw, "q"), qbn._ptr(gi, "g_idx"), K, N, g,
                                                  qbn._ptr(out, "out"), qbn._ptr(perm, "perm"),
                                                  qbn._ptr(status, "status")),
                     "qbn_gptq_resolve_g_idx", (qw, gi, out, perm, status))
    _replays_match(step, [out, perm, status], "resolve g_idx K=%d group %d" % (K, g))
    assert int(status[0].item()) == 0
