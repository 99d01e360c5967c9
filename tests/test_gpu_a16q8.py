"""GPU parity of the integer-exact NVFP4 x Q8_K decode (qbn_quantized_gemv_q8
with an NVFP4 weight): every output must equal the oracle's bit for bit, in
binary16 and in its binary32 widening, for every launch path."""
import numpy as np
import pytest
import torch

import bit_block_quantized_nibble_amd as qbn
import oracle
import workloads
from gpu_util import DEV, dev, host_bits, say, x_dev

pytestmark = pytest.mark.gpu


def _weights(rng, n, k, all_scales=False):
    codes, scales = workloads.nvfp4_weights(rng, n, k)
    if all_scales:  # every finite E4M3FN encoding, both signs, subnormals and 448 included
        finite = np.array([b for b in range(256) if b not in (0x7F, 0xFF)], np.uint8)
        scales = rng.choice(finite, size=scales.shape).astype(np.uint8)
    return codes, scales


def _run(codes, scales, scale2, n, k, q, d, ydt, what):
    w = qbn.QTensor("nvfp4", n, k, dev(codes), dev(scales), scale2=scale2)
    y = torch.empty(n, dtype=ydt, device=DEV)
    say("gemv_q8 nvfp4", what, n, k, ydt)
    qbn.quantized_gemv_q8(w, dev(q), dev(d), None, y)
    torch.cuda.synchronize()
    return host_bits(y) if ydt == torch.float32 else y.cpu().view(torch.int16).numpy().view(np.uint16)


def _check(codes, scales, scale2, n, k, q, d, what):
    y32_ref, y16_ref = oracle.nvfp4_a16q8_rows(codes, scales, scale2, k, q, d, range(n))
    want32 = y16_ref.view(np.float16).astype(np.float32).view(np.uint32)
    got16 = _run(codes, scales, scale2, n, k, q, d, torch.float16, what)
    bad = np.flatnonzero(got16 != y16_ref)
    assert bad.size == 0, "%s: %d of %d binary16 outputs differ; first row %d: got 0x%04x want 0x%04x (acc %r)" % (
        what, bad.size, n, bad[0], got16[bad[0]], y16_ref[bad[0]], float(y32_ref[bad[0]]))
    got32 = _run(codes, scales, scale2, n, k, q, d, torch.float32, what + " f32")
    assert np.array_equal(got32, want32), "%s: binary32 widening differs" % what


# row lengths in 256-blocks: 1..16 (one block per lane quad, idle quads for
# short rows), 17..32 (two per quad), longer rows (16-block chunks)
SHAPES = [(1, 256), (7, 512), (37, 1024), (19, 3072), (130, 4096), (9, 5120), (5, 8192), (3, 256 * 33),
          (2, 256 * 70)]


@pytest.mark.parametrize("n,k", SHAPES)
@pytest.mark.parametrize("xdt", ["f32", "bf16"])
def test_a16q8_bit_exact(n, k, xdt):
    rng = np.random.default_rng(n * 7 + k)
    codes, scales = _weights(rng, n, k)
    x32 = workloads.x_f32(rng, k)
    x = x32 if xdt == "f32" else workloads.bf16_bits_from_f32(x32)
    q, d, _ = oracle.q8_quantize(x)
    _check(codes, scales, float(workloads.SCALE2_NVFP4), n, k, q, d, "n=%d k=%d %s" % (n, k, xdt))


def test_a16q8_every_scale_encoding_and_wide_activations():
    rng = np.random.default_rng(3)
    n, k = 64, 2048
    codes, scales = _weights(rng, n, k, all_scales=True)
    x = (rng.standard_normal(k) * np.repeat(10.0 ** rng.uniform(-6, 6, k // 256), 256)).astype(np.float32)
    x[256:512] = 0.0  # a zero block
    q, d, _ = oracle.q8_quantize(x)
    for s2 in (1.0, 0.01, 3.0e-3, 2.0 ** -20):
        _check(codes, scales, float(np.float32(s2)), n, k, q, d, "all scales, scale2 %g" % s2)


def test_a16q8_block_order_tie():
    """Block contributions 1, 2^-24, 2^-24 in ascending order round back to 1
    (each 2^-24 is a tie to even); another order would give 1 + 2^-23."""
    k = 768
    codes = np.zeros((1, k // 2), np.uint8)
    scales = np.zeros((1, k // 16), np.uint8)
    x = np.zeros(k, np.float32)
    for b, (code, sb, xv, sc) in enumerate([(6, 0x28, 1.0, 1.0), (1, 0x01, 2.0 ** -14, 2.0 ** -14),
                                            (1, 0x01, 2.0 ** -14, 2.0 ** -14)]):
        codes[0, 128 * b] = code
        scales[0, 16 * b] = sb
        x[256 * b + 255] = -127.0 * sc
        x[256 * b] = xv
    q, d, _ = oracle.q8_quantize(x)
    got = _run(codes, scales, 1.0, 1, k, q, d, torch.float32, "order tie")
    assert got.view(np.float32)[0] == 1.0


def test_a16q8_workload_end_to_end_all_rows():
    """The NVFP4 4096 x 4096 weights with bf16 x: device quantizer, then the
    decode; all 4096 outputs bit-exact against the oracle chain."""
    inp = workloads.workload(2)
    n, k = inp["n"], inp["k"]
    say("gemv_q8 nvfp4 full workload", n, k)
    qd, dd, bd = qbn.quantize_q8(x_dev(inp["x"]))
    w = qbn.QTensor("nvfp4", n, k, dev(inp["data"]), dev(inp["scales"]), scale2=inp["scale2"])
    y = torch.empty(n, dtype=torch.float16, device=DEV)
    qbn.quantized_gemv_q8(w, qd, dd, None, y)
    torch.cuda.synchronize()
    got = y.cpu().view(torch.int16).numpy().view(np.uint16)
    q, d, _ = oracle.q8_quantize(inp["x"])
    assert np.array_equal(qd.cpu().numpy(), q) and np.array_equal(host_bits(dd), d.view(np.uint32))
    _, y16 = oracle.nvfp4_a16q8_rows(inp["data"], inp["scales"], inp["scale2"], k, q, d, range(n))
    assert np.array_equal(got, y16), "%d of %d rows differ" % (int((got != y16).sum()), n)


def test_a16q8_deterministic_and_empty():
    rng = np.random.default_rng(9)
    n, k = 300, 4096
    codes, scales = _weights(rng, n, k)
    q, d, _ = oracle.q8_quantize(workloads.x_f32(rng, k))
    a = _run(codes, scales, 0.5, n, k, q, d, torch.float16, "run 1")
    b = _run(codes, scales, 0.5, n, k, q, d, torch.float16, "run 2")
    assert np.array_equal(a, b)
    say("gemv_q8 nvfp4 k = 0")
    w0 = qbn.QTensor("nvfp4", 5, 0, torch.empty(5, 0, dtype=torch.uint8, device=DEV),
                     torch.empty(5, 0, dtype=torch.uint8, device=DEV))
    y = torch.full((5,), 7.0, dtype=torch.float16, device=DEV)
    e = torch.empty(0, dtype=torch.int8, device=DEV)
    qbn.quantized_gemv_q8(w0, e, e.float(), None, y)
    torch.cuda.synchronize()
    assert (y.float().cpu() == 0).all()
