"""GPU parity of the GPTQ metadata conversions: qzeros (both conventions) and
act-order resolution are integer work and must match the oracle bit for bit;
the resolved layer's GEMV on permuted activations must match the act-order
layer's output within the GEMV tolerance."""
import numpy as np
import pytest
import torch

import bit_block_quantized_nibble_amd as qbn
import oracle
import workloads
from gpu_util import DEV, assert_within_tolerance, dev, host_bits, say, x_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("G,N", [(1, 8), (3, 40), (32, 11008), (7, 264)])
@pytest.mark.parametrize("version", [1, 2])
def test_qzeros_both_directions(G, N, version):
    rng = np.random.default_rng(G * 7 + N + version)
    z = rng.integers(version == 1, 16 + (version == 1), (G, N)).astype(np.uint8)
    qz_ref = oracle.qzeros_pack(z, version)
    say("qzeros pack", G, N, version)
    qz = qbn.gptq_qzeros(dev(z), version, False, N)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(qz).reshape(qz_ref.shape), qz_ref)
    words = rng.integers(0, 2**32, (G, N // 8), dtype=np.uint32)
    say("qzeros unpack", G, N, version)
    zl = qbn.gptq_qzeros(dev(words), version, True, N)
    torch.cuda.synchronize()
    assert np.array_equal(zl.cpu().numpy(), oracle.qzeros_unpack(words, version))


def _act_order(rng, K, g):
    return rng.permutation(np.arange(K) // g).astype(np.int32)


@pytest.mark.parametrize("K,N,g", [(256, 64, 32), (4096, 11008, 128), (1024, 40, 8), (128, 8, 128),
                                   (1160, 300, 8), (65536, 8, 8), (2048, 256, 2048), (28672, 520, 128),
                                   (512, 42, 64), (1024, 1001, 128), (8192, 64, 8)])
def test_resolve_g_idx_bit_exact(K, N, g):
    rng = np.random.default_rng(K + N + g)
    qw = rng.integers(0, 2**32, (K // 8, N), dtype=np.uint32)
    g_idx = _act_order(rng, K, g)
    say("resolve g_idx", K, N, g)
    out, perm, status = qbn.gptq_resolve_g_idx(dev(qw), dev(g_idx), g)
    torch.cuda.synchronize()
    rc, perm_ref = oracle.resolve_g_idx(g_idx, g)
    assert int(status.cpu()[0]) == rc == 0
    assert np.array_equal(perm.cpu().numpy(), perm_ref)
    want = oracle.gptq_pack(oracle.gptq_unpack(qw)[perm_ref])
    assert np.array_equal(host_bits(out).reshape(want.shape), want)


@pytest.mark.parametrize("order", ["sorted", "reversed", "interleaved"])
def test_resolve_g_idx_structured_orders(order):
    """g_idx already in group order (the identity), groups in reverse order,
    and rows dealt to groups in turn (every wave sees every group)."""
    K, N, g = 3072, 264, 64
    G = K // g
    base = np.arange(K) // g
    g_idx = {"sorted": base, "reversed": G - 1 - base, "interleaved": np.arange(K) % G}[order].astype(np.int32)
    rng = np.random.default_rng(len(order))
    qw = rng.integers(0, 2**32, (K // 8, N), dtype=np.uint32)
    say("resolve g_idx", order)
    out, perm, status = qbn.gptq_resolve_g_idx(dev(qw), dev(g_idx), g)
    torch.cuda.synchronize()
    rc, perm_ref = oracle.resolve_g_idx(g_idx, g)
    assert int(status.cpu()[0]) == rc == 0
    assert np.array_equal(perm.cpu().numpy(), perm_ref)
    want = oracle.gptq_pack(oracle.gptq_unpack(qw)[perm_ref])
    assert np.array_equal(host_bits(out).reshape(want.shape), want)


def test_resolve_g_idx_errors_keep_identity():
    rng = np.random.default_rng(1)
    K, N, g = 256, 16, 32
    qw = rng.integers(0, 2**32, (K // 8, N), dtype=np.uint32)
    for bad_value, want in ((K // g, -1), (1, -2)):
        g_idx = (np.arange(K) // g).astype(np.int32)
        g_idx[5] = bad_value
        say("resolve g_idx error", want)
        out, perm, status = qbn.gptq_resolve_g_idx(dev(qw), dev(g_idx), g)
        torch.cuda.synchronize()
        assert int(status.cpu()[0]) == want == oracle.resolve_g_idx(g_idx, g)[0]
        assert np.array_equal(perm.cpu().numpy(), np.arange(K))
        assert np.array_equal(host_bits(out).reshape(qw.shape), qw)


@pytest.mark.parametrize("xdt", ["f32", "bf16"])
def test_act_order_layer_end_to_end(xdt):
    """Resolve, permute x on the device, GEMV: the act-order layer's outputs."""
    rng = np.random.default_rng(7)
    K, N, g = 2048, 264, 128
    q = rng.integers(0, 16, (K, N)).astype(np.uint8)
    qw = oracle.gptq_pack(q)
    s = rng.uniform(1e-3, 1e-2, (K // g, N)).astype(np.float16)
    z = rng.integers(0, 16, (K // g, N)).astype(np.uint8)
    g_idx = _act_order(rng, K, g)
    x32 = workloads.x_f32(rng, K)
    x = x32 if xdt == "f32" else workloads.bf16_bits_from_f32(x32)
    say("act-order layer", xdt)
    out, perm, status = qbn.gptq_resolve_g_idx(dev(qw), dev(g_idx), g)
    xp = qbn.permute(x_dev(x), perm)
    w = qbn.QTensor("gptq4", N, K, out, dev(s.view(np.uint16)), dev(z), group=g)
    y = qbn.quantized_gemv(w, xp)
    torch.cuda.synchronize()
    assert int(status.cpu()[0]) == 0
    _, perm_ref = oracle.resolve_g_idx(g_idx, g)
    y_ref, s_ref = oracle.int4_gemv("gptq4", oracle.gptq_pack(q[perm_ref]), s, z, g, x[perm_ref], range(N))
    assert_within_tolerance(y.cpu().numpy(), y_ref, s_ref, "act-order layer " + xdt)


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16, torch.float16])
def test_permute(dt):
    rng = np.random.default_rng(3)
    n = 5000
    src = torch.from_numpy(rng.standard_normal(n).astype(np.float32)).to(dt).to(DEV)
    perm = rng.permutation(n).astype(np.int32)
    say("permute", dt)
    out = qbn.permute(src, dev(perm))
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), src.cpu()[torch.from_numpy(perm).long()])
