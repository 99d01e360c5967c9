"""GPU parity: qbn_repack moves int4 codes between GPTQ, AWQ and Q4_0
bit-exactly (compared with the oracle's pack(unpack(...)) through the
logical matrix), on ragged tiles, on the verification probes and on the full
4096 x 11008 workload, including the GPTQ -> AWQ -> Q4_0 -> AWQ -> GPTQ round
trip. The Q4_0 directions fail closed ("Bit Packing Architecture",
'Repacking between formats': source and target weights must dequantize
bit-identically): a zero point other than 8, or Q4_0 blocks of one target
group with different d, is refused with its first index and nothing is
written."""
import numpy as np
import pytest
import torch

import bit_block_quantized_nibble_amd as qbn
import oracle
import workloads
from gpu_util import DEV, dev, host_bits, say

pytestmark = pytest.mark.gpu


def _q4_0_d_from_scales(scales_u16, K, group):
    """Q4_0 d bits [N][K/32] = bit copy of the group scale of each block."""
    return np.ascontiguousarray(np.repeat(scales_u16.T, group // 32, axis=1))


def _mk(fmt, q, scales, zeros, group):
    K, N = q.shape
    if fmt == "gptq4":
        return qbn.QTensor("gptq4", N, K, dev(oracle.gptq_pack(q)), dev(scales), dev(zeros), group=group)
    if fmt == "awq4":
        return qbn.QTensor("awq4", N, K, dev(oracle.awq_pack(q)), dev(scales), dev(zeros), group=group)
    d = _q4_0_d_from_scales(scales, K, group)
    return qbn.QTensor("q4_0", N, K, dev(oracle.q4_0_pack(q, d)))


def _expect(fmt, q, scales, group):
    K, N = q.shape
    if fmt == "gptq4":
        return oracle.gptq_pack(q)
    if fmt == "awq4":
        return oracle.awq_pack(q)
    return oracle.q4_0_pack(q, _q4_0_d_from_scales(scales, K, group))


DIRS = [("gptq4", "awq4"), ("awq4", "gptq4"), ("gptq4", "q4_0"), ("awq4", "q4_0"), ("q4_0", "gptq4"),
        ("q4_0", "awq4")]


@pytest.mark.parametrize("src,dst", DIRS)
@pytest.mark.parametrize("K,N,g", [(256, 64, 128), (512, 200, 128), (96, 8, 32), (1024, 136, 256), (4096, 72, 128)])
def test_repack_random(src, dst, K, N, g):
    if "awq4" in (src, dst) and N % 8:
        pytest.skip("AWQ needs N % 8 == 0")
    rng = np.random.default_rng(K * 7 + N + g)
    q = rng.integers(0, 16, (K, N)).astype(np.uint8)
    scales = rng.uniform(-0.01, 0.01, (K // g, N)).astype(np.float16).view(np.uint16)
    zeros = rng.integers(0, 16, (K // g, N)).astype(np.uint8)
    if "q4_0" in (src, dst):
        zeros[:] = 8  # the only zero point Q4_0 holds; the scales round-trip as block d values
    w = _mk(src, q, scales, zeros, g)
    say("repack", src, "->", dst, K, N, g)
    out = qbn.repack(w, dst, dst_group=g if dst != "q4_0" else None)
    torch.cuda.synchronize()
    want = _expect(dst, q, scales, g)
    got = host_bits(out.data)
    assert np.array_equal(got.reshape(want.shape).view(np.uint8), want.view(np.uint8))
    if dst != "q4_0":
        assert np.array_equal(host_bits(out.scales).view(np.uint16).reshape(scales.shape), scales)
        assert np.array_equal(host_bits(out.zeros).reshape(zeros.shape), zeros)


def test_repack_probes_all_directions():
    K, N, g = 256, 256, 128
    pat, rand, full = workloads.layout_probes(K, N)
    scales = np.full((K // g, N), 0x3C00, np.uint16)
    zeros = np.full((K // g, N), 8, np.uint8)
    for name, probe in (("patterned", pat), ("random", rand), ("all-15", full)):
        for src, dst in DIRS:
            say("repack probe", name, src, dst)
            out = qbn.repack(_mk(src, probe, scales, zeros, g), dst, dst_group=g if dst != "q4_0" else None)
            torch.cuda.synchronize()
            want = _expect(dst, probe, scales, g)
            assert np.array_equal(host_bits(out.data).reshape(want.shape).view(np.uint8), want.view(np.uint8)), \
                (name, src, dst)


def test_workload5_refused_with_random_zero_points():
    """The workload's zero points are uniform over 0..15: Q4_0 cannot hold
    them, so GPTQ / AWQ -> Q4_0 is refused at the first zero point != 8 and
    the destination keeps its contents."""
    inp = workloads.workload(5)
    K, N, g = inp["K"], inp["N"], inp["group"]
    zeros = inp["zeros"]
    gptq = qbn.QTensor("gptq4", N, K, dev(inp["qweight"]), dev(inp["scales"].view(np.uint16)), dev(zeros), group=g)
    awq = qbn.repack(gptq, "awq4")
    first = int(np.flatnonzero(zeros.ravel() != 8)[0])
    for src in (gptq, awq):
        sentinel = torch.full((N, K // 32, 18), 0xA5, dtype=torch.uint8, device=DEV)
        say("workload 5 refusal", src.format, "-> q4_0")
        with pytest.raises(qbn.RepackRefused) as e:
            qbn.repack(src, "q4_0", data=sentinel)
        assert e.value.index == first
        torch.cuda.synchronize()
        assert (sentinel == 0xA5).all().item()


def test_workload5_round_trip_and_dequant_identity():
    """Workload 5's codes and scales with every zero point 8 (what Q4_0 can
    hold): the round trip GPTQ -> AWQ -> Q4_0 -> AWQ -> GPTQ is bit-exact and
    all four layouts dequantize to the same values everywhere."""
    inp = workloads.workload(5)
    K, N, g = inp["K"], inp["N"], inp["group"]
    scales = inp["scales"].view(np.uint16)
    zeros = np.full_like(inp["zeros"], 8)
    qw = inp["qweight"]
    gptq = qbn.QTensor("gptq4", N, K, dev(qw), dev(scales), dev(zeros), group=g)
    say("workload 5: gptq -> awq")
    awq = qbn.repack(gptq, "awq4")
    say("workload 5: awq -> q4_0")
    q40 = qbn.repack(awq, "q4_0")
    say("workload 5: q4_0 -> awq")
    awq2 = qbn.repack(q40, "awq4", dst_group=g)
    say("workload 5: awq -> gptq")
    gptq2 = qbn.repack(awq2, "gptq4")
    torch.cuda.synchronize()
    q = oracle.gptq_unpack(qw)
    assert np.array_equal(host_bits(awq.data).view(np.uint32), oracle.awq_pack(q))
    assert np.array_equal(host_bits(q40.data).reshape(N, K // 32, 18),
                          oracle.q4_0_pack(q, _q4_0_d_from_scales(scales, K, g)))
    assert np.array_equal(host_bits(gptq2.data).view(np.uint32), qw)
    assert np.array_equal(host_bits(gptq2.scales).view(np.uint16).reshape(scales.shape), scales)
    assert (host_bits(gptq2.zeros) == 8).all()
    say("workload 5: dequant identities")
    wg = host_bits(qbn.dequantize(gptq, dtype=torch.float32, layout="kn"))
    wa = host_bits(qbn.dequantize(awq, dtype=torch.float32, layout="kn"))
    w0 = host_bits(qbn.dequantize(q40, dtype=torch.float32, layout="kn"))
    torch.cuda.synchronize()
    assert np.array_equal(wg, wa)
    assert np.array_equal(w0, wg)


@pytest.mark.parametrize("dst", ["gptq4", "awq4"])
def test_q4_0_source_refused_when_a_group_mixes_d(dst):
    """Q4_0 -> GPTQ / AWQ with group 128: a column whose four blocks of one
    group carry different d cannot share one scale; the first such block is
    reported through the status array and nothing is written."""
    K, N, g = 512, 64, 128
    rng = np.random.default_rng(17)
    q = rng.integers(0, 16, (K, N)).astype(np.uint8)
    scales = rng.uniform(0.001, 0.01, (K // g, N)).astype(np.float16).view(np.uint16)
    blocks = oracle.q4_0_pack(q, _q4_0_d_from_scales(scales, K, g))
    blocks[9, 6, 0] ^= 0x01   # column 9, block 6 (group 1, its third block)
    blocks[40, 2, 1] ^= 0x02  # a later column
    src = qbn.QTensor("q4_0", N, K, dev(blocks))
    out = qbn.repack_target(src, dst, g)
    out.data.fill_(0x5A5A5A5A)
    status = torch.empty(qbn.REPACK_STATUS_WORDS, dtype=torch.int64, device=DEV)
    say("q4_0 mixed-d refusal ->", dst)
    qbn.prepare_repack(src, out, status)()
    torch.cuda.synchronize()
    assert int(status[0].item()) == 9 * (K // 32) + 6
    assert (out.data == 0x5A5A5A5A).all().item()
    with pytest.raises(qbn.RepackRefused):
        qbn.repack(src, dst, dst_group=g)
    # with group 32 every block is its own group: accepted, and status[0] is -1
    ok = qbn.repack_target(src, dst, 32)
    qbn.prepare_repack(src, ok, status)()
    torch.cuda.synchronize()
    assert int(status[0].item()) == -1
    want = oracle.gptq_pack(q) if dst == "gptq4" else oracle.awq_pack(q)
    assert np.array_equal(host_bits(ok.data).reshape(want.shape).view(np.uint32), want.view(np.uint32))


def test_repack_validate_q4_0_group_scales():
    # Q4_0 -> GPTQ takes each group's scale from its first block; the
    # validator flags a group whose blocks disagree
    K, N, g = 256, 16, 128
    rng = np.random.default_rng(5)
    q = rng.integers(0, 16, (K, N)).astype(np.uint8)
    scales = rng.uniform(0.001, 0.01, (K // g, N)).astype(np.float16).view(np.uint16)
    blocks = oracle.q4_0_pack(q, _q4_0_d_from_scales(scales, K, g))
    w = qbn.QTensor("q4_0", N, K, dev(blocks), group=g)
    assert qbn.validate(w) == -1
    blocks[3, 5, 0] ^= 0x10
    w = qbn.QTensor("q4_0", N, K, dev(blocks), group=g)
    assert qbn.validate(w) == 3 * (K // 32) + 5


@pytest.mark.parametrize("src,dst", [("gptq4", "q4_0"), ("awq4", "q4_0"), ("q4_0", "gptq4"), ("q4_0", "awq4")])
@pytest.mark.parametrize("offset", [0, 4, 2])
def test_repack_q4_0_run_modes(src, dst, offset):
    """k % 256 == 0: 16-byte run pieces on a 16-byte aligned Q4_0 buffer,
    4-byte words at a 4-byte offset, 2-byte units at a 2-byte offset."""
    K, N, g = 512, 264, 128
    rng = np.random.default_rng(offset * 11 + len(src))
    q = rng.integers(0, 16, (K, N)).astype(np.uint8)
    scales = rng.uniform(-0.01, 0.01, (K // g, N)).astype(np.float16).view(np.uint16)
    zeros = np.full((K // g, N), 8, np.uint8)
    nbytes = N * (K // 32) * 18
    raw = torch.zeros(nbytes + 16, dtype=torch.uint8, device=DEV)
    q4 = raw[offset:offset + nbytes].view(N, K // 32, 18)
    say("repack run mode", src, "->", dst, "offset", offset)
    if src == "q4_0":
        q4.copy_(dev(_expect("q4_0", q, scales, g)))
        w = qbn.QTensor("q4_0", N, K, q4)
        out = qbn.repack(w, dst, dst_group=g)
        torch.cuda.synchronize()
        want = _expect(dst, q, scales, g)
        assert np.array_equal(host_bits(out.data).reshape(want.shape).view(np.uint8), want.view(np.uint8))
    else:
        w = _mk(src, q, scales, zeros, g)
        qbn.repack(w, "q4_0", data=q4)
        torch.cuda.synchronize()
        want = _expect("q4_0", q, scales, g)
        assert np.array_equal(q4.cpu().numpy().reshape(want.shape), want)
        assert (raw[:offset].cpu() == 0).all() and (raw[offset + nbytes:].cpu() == 0).all()


@pytest.mark.parametrize("offset", list(range(16)))
def test_zero_point_scan_finds_the_first_index_at_any_alignment(offset):
    """The refusal scan reads zero points 16 bytes at a time between a head
    and a tail checked byte by byte: the first zero point other than 8 is
    found wherever it sits (head, a 16-byte piece, tail) for a buffer at
    any byte offset, and a clean buffer is accepted."""
    K, N, g = 256, 200, 128
    rng = np.random.default_rng(offset)
    q = rng.integers(0, 16, (K, N)).astype(np.uint8)
    scales = rng.integers(0x2000, 0x3C00, (K // g, N)).astype(np.uint16)
    count = (K // g) * N
    buf = torch.full((count + 32,), 8, dtype=torch.uint8, device=DEV)
    zeros = buf[offset:offset + count].view(K // g, N)
    src = qbn.QTensor("gptq4", N, K, dev(oracle.gptq_pack(q)), dev(scales), zeros, group=g)
    head = (16 - offset) % 16
    for first in sorted({0, max(head - 1, 0), head, head + 37, count - 17, count - 1}):
        buf[offset:offset + count] = 8
        buf[offset + first] = 3
        buf[offset + count - 1] = 15  # a later offender too, except when first is the last one
        say("zero-point scan", offset, first)
        with pytest.raises(qbn.RepackRefused) as e:
            qbn.repack(src, "q4_0")
        assert e.value.index == first, (offset, first)
    buf[offset:offset + count] = 8
    buf[:offset] = 0        # bytes outside the view are not zero points
    buf[offset + count:] = 0
    out = qbn.repack(src, "q4_0")
    torch.cuda.synchronize()
    want = oracle.q4_0_pack(q, _q4_0_d_from_scales(scales, K, g))
    assert np.array_equal(host_bits(out.data).reshape(want.shape).view(np.uint8), want.view(np.uint8))
