"""Host-side tests of the C ABI that need no GPU: the library loads, exports
every entry point include/qbn.h declares, reports its sizes, and rejects bad
arguments with the documented status codes before anything is launched
(all pointers below are never dereferenced: every call fails its host checks
or is an empty no-op)."""
import ctypes
import os
import re

import pytest

import bit_block_quantized_nibble_amd as qbn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
OK, NULL, FORMAT, UNSUP, SHAPE, ALIGN, SCALE2, NANS, DTYPE, HIP, GROUP = range(11)
MX, NV, QK, Q0, GP, AW = 1, 2, 3, 4, 5, 6
CKE = 8
F32, BF16 = 0, 1
A = 0x10000  # an aligned fake address
B = 0x20000
C = 0x30000


@pytest.fixture(scope="module")
def lib():
    return qbn._load()


def T(fmt, n, k, data=A, scales=B, zeros=C, scale2=1.0, group=0, reserved=0):
    t = qbn._CTensor()
    t.format, t.group, t.n, t.k = fmt, group, n, k
    t.data, t.scales, t.zeros = data, scales, zeros
    t.scale2, t.reserved = scale2, reserved
    return ctypes.byref(t)


def test_exports_every_declared_symbol(lib):
    header = open(os.path.join(ROOT, "include", "qbn.h")).read()
    declared = re.findall(r"QBN_API\s+[\w\s\*]+?\b(qbn_\w+)\s*\(", header)
    assert len(declared) == 23
    assert set(declared) == set(qbn.EXPORTED)
    so = ctypes.CDLL(qbn.lib_path())
    for name in declared:
        assert hasattr(so, name), name


def test_abi_and_struct(lib):
    assert lib.qbn_abi_version() == 2
    assert lib.qbn_tensor_struct_size() == ctypes.sizeof(qbn._CTensor) == 56
    for s in range(11):
        assert lib.qbn_status_string(s)
    assert lib.qbn_status_string(99) == b"unknown status"


def test_bytes_match_page_bit_budgets(lib):
    # Four Bits, Three Contracts sections 3-5; Chapter 7 section 7.1
    n, k = 4096, 4096
    mx = lib.qbn_bytes(MX, n, k, 0, 0) + lib.qbn_bytes(MX, n, k, 0, 1)
    nv = lib.qbn_bytes(NV, n, k, 0, 0) + lib.qbn_bytes(NV, n, k, 0, 1)
    qk = lib.qbn_bytes(QK, n, k, 0, 0)
    q0 = lib.qbn_bytes(Q0, n, k, 0, 0)
    assert mx * 8 / (n * k) == 4.25
    assert nv * 8 / (n * k) == 4.5
    assert qk * 8 / (n * k) == 4.5 and lib.qbn_bytes(QK, 1, 256, 0, 0) == 144
    assert q0 * 8 / (n * k) == 4.5 and lib.qbn_bytes(Q0, 1, 32, 0, 0) == 18
    assert lib.qbn_bytes(GP, 11008, 4096, 128, 0) == 22544384
    assert lib.qbn_bytes(GP, 11008, 4096, 128, 1) == 2 * 32 * 11008
    assert lib.qbn_bytes(AW, 11008, 4096, 128, 2) == 32 * 11008
    assert lib.qbn_bytes(QK, 1, 255, 0, 0) == -1
    assert lib.qbn_bytes(7, 1, 32, 0, 0) == -1
    assert lib.qbn_bytes(MX, 1, 32, 0, 3) == -1
    assert lib.qbn_bytes(QK, 1, 256, 0, 1) == 0
    # Why 4-Bit Quantization Is King, section 5: 36 bytes per 64 weights
    cke = lib.qbn_bytes(CKE, n, k, 0, 0)
    assert cke * 8 / (n * k) == 4.5 and lib.qbn_bytes(CKE, 1, 64, 0, 0) == 36
    assert lib.qbn_bytes(CKE, 1, 64, 0, 1) == 0 and lib.qbn_bytes(CKE, 1, 96, 0, 0) == -1


def test_gemv_rejections(lib):
    g = lib.qbn_quantized_gemv
    assert g(None, A, F32, B, F32, None) == NULL
    assert g(T(9, 4, 32), A, F32, B, F32, None) == FORMAT
    assert g(T(MX, 4, 32, reserved=1), A, F32, B, F32, None) == FORMAT
    assert g(T(MX, -1, 32), A, F32, B, F32, None) == SHAPE
    assert g(T(MX, 4, 48), A, F32, B, F32, None) == SHAPE
    assert g(T(NV, 4, 40), A, F32, B, F32, None) == SHAPE
    assert g(T(QK, 4, 512 + 32), A, F32, B, F32, None) == SHAPE
    assert g(T(Q0, 4, 64), A + 8, F32, B, F32, None) == ALIGN
    assert g(T(GP, 16, 64, group=32), A, F32, B + 2, F32, None) == ALIGN
    assert g(T(GP, 16, 64, group=32, zeros=None), A, F32, B, F32, None) == NULL
    assert g(T(GP, 16, 64, group=12), A, F32, B, F32, None) == GROUP
    assert g(T(AW, 12, 64, group=32), A, F32, B, F32, None) == SHAPE
    assert g(T(MX, 4, 64), A, 7, B, F32, None) == FORMAT
    assert g(T(MX, 4, 64), A, 2, B, F32, None) == DTYPE
    assert g(T(MX, 4, 64), A, F32, B, BF16, None) == DTYPE
    assert g(T(MX, 4, 64, data=None), A, F32, B, F32, None) == NULL
    assert g(T(MX, 4, 64, scales=None), A, F32, B, F32, None) == NULL
    assert g(T(MX, 4, 64, data=A + 8), A, F32, B, F32, None) == ALIGN
    assert g(T(MX, 4, 64), A + 4, F32, B, F32, None) == ALIGN
    assert g(T(MX, 4, 64), A, F32, B + 2, F32, None) == ALIGN
    assert g(T(MX, 4, 64), None, F32, B, F32, None) == NULL
    assert g(T(MX, 4, 64), A, F32, None, F32, None) == NULL
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        assert g(T(NV, 4, 64, scale2=bad), A, F32, B, F32, None) == SCALE2
    # empty: nothing to do, nothing launched
    assert g(T(MX, 0, 64, data=None, scales=None), None, F32, None, F32, None) == OK


def test_quantize_q8_rejections(lib):
    f = lib.qbn_quantize_q8
    assert f(A, 7, 256, B, C, C, None) == FORMAT
    assert f(A, 2, 256, B, C, C, None) == DTYPE
    assert f(A, F32, 300, B, C, C, None) == SHAPE
    assert f(A, F32, -256, B, C, C, None) == SHAPE
    assert f(None, F32, 256, B, C, C, None) == NULL
    assert f(A, F32, 256, None, C, C, None) == NULL
    assert f(A, F32, 256, B, None, C, None) == NULL
    assert f(A, F32, 256, B, C, None, None) == NULL
    assert f(A + 8, F32, 256, B, C, C, None) == ALIGN
    assert f(A, BF16, 256, B + 4, C, C, None) == ALIGN
    assert f(A, F32, 256, B, C + 2, C, None) == ALIGN
    assert f(A, F32, 256, B, C, C + 4, None) == ALIGN
    assert f(None, F32, 0, None, None, None, None) == OK


def test_gemv_q8_rejections(lib):
    g = lib.qbn_quantized_gemv_q8
    assert g(None, A, B, C, A, F32, None) == NULL
    assert g(T(MX, 4, 256), A, B, C, A, F32, None) == UNSUP
    assert g(T(Q0, 4, 256), A, B, C, A, F32, None) == UNSUP
    assert g(T(QK, 4, 300), A, B, C, A, F32, None) == SHAPE
    assert g(T(QK, 4, 256), A, B, C, A, BF16, None) == DTYPE
    assert g(T(QK, 4, 256), A, B, C, A, 9, None) == FORMAT
    assert g(T(QK, 4, 256), A, B, C, None, F32, None) == NULL
    assert g(T(QK, 4, 256), A, B, C, A + 2, F32, None) == ALIGN
    assert g(T(QK, 4, 256), None, B, C, A, F32, None) == NULL
    assert g(T(QK, 4, 256), A, None, C, A, F32, None) == NULL
    assert g(T(QK, 4, 256), A, B, None, A, F32, None) == NULL
    assert g(T(QK, 4, 256), A + 4, B, C, A, F32, None) == ALIGN
    assert g(T(QK, 4, 256), A, B + 1, C, A, F32, None) == ALIGN
    assert g(T(QK, 4, 256), A, B, C + 4, A, F32, None) == ALIGN
    assert g(T(QK, 4, 256, data=A + 8), A, B, C, A, F32, None) == ALIGN
    assert g(T(QK, 0, 256, data=None), None, None, None, None, F32, None) == OK
    # NVFP4: the integer-exact route; k in whole 256-blocks, bsums unused, f16 or f32 output
    F16 = 2
    assert g(T(NV, 4, 272), A, B, None, A, F32, None) == SHAPE
    assert g(T(NV, 4, 256), A, B, None, A, BF16, None) == DTYPE
    assert g(T(NV, 4, 256, scale2=0.0), A, B, None, A, F32, None) == SCALE2
    assert g(T(NV, 4, 256, scales=None), A, B, None, A, F32, None) == NULL
    assert g(T(NV, 4, 256), A, B, None, A + 2, F32, None) == ALIGN
    assert g(T(NV, 4, 256), A, B, None, A + 1, F16, None) == ALIGN
    assert g(T(NV, 4, 256), A + 8, B, None, A, F16, None) == ALIGN
    assert g(T(NV, 4, 256), A, None, None, A, F16, None) == NULL
    assert g(T(QK, 4, 256), A, B, C, A, F16, None) == DTYPE


def test_mx_rejections(lib):
    q = lib.qbn_quantize_mx
    MX8 = 7
    assert q(A, F32, 4, 64, 64, 9, B, C, None) == FORMAT
    assert q(A, F32, 4, 64, 64, QK, B, C, None) == UNSUP
    assert q(A, 2, 4, 64, 64, MX, B, C, None) == DTYPE
    assert q(A, F32, 4, 48, 48, MX, B, C, None) == SHAPE
    assert q(A, F32, 4, 64, 32, MX, B, C, None) == SHAPE
    assert q(A, F32, 4, 64, 66, MX, B, C, None) == ALIGN
    assert q(A + 8, F32, 4, 64, 64, MX, B, C, None) == ALIGN
    assert q(A, F32, 4, 64, 64, MX8, B + 2, C, None) == ALIGN
    assert q(A, F32, 4, 64, 64, MX, B + 1, C, None) == ALIGN
    assert q(None, F32, 4, 64, 64, MX, B, C, None) == NULL
    assert q(None, F32, 0, 64, 64, MX, None, None, None) == OK
    g = lib.qbn_quantized_gemm_mx
    assert g(T(NV, 8, 64), 4, MX, A, B, C, BF16, 8, None) == UNSUP
    # MXFP8 activations are refused: the FP8 x FP4 instruction truncates each
    # run of 8 products 13 bits below the run's largest, past the tolerance
    assert g(T(MX, 8, 64), 4, MX8, A, B, C, BF16, 8, None) == UNSUP
    assert g(T(MX, 8, 64), 4, MX8, A + 8, B, C, BF16, 8, None) == UNSUP
    assert g(T(MX, 8, 64), 4, 9, A, B, C, BF16, 8, None) == FORMAT
    assert g(T(MX, 8, 64), 4, MX, A, B, C, 2, 8, None) == DTYPE
    assert g(T(MX, 8, 64), 4, MX, A, B, C, BF16, 4, None) == SHAPE
    assert g(T(MX, 8, 64), -1, MX, A, B, C, BF16, 8, None) == SHAPE
    assert g(T(MX, 8, 64), 4, MX, A + 8, B, C, BF16, 8, None) == ALIGN
    assert g(T(MX, 8, 64), 4, MX, A, B, C + 2, F32, 8, None) == ALIGN
    assert g(T(MX, 8, 64), 4, MX, None, B, C, BF16, 8, None) == NULL
    assert g(T(MX, 8, 64), 4, MX, A, None, C, BF16, 8, None) == NULL
    assert g(T(MX, 8, 64), 0, MX, None, None, None, BF16, 8, None) == OK


def test_gemm_rejections(lib):
    g = lib.qbn_quantized_gemm
    assert g(T(NV, 8, 64), 4, A, BF16, 64, B, BF16, 8, None) == UNSUP
    assert g(T(MX, 8, 64), 4, A, F32, 64, B, BF16, 8, None) == DTYPE
    assert g(T(MX, 8, 64), 4, A, BF16, 64, B, F32, 8, None) == DTYPE
    assert g(T(MX, 8, 64), -1, A, BF16, 64, B, BF16, 8, None) == SHAPE
    assert g(T(MX, 8, 64), 4, A, BF16, 32, B, BF16, 8, None) == SHAPE
    assert g(T(MX, 8, 64), 4, A, BF16, 68, B, BF16, 8, None) == ALIGN
    assert g(T(MX, 8, 64), 4, A, BF16, 64, B, BF16, 4, None) == SHAPE
    assert g(T(MX, 8, 64), 4, A, BF16, 64, B + 1, BF16, 12, None) == ALIGN
    assert g(T(MX, 8, 64), 4, A + 8, BF16, 64, B, BF16, 8, None) == ALIGN
    assert g(T(MX, 8, 64), 0, None, BF16, 64, None, BF16, 8, None) == OK
    # int4 layouts: f32 output allowed, groups and k in units of 32
    assert g(T(GP, 8, 64, group=8), 4, A, BF16, 64, B, BF16, 8, None) == GROUP
    assert g(T(AW, 8, 96, group=48), 4, A, BF16, 96, B, BF16, 8, None) == GROUP
    assert g(T(GP, 8, 64, group=64), 4, A, F32, 64, B, F32, 8, None) == DTYPE
    assert g(T(GP, 8, 64, group=64), 4, A, BF16, 64, B + 2, F32, 8, None) == ALIGN
    assert g(T(Q0, 8, 48), 4, A, BF16, 64, B, BF16, 8, None) == SHAPE
    assert g(T(GP, 8, 64, group=32), 4, A, BF16, 60, B, F32, 8, None) == SHAPE
    assert g(T(GP, 8, 64, group=32), 0, None, BF16, 64, None, F32, 8, None) == OK
    assert g(T(CKE, 8, 64, scale2=0.01), 4, A, BF16, 64, B, BF16, 8, None) == UNSUP


def test_dequant_rejections(lib):
    d = lib.qbn_dequantize
    assert d(T(MX, 4, 64), A, 2, 0, None) == DTYPE
    assert d(T(MX, 4, 64), A, 5, 0, None) == FORMAT
    assert d(T(MX, 4, 64), A, F32, 2, None) == FORMAT
    assert d(T(MX, 4, 64), A + 4, F32, 0, None) == ALIGN
    assert d(T(MX, 4, 64), None, F32, 0, None) == NULL
    assert d(T(Q0, 4, 64, data=A + 1), B, F32, 0, None) == ALIGN
    assert d(T(GP, 8, 64, group=0), B, F32, 0, None) == GROUP
    assert d(T(GP, 8, 64, group=12), B, F32, 0, None) == GROUP
    assert d(T(GP, 8, 64, group=48), B, F32, 0, None) == SHAPE
    assert d(T(AW, 12, 64, group=32), B, F32, 0, None) == SHAPE
    assert d(T(GP, 8, 64, group=32, zeros=None), B, F32, 0, None) == NULL
    assert d(T(GP, 8, 64, group=32, scales=B + 1), B, F32, 0, None) == ALIGN


def test_repack_rejections(lib):
    r = lib.qbn_repack
    S = 0x40000  # a fake status array (8-byte aligned)
    gp = T(GP, 8, 64, group=32)
    assert r(T(MX, 8, 64), T(Q0, 8, 64), S, None) == UNSUP
    assert r(gp, T(GP, 8, 64, group=32), S, None) == UNSUP
    assert r(gp, T(11, 8, 64, group=32), S, None) == FORMAT
    assert r(gp, T(AW, 8, 64, group=32, reserved=1), S, None) == FORMAT
    assert r(gp, None, S, None) == NULL
    assert r(T(GP, 12, 64, group=32), T(AW, 12, 64, group=32), S, None) == SHAPE   # AWQ needs n % 8 == 0
    assert r(gp, T(AW, 8, 128, group=32), S, None) == SHAPE                        # n, k must match
    assert r(gp, T(AW, 8, 64, group=64), S, None) == GROUP                         # GPTQ <-> AWQ keep the group
    assert r(T(GP, 8, 64, group=16), T(Q0, 8, 64), S, None) == GROUP               # Q4_0 needs whole groups of 32
    assert r(T(Q0, 8, 64), T(GP, 8, 64, group=16), S, None) == GROUP
    assert r(T(Q0, 8, 64), T(GP, 8, 96, group=96), S, None) == SHAPE
    assert r(T(Q0, 8, 64), T(GP, 8, 64, group=96), S, None) == SHAPE               # k % group
    assert r(T(Q0, 8, 64), T(GP, 8, 64, group=32, scales=None), S, None) == NULL   # dst scales are outputs
    assert r(gp, T(AW, 8, 64, group=32, data=None), S, None) == NULL
    assert r(gp, T(AW, 8, 64, group=32, data=A + 2), S, None) == ALIGN
    assert r(gp, T(Q0, 8, 64, data=A + 1), S, None) == ALIGN
    # the Q4_0 directions can refuse and need the status array
    assert r(gp, T(Q0, 8, 64), None, None) == NULL
    assert r(T(Q0, 8, 64), T(AW, 8, 64, group=32), None, None) == NULL
    assert r(gp, T(Q0, 8, 64), S + 4, None) == ALIGN
    assert r(T(GP, 8, 0, group=32), T(AW, 8, 0, group=32), None, None) == OK      # empty, status not needed
    # the allocation-free variant applies the same rules to its single result word
    rn = lib.qbn_repack_noalloc
    assert rn(gp, T(Q0, 8, 64), None, None) == NULL
    assert rn(gp, T(Q0, 8, 64), S + 4, None) == ALIGN
    assert rn(gp, T(AW, 8, 64, group=64), S, None) == GROUP
    assert rn(T(MX, 8, 64), T(Q0, 8, 64), S, None) == UNSUP
    assert rn(T(GP, 8, 0, group=32), T(AW, 8, 0, group=32), None, None) == OK


def test_validate_rejections(lib):
    for v in (lib.qbn_validate_async,):
        assert v(T(MX, 4, 64), None, None) == NULL
        assert v(T(MX, 4, 64), A + 4, None) == ALIGN
    host = ctypes.c_int64(0)
    # the synchronous form takes a host int64 and reports argument errors
    # before it allocates anything
    for v, out in ((lib.qbn_validate, ctypes.byref(host)), (lib.qbn_validate_async, A)):
        assert v(T(NV, 4, 64, scale2=0.0), out, None) == SCALE2
        assert v(T(Q0, 4, 64, group=48), out, None) == GROUP
        assert v(T(Q0, 4, 96, group=64), out, None) == SHAPE
        assert v(T(MX, 4, 48), out, None) == SHAPE
        assert v(None, out, None) == NULL


def test_binding_refuses_host_tensors():
    import torch

    w = qbn.QTensor("mxfp4", 2, 32, torch.zeros(2, 16, dtype=torch.uint8), torch.zeros(2, 1, dtype=torch.uint8))
    with pytest.raises(ValueError):
        qbn.quantized_gemv(w, torch.zeros(32), torch.zeros(2))


def test_gptq_meta_rejections(lib):
    z = lib.qbn_gptq_qzeros
    assert z(A, B, 4, 64, 3, 1, None) == FORMAT
    assert z(A, B, 4, 64, 1, 2, None) == FORMAT
    assert z(A, B, 4, 60, 2, 1, None) == SHAPE
    assert z(A, B, -1, 64, 2, 1, None) == SHAPE
    assert z(None, B, 4, 64, 2, 1, None) == NULL
    assert z(A + 2, B, 4, 64, 2, 1, None) == ALIGN     # qzeros words 4-byte aligned
    assert z(A, B + 4, 4, 64, 2, 1, None) == ALIGN     # zero points 8-byte aligned
    assert z(None, None, 0, 64, 2, 1, None) == OK
    r = lib.qbn_gptq_resolve_g_idx
    assert r(A, B, 256, 64, 12, C, A, B, None) == GROUP
    assert r(A, B, 250, 64, 8, C, A, B, None) == SHAPE
    assert r(A, B, 256, 64, 96, C, A, B, None) == SHAPE   # k % group
    assert r(A, B, 8 * 9000, 64, 8, C, A, B, None) == SHAPE  # more than 8192 groups
    assert r(A, None, 256, 64, 32, C, A, B, None) == NULL
    assert r(A, B, 256, 64, 32, A, C, B, None) == UNSUP     # qweight_out aliases qweight
    assert r(A, B + 2, 256, 64, 32, C, A, B, None) == ALIGN
    p = lib.qbn_permute
    assert p(A, B, 16, 7, C, None) == FORMAT
    assert p(A, B, -1, F32, C, None) == SHAPE
    assert p(A, B, 16, F32, A, None) == UNSUP
    assert p(A + 2, B, 16, F32, C, None) == ALIGN
    assert p(None, B, 16, F32, C, None) == NULL
    assert p(None, None, 0, F32, None, None) == OK


def test_encode_rejections(lib):
    q = lib.qbn_quantize_nvfp4
    assert q(A, F32, 4, 64, 64, ctypes.c_float(1.0), 2, B, C, None) == FORMAT
    assert q(A, 2, 4, 64, 64, ctypes.c_float(1.0), 0, B, C, None) == DTYPE
    assert q(A, F32, 4, 64, 64, ctypes.c_float(0.0), 0, B, C, None) == SCALE2
    assert q(A, F32, 4, 64, 64, ctypes.c_float(float("inf")), 0, B, C, None) == SCALE2
    assert q(A, F32, 4, 40, 40, ctypes.c_float(1.0), 0, B, C, None) == SHAPE
    assert q(A, F32, 4, 64, 32, ctypes.c_float(1.0), 0, B, C, None) == SHAPE
    assert q(None, F32, 4, 64, 64, ctypes.c_float(1.0), 0, B, C, None) == NULL
    assert q(A + 2, F32, 4, 64, 64, ctypes.c_float(1.0), 0, B, C, None) == ALIGN
    assert q(A, F32, 4, 64, 64, ctypes.c_float(1.0), 0, B + 4, C, None) == ALIGN
    assert q(None, F32, 0, 64, 64, ctypes.c_float(1.0), 0, None, None, None) == OK
    i = lib.qbn_quantize_int4_sym
    assert i(A, F32, 4, 64, 64, 3, B, C, None) == GROUP
    assert i(A, F32, 4, 64, 64, 0, B, C, None) == GROUP
    assert i(A, F32, 4, 60, 60, 8, B, C, None) == SHAPE
    assert i(A, 2, 4, 64, 64, 8, B, C, None) == DTYPE
    assert i(A, F32, 4, 64, 64, 8, B, C + 2, None) == ALIGN
    assert i(A, F32, 4, 64, 64, 8, None, C, None) == NULL
    p = lib.qbn_pack_bits
    assert p(A, 64, 9, 0, B, None, None) == FORMAT
    assert p(A, 64, 6, 6, B, C, None) == FORMAT
    assert p(A, 64, 6, 4, B, None, None) == NULL
    assert p(A, 64, 3, 0, B + 2, None, None) == ALIGN
    assert p(A, -1, 3, 0, B, None, None) == SHAPE
    assert p(None, 0, 3, 0, None, None, None) == OK
    u = lib.qbn_unpack_bits
    assert u(A, None, 64, 0, 0, B, None) == FORMAT
    assert u(A, None, 64, 6, 2, B, None) == NULL
    assert u(A + 1, None, 64, 5, 0, B, None) == ALIGN


def test_cke_rejections(lib):
    g = lib.qbn_quantized_gemv
    assert g(T(CKE, 4, 96, scale2=0.01), A, F32, B, F32, None) == SHAPE
    assert g(T(CKE, 4, 64, scale2=0.0), A, F32, B, F32, None) == SCALE2
    assert g(T(CKE, 4, 64, scale2=float("inf")), A, F32, B, F32, None) == SCALE2
    assert g(T(CKE, 4, 64, data=A + 2, scale2=0.01), A, F32, B, F32, None) == ALIGN
    assert g(T(CKE, 4, 64, data=None, scale2=0.01), A, F32, B, F32, None) == NULL
    assert g(T(CKE, 4, 64, scale2=0.01), A, F32, B, BF16, None) == DTYPE
    assert g(T(CKE, 0, 64, scale2=0.01), A, F32, B, F32, None) == OK
    # scales are ignored by this format: NULL is accepted (and A + 4 is aligned)
    assert g(T(CKE, 0, 64, data=A + 4, scales=None, scale2=0.01), A, F32, B, F32, None) == OK
    assert lib.qbn_quantized_gemm(T(CKE, 8, 64, scale2=0.01), 4, A, BF16, 64, B, BF16, 8, None) == UNSUP
    assert lib.qbn_quantized_gemv_q8(T(CKE, 8, 256, scale2=0.01), A, B, C, B, F32, None) == UNSUP
    assert lib.qbn_dequantize(T(CKE, 4, 96, scale2=0.01), B, F32, 0, None) == SHAPE
    assert lib.qbn_dequantize(T(CKE, 4, 64, scale2=0.01), B + 8, F32, 0, None) == ALIGN
    r = lib.qbn_repack
    nv, cke = T(NV, 4, 64, scale2=0.01), T(CKE, 4, 64, scale2=0.01)
    assert r(cke, T(GP, 4, 64, group=64), None, None) == UNSUP
    assert r(T(GP, 4, 64, group=64), cke, None, None) == UNSUP
    assert r(nv, T(NV, 4, 64, scale2=0.01), None, None) == UNSUP
    assert r(T(NV, 4, 32, scale2=0.01), T(CKE, 4, 32, scale2=0.01), None, None) == SHAPE
    assert r(nv, T(CKE, 4, 64, data=B + 2, scale2=0.01), None, None) == ALIGN
    assert r(nv, T(CKE, 4, 64, data=None, scale2=0.01), None, None) == NULL
    assert r(nv, T(CKE, 4, 64, scale2=0.0), None, None) == SCALE2  # dst is a complete tensor
    assert r(cke, T(NV, 4, 64, data=B + 4, scale2=0.01), None, None) == ALIGN
    assert r(cke, T(NV, 4, 64, scales=None, scale2=0.01), None, None) == NULL
    assert r(T(CKE, 0, 64, scale2=0.01), T(NV, 0, 64, data=None, scales=None, scale2=0.01), None, None) == OK
    assert lib.qbn_validate_async(T(CKE, 4, 96, scale2=0.01), B, None) == SHAPE
    assert lib.qbn_validate_async(T(CKE, 4, 64, scale2=0.01), None, None) == NULL
