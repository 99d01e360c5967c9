"""The Python binding refuses, before anything is launched, every tensor that
holds fewer bytes than the call would read or write through its raw pointer
(the C ABI takes plain pointers and cannot check). These run on the CPU: the
size checks come before the device checks, so an undersized host tensor is
refused for its size ("needs ... bytes"), a correctly sized one for not
being a device tensor."""
import pytest
import torch

import bit_block_quantized_nibble_amd as qbn

U8, I32, F32, BF16, I64 = torch.uint8, torch.int32, torch.float32, torch.bfloat16, torch.int64


def z(*shape, dtype=U8):
    return torch.zeros(*shape, dtype=dtype)


def nv(n=8, k=64, data=None, scales=None):
    return qbn.QTensor("nvfp4", n, k, z(n, k // 2) if data is None else data,
                       z(n, k // 16) if scales is None else scales, scale2=0.5)


def test_full_sized_host_tensors_reach_the_device_check():
    with pytest.raises(ValueError, match="device"):
        qbn.quantized_gemv(nv(), z(64, dtype=F32), z(8, dtype=F32))


@pytest.mark.parametrize("case", ["data", "scales", "gptq_zeros", "gptq_scales", "q4k_data", "q4_0_data"])
def test_undersized_weight_buffers(case):
    x, y = z(256, dtype=F32), z(64, dtype=F32)
    if case == "data":
        w = nv(data=z(8, 31))
    elif case == "scales":
        w = nv(scales=z(8 * 4 - 1))
    elif case == "gptq_zeros":
        w = qbn.QTensor("gptq4", 64, 256, z(32, 64, dtype=I32), z(2, 64, dtype=torch.float16), z(2, 63), group=128)
    elif case == "gptq_scales":
        w = qbn.QTensor("gptq4", 64, 256, z(32, 64, dtype=I32), z(1, 64, dtype=torch.float16), z(2, 64), group=128)
    elif case == "q4k_data":
        w = qbn.QTensor("q4_k", 64, 256, z(64 * 144 - 1))
    else:
        w = qbn.QTensor("q4_0", 64, 256, z(64, 8, 17))
    with pytest.raises(ValueError, match="needs"):
        qbn.quantized_gemv(w, x[:w.k], y)


def test_gemv_vectors():
    w = nv()
    with pytest.raises(ValueError, match="x holds"):
        qbn.quantized_gemv(w, z(63, dtype=F32), z(8, dtype=F32))
    with pytest.raises(ValueError, match="y holds"):
        qbn.quantized_gemv(w, z(64, dtype=F32), z(7, dtype=F32))
    with pytest.raises(TypeError):
        qbn.quantized_gemv(w, z(64, dtype=F32), z(8, dtype=BF16))
    with pytest.raises(ValueError, match="needs"):
        qbn.prepare_gemv(w, z(64, dtype=BF16)[:63], z(8, dtype=F32))


def test_gemm_matrices():
    w = qbn.QTensor("mxfp4", 16, 64, z(16, 32), z(16, 2))
    with pytest.raises(ValueError, match="x must be at least"):
        qbn.quantized_gemm(w, z(4, 63, dtype=BF16), z(4, 16, dtype=BF16))
    with pytest.raises(ValueError, match="y must be at least"):
        qbn.quantized_gemm(w, z(4, 64, dtype=BF16), z(3, 16, dtype=BF16))
    with pytest.raises(ValueError, match="y must be at least"):
        qbn.prepare_gemm(w, z(4, 64, dtype=BF16), z(4, 15, dtype=BF16))
    with pytest.raises(ValueError, match="xcodes holds"):
        qbn.quantized_gemm_mx(w, z(4, 31), z(4, 2), "mxfp4", z(4, 16, dtype=BF16))
    with pytest.raises(ValueError, match="xscales holds"):
        qbn.quantized_gemm_mx(w, z(4, 32), z(4, 1), "mxfp4", z(4, 16, dtype=BF16))


def test_dequantize_and_activation_quantizers():
    w = nv()
    with pytest.raises(ValueError, match="out holds"):
        qbn.dequantize(w, out=z(8, 63, dtype=F32))
    with pytest.raises(ValueError, match="out holds"):
        qbn.prepare_dequantize(w, z(8 * 64 - 1, dtype=BF16))
    with pytest.raises(ValueError, match="q holds"):
        qbn.quantize_q8(z(256, dtype=F32), q=z(255, dtype=torch.int8))
    with pytest.raises(ValueError, match="bsums holds"):
        qbn.quantize_q8(z(256, dtype=F32), bsums=z(7, dtype=I32))
    with pytest.raises(ValueError, match="codes holds"):
        qbn.quantize_mx(z(2, 64, dtype=F32), "mxfp4", codes=z(2, 31))
    qk = qbn.QTensor("q4_k", 4, 256, z(4 * 144))
    with pytest.raises(ValueError, match="bsums holds"):
        qbn.quantized_gemv_q8(qk, z(256, dtype=torch.int8), z(1, dtype=F32), z(7, dtype=I32), z(4, dtype=F32))
    with pytest.raises(ValueError, match="y holds"):
        qbn.quantized_gemv_q8(qk, z(256, dtype=torch.int8), z(1, dtype=F32), z(8, dtype=I32), z(3, dtype=F32))


def test_repack_destinations_and_status():
    src = qbn.QTensor("gptq4", 64, 256, z(32, 64, dtype=I32), z(2, 64, dtype=torch.float16), z(2, 64), group=128)
    with pytest.raises(ValueError, match="data holds"):
        qbn.repack(src, "awq4", data=z(256, 7, dtype=I32))
    with pytest.raises(ValueError, match="data holds"):
        qbn.repack(src, "q4_0", data=z(64 * 8 * 18 - 1))
    dst = qbn.repack_target(src, "q4_0")
    with pytest.raises(ValueError, match="status holds"):
        qbn.prepare_repack(src, dst, z(qbn.REPACK_STATUS_WORDS - 1, dtype=I64))


def test_gptq_metadata_and_permute():
    with pytest.raises(ValueError, match="src holds"):
        qbn.gptq_qzeros(z(2, 7, dtype=I32), 2, True, 64)
    with pytest.raises(ValueError, match="perm holds"):
        qbn.permute(z(64, dtype=F32), z(63, dtype=I32))
    with pytest.raises(ValueError, match="words_lo holds"):
        qbn.unpack_bits(z(2, dtype=I32), None, 32, 3)
