"""GPU: qbn_validate finds the first invalid scale / metadata element (the
fail-closed load-time check) and reports -1 on clean tensors."""
import numpy as np
import pytest
import torch

import bit_block_quantized_nibble_amd as qbn
import workloads
from gpu_util import DEV, dev, qtensor, say

pytestmark = pytest.mark.gpu


def test_validate_clean_workloads():
    for c in (1, 2, 3, 5):
        inp = workloads.workload(c, n=64 if c != 5 else 64, k=1024 if c != 5 else 256, seed=3)
        say("validate clean", c)
        assert qbn.validate(qtensor(inp)) == -1


def test_validate_mxfp4_nan_scale():
    inp = workloads.workload(1, n=40, k=1024, seed=4)
    s = inp["scales"].copy()
    s.reshape(-1)[[777, 301, 900]] = 0xFF
    inp["scales"] = s
    say("validate mxfp4")
    assert qbn.validate(qtensor(inp)) == 301


@pytest.mark.parametrize("bad", [0x7F, 0xFF])
def test_validate_nvfp4_nan_scale(bad):
    inp = workloads.workload(2, n=40, k=4096, seed=5)
    s = inp["scales"].copy()
    s.reshape(-1)[[5000, 4999]] = bad
    inp["scales"] = s
    say("validate nvfp4", bad)
    assert qbn.validate(qtensor(inp)) == 4999


def test_validate_q4k_nonfinite_header():
    inp = workloads.workload(3, n=8, k=4096, seed=6)
    blocks = inp["data"].copy()
    blocks.reshape(-1, 144)[70, 2:4] = np.array([np.inf], np.float16).view(np.uint8)
    blocks.reshape(-1, 144)[90, 0:2] = np.array([np.nan], np.float16).view(np.uint8)
    inp["data"] = blocks
    say("validate q4_k")
    assert qbn.validate(qtensor(inp)) == 70


def test_validate_q4_0_group_uniformity():
    n, k = 4, 256
    rng = np.random.default_rng(7)
    blocks = workloads.q4_0_weights(rng, n, k)
    # make every group of 4 blocks share d, then break one
    b = blocks.reshape(n, k // 32, 18)
    for r in range(n):
        for g0 in range(0, k // 32, 4):
            b[r, g0 + 1:g0 + 4, 0:2] = b[r, g0, 0:2]
    w = qbn.QTensor("q4_0", n, k, dev(blocks), group=128)
    say("validate q4_0 group")
    assert qbn.validate(w) == -1
    b[2, 6, 0] ^= 1
    w = qbn.QTensor("q4_0", n, k, dev(blocks), group=128)
    assert qbn.validate(w) == 2 * (k // 32) + 6
    w0 = qbn.QTensor("q4_0", n, k, dev(blocks), group=0)
    assert qbn.validate(w0) == -1


def test_validate_affine_companions():
    inp = workloads.workload(5, n=64, k=512, seed=8)
    z = inp["zeros"].copy()
    z.reshape(-1)[100] = 16
    inp["zeros"] = z
    say("validate gptq zeros")
    assert qbn.validate(qtensor(inp)) == 100
    s = inp["scales"].copy()
    s.reshape(-1)[50] = np.float16(np.inf)
    inp["scales"] = s
    assert qbn.validate(qtensor(inp)) == 50


def test_validate_async_and_sync_agree_and_status_codes():
    """qbn_validate_async leaves the index in device memory; qbn_validate
    waits, returns QBN_ERR_NAN_SCALE (7) on a finding and QBN_OK when clean,
    and hands the index back in host memory."""
    import ctypes

    inp = workloads.workload(2, n=48, k=512, seed=9)
    s = inp["scales"].copy()
    s.reshape(-1)[[1500, 700]] = 0x7F
    inp["scales"] = s
    w = qtensor(inp)
    say("validate async")
    out = qbn.validate_async(w)
    torch.cuda.synchronize()
    assert int(out.item()) == 700
    lib = qbn._load()
    host = ctypes.c_int64(123)
    ct = w._c()
    say("validate sync, raw status")
    assert lib.qbn_validate(ctypes.byref(ct), ctypes.byref(host), None) == 7
    assert host.value == 700
    clean = qtensor(workloads.workload(2, n=48, k=512, seed=9))
    ct2 = clean._c()
    assert lib.qbn_validate(ctypes.byref(ct2), ctypes.byref(host), None) == 0
    assert host.value == -1
    assert lib.qbn_validate(ctypes.byref(ct2), None, None) == 0  # the result pointer may be NULL
