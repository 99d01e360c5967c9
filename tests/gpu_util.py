"""Helpers shared by the GPU parity tests: move seeded host inputs to the
device, build QTensors, and compare against the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import bit_block_quantized_nibble_amd as qbn
import oracle

DEV = torch.device("cuda:0")
ORACLE_FMT = {"mxfp4": oracle.MXFP4, "nvfp4": oracle.NVFP4, "q4_k": oracle.Q4_K, "q4_0": oracle.Q4_0}


def say(*a):
    """Name the case before a GPU step, flushed, so a failing run shows it."""
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV)
    if a.dtype == np.uint32:
        return torch.from_numpy(a.view(np.int32)).to(DEV)
    return torch.from_numpy(a).to(DEV)


def x_dev(x: np.ndarray) -> torch.Tensor:
    if x.dtype == np.uint16:
        return dev(x).view(torch.bfloat16)
    return dev(x)


def host_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bits of a device tensor: uint32 for float32, uint16 for bfloat16."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.int32:
        return t.numpy().view(np.uint32)
    return t.numpy()


def qtensor(inp: dict) -> qbn.QTensor:
    fmt = inp["fmt"]
    if fmt in ("gptq4", "awq4"):
        return qbn.QTensor(fmt, inp["N"], inp["K"], dev(inp["qweight"]), dev(inp["scales"].view(np.uint16)),
                           dev(inp["zeros"]), group=inp["group"])
    return qbn.QTensor(fmt, inp["n"], inp["k"], dev(inp["data"]),
                       None if inp.get("scales") is None else dev(inp["scales"]), scale2=inp.get("scale2", 1.0))


def assert_f32_bits_equal(got_bits: np.ndarray, want: np.ndarray, what: str):
    want = np.ascontiguousarray(want, dtype=np.float32)
    wb = want.view(np.uint32)
    g = got_bits.reshape(wb.shape)
    gf = g.view(np.float32)
    both_nan = np.isnan(gf) & np.isnan(want)
    bad = (g != wb) & ~both_nan
    if bad.any():
        idx = np.argwhere(bad)[0]
        raise AssertionError("%s: %d of %d values differ; first at %s: got %r (0x%08x) want %r (0x%08x)" % (
            what, int(bad.sum()), bad.size, tuple(idx), float(gf[tuple(idx)]), int(g[tuple(idx)]),
            float(want[tuple(idx)]), int(wb[tuple(idx)])))


def assert_bf16_bits_equal(got_bits: np.ndarray, want_f32: np.ndarray, what: str):
    want_bits = oracle.bf16_rne_array(want_f32)
    g = got_bits.reshape(want_bits.shape)
    gnan = ((g & 0x7F80) == 0x7F80) & ((g & 0x7F) != 0)
    wnan = np.isnan(np.ascontiguousarray(want_f32, dtype=np.float32))
    bad = (g != want_bits) & ~(gnan & wnan)
    if bad.any():
        idx = np.argwhere(bad)[0]
        raise AssertionError("%s: %d of %d bf16 values differ; first at %s: got 0x%04x want 0x%04x" % (
            what, int(bad.sum()), bad.size, tuple(idx), int(g[tuple(idx)]), int(want_bits[tuple(idx)])))


def assert_within_tolerance(y: np.ndarray, y_ref: np.ndarray, s_ref: np.ndarray, what: str):
    """|y - y_ref| <= 1e-5 * sum|w x| + 1e-6, element by element."""
    y = np.asarray(y, dtype=np.float64)
    err = np.abs(y - y_ref)
    bound = 1e-5 * s_ref + 1e-6
    bad = ~(err <= bound)
    if bad.any():
        i = int(np.argwhere(bad)[0][0])
        raise AssertionError("%s: %d of %d outputs outside tolerance; first row %d: got %r want %r (bound %g)" % (
            what, int(bad.sum()), bad.size, i, float(y[i]), float(y_ref[i]), float(bound[i])))
    return float((err / bound).max()) if err.size else 0.0
