#!/usr/bin/env python3
"""Throughput of the 4-bit block-quantized hot path on one MI355X.

Default workload (the headline one, the largest configuration): the MXFP4
prefill GEMM, W 8192 x 8192 (E2M1 codes, E8M0 scale per 32) times X bf16
2048 x 8192, fp32 accumulation, Y bf16; a step is one GEMM, the metric FP4
GEMM TFLOP/s against the dense bf16 matrix peak (the contraction runs on the
bf16 matrix cores: the activations are bf16). The same run also times the
two large decode GEMVs of the metric's GEMV half (Q4_K 14336 x 4096 and
NVFP4 4096 x 4096, listed under "also"). The other workloads (--workload)
measure the remaining kernels of the path on their own shapes.

Timing. Inputs are generated on the host once and copied to HBM before the
timed region. Each step reads its own copy of the weights, cycling through R
copies that together exceed 600 MB, so every launch streams its weights from
HBM rather than from the 32 MB of L2 or the 256 MB MALL. The K timed steps
are captured once into a HIP graph and replayed between two HIP events
(launch overhead is then the GPU's, not Python's): ms_per_step and value
come from that replay. Before it, the same graph is replayed untimed until
W steps have run (MFMA-heavy work needs ~0.1 s for its clocks to settle).
Outside the timed region the line also gives, as context, the step time
with one weight copy (cache-resident, not HBM) and a plain device copy's
rate on the same box. The CPU baseline times the CPU oracle on the same
workload and inputs, on one thread and on every host core, in the same unit.

The per-launch duration used for the roofline is the event-timed replay
divided by K: the graph issues the K launches back to back on one stream, so
this is each kernel's average duration plus the (small) inter-kernel gap.
Event pairs around individual launches are not used: each pair adds several
microseconds of marker overhead, more than the kernels themselves take.

roofline.traffic is the HBM-side traffic per launch measured with rocprofv3
(FETCH_SIZE and WRITE_SIZE in separate runs, scaled by the same counters on
a device copy of known size), read from profiles/traffic.json. It is
reported only while the kernel's source files hash to the value recorded
with the measurement; after any change to them it is null.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, AMD published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak, AMD published
FP4_MFMA_PEAK_TFLOPS = 10100.0  # MI355X dense FP4 matrix peak, AMD published (context only)
FP8_MFMA_PEAK_TFLOPS = 5000.0  # MI355X dense FP8 matrix peak, AMD published
ROTATE_BYTES = 600e6

# Algorithmic bytes / flops per step (read + write of every operand once).
WORKLOADS = {
    "nvfp4_gemv": dict(
        cfg=2, kind="gemv", unit="GB/s",
        desc="NVFP4 decode GEMV 4096x4096: E2M1 codes, E4M3FN scale per 16, f32 scale2=0.01, x bf16, y f32, batch 1",
        bytes=4096 * 2048 + 4096 * 256 + 4 + 4096 * 2 + 4096 * 4),
    "nvfp4_cke_gemv": dict(
        cfg=8, kind="gemv", unit="GB/s",
        desc="NVFP4 decode GEMV 4096x4096 in CKE's 36-byte split-half blocks of 64 (four E4M3FN subscales, "
             "32 code bytes), f32 scale2=0.01, x bf16, y f32, batch 1",
        bytes=4096 * 64 * 36 + 4 + 4096 * 2 + 4096 * 4),
    "mxfp4_gemv": dict(
        cfg=1, kind="gemv", unit="GB/s",
        desc="MXFP4 dequant-GEMV 256x1024: E2M1 codes, E8M0 scale per 32, x f32, y f32, batch 1",
        bytes=256 * 512 + 256 * 32 + 1024 * 4 + 256 * 4),
    "q4k_gemv": dict(
        cfg=3, kind="gemv", unit="GB/s",
        desc="Q4_K decode GEMV 14336x4096: 144-byte super-blocks of 256, x f32, y f32, batch 1",
        bytes=14336 * 16 * 144 + 4096 * 4 + 14336 * 4),
    "q4k_w4a8_gemv": dict(
        cfg=6, kind="w4a8", unit="GB/s", dtype="i8",
        desc="W4A8 decode: int8 quantization of x f32 [4096] (scale per 256) + Q4_K x int8 GEMV 14336x4096, y f32",
        bytes=14336 * 16 * 144 + 4096 * 4 + 2 * (4096 + 16 * 4 + 128 * 4) + 14336 * 4,
        kernel_bytes=14336 * 16 * 144 + 4096 + 16 * 4 + 128 * 4 + 14336 * 4),
    "nvfp4_a16q8_gemv": dict(
        cfg=2, kind="a16q8", unit="GB/s", dtype="i64",
        desc="integer-exact NVFP4 decode: Q8_K quantization of x bf16 [4096] + NVFP4 4096x4096 x int8 GEMV "
             "(exact block totals, pinned binary32 epilogue), y f16",
        bytes=4096 * 2048 + 4096 * 256 + 4096 * 2 + 2 * (4096 + 16 * 4 + 128 * 4) + 4096 * 2,
        kernel_bytes=4096 * 2048 + 4096 * 256 + 4096 + 16 * 4 + 4096 * 2),
    "gptq_gemv": dict(
        cfg=7, kind="int4gemv", fmt="gptq4", unit="GB/s",
        desc="GPTQ int4 decode GEMV 11008x4096 (int32 [K/8][N] packed along k, fp16 scales and u8 zero points per "
             "group of 128), x f32, y f32, batch 1",
        bytes=(4096 // 8) * 11008 * 4 + 32 * 11008 * 2 + 32 * 11008 + 4096 * 4 + 11008 * 4),
    "awq_gemv": dict(
        cfg=7, kind="int4gemv", fmt="awq4", unit="GB/s",
        desc="AWQ int4 decode GEMV 11008x4096 (int32 [K][N/8] packed along n in the 0,2,4,6,1,3,5,7 slot order, "
             "fp16 scales and u8 zero points per group of 128), x f32, y f32, batch 1",
        bytes=4096 * (11008 // 8) * 4 + 32 * 11008 * 2 + 32 * 11008 + 4096 * 4 + 11008 * 4),
    "q4_0_gemv": dict(
        cfg=7, kind="int4gemv", fmt="q4_0", unit="GB/s",
        desc="Q4_0 decode GEMV 11008x4096 (18-byte blocks of 32: fp16 d, w = d(q-8)), x f32, y f32, batch 1",
        bytes=11008 * 128 * 18 + 4096 * 4 + 11008 * 4),
    "nvfp4_encode": dict(
        cfg=2, kind="encode", unit="GB/s", dtype="f32",
        desc="NVFP4 encode of a bf16 4096x4096 weight (block scale E4M3(amax / 6 scale2), E2M1 ties to even, "
             "scale2 = 0.01): read bf16, write codes and scale bytes",
        bytes=4096 * 4096 * 2 + 4096 * 2048 + 4096 * 256),
    "mxfp4_gemm": dict(
        cfg=4, kind="gemm", unit="TFLOP/s", dtype="bf16",
        desc="MXFP4 prefill GEMM: W 8192x8192 (E2M1, E8M0 per 32) x X bf16 2048x8192 -> Y bf16, fp32 accumulate",
        flops=2.0 * 2048 * 8192 * 8192, bytes=8192 * 4096 + 8192 * 256 + 2048 * 8192 * 2 * 2),
    "gptq_gemm": dict(
        cfg=9, kind="int4gemm", fmt="gptq4", unit="TFLOP/s", dtype="bf16",
        desc="int4 prefill GEMM straight from GPTQ (int32 [K/8][N], fp16 scales, u8 zeros, group 128): "
             "X bf16 2048x4096 x W 4096x11008 -> Y bf16, bf16 MFMA on (q - z), fp32 group rescale",
        flops=2.0 * 2048 * 4096 * 11008, bytes=22544384 + 704512 + 352256 + 2048 * 4096 * 2 + 2048 * 11008 * 2),
    "awq_gemm": dict(
        cfg=9, kind="int4gemm", fmt="awq4", unit="TFLOP/s", dtype="bf16",
        desc="int4 prefill GEMM straight from AWQ (int32 [K][N/8], fp16 scales, u8 zeros, group 128): "
             "X bf16 2048x4096 x W 4096x11008 -> Y bf16, bf16 MFMA on (q - z), fp32 group rescale",
        flops=2.0 * 2048 * 4096 * 11008, bytes=22544384 + 704512 + 352256 + 2048 * 4096 * 2 + 2048 * 11008 * 2),
    "q4_0_gemm": dict(
        cfg=9, kind="int4gemm", fmt="q4_0", unit="TFLOP/s", dtype="bf16",
        desc="int4 prefill GEMM straight from GGUF Q4_0 (18-byte blocks of 32 along k): "
             "X bf16 2048x4096 x W 4096x11008 -> Y bf16, bf16 MFMA on (q - 8), fp32 rescale per block",
        flops=2.0 * 2048 * 4096 * 11008, bytes=25362432 + 2048 * 4096 * 2 + 2048 * 11008 * 2),
    "mxfp4_w4a4_gemm": dict(
        cfg=4, kind="mxgemm", unit="TFLOP/s", dtype="fp4",
        desc="MX-native W4A4 GEMM: OCP MX quantization of X bf16 2048x8192 to MXFP4 + W 8192x8192 MXFP4 on the "
             "block-scaled FP4 matrix cores -> Y bf16, fp32 accumulate",
        flops=2.0 * 2048 * 8192 * 8192,
        bytes=8192 * 4096 + 8192 * 256 + 2048 * 8192 * 2 + 2 * (2048 * 4096 + 2048 * 256) + 2048 * 8192 * 2,
        kernel_bytes=8192 * 4096 + 8192 * 256 + 2048 * 4096 + 2048 * 256 + 2048 * 8192 * 2),
    "gptq_to_awq": dict(
        cfg=5, kind="repack", unit="GB/s", src="gptq4", dst="awq4",
        desc="int4 repack GPTQ int32 [K/8][N] -> AWQ int32 [K][N/8], K x N = 4096 x 11008",
        bytes=2 * 22544384),
    "awq_to_q4_0": dict(
        cfg=5, kind="repack", unit="GB/s", src="awq4", dst="q4_0",
        desc="int4 repack AWQ int32 [K][N/8] + fp16 group-128 scales -> GGUF Q4_0 blocks, K x N = 4096 x 11008, "
             "every zero point 8 (the only one Q4_0 holds)",
        bytes=22544384 + 704512 + 352256 + 25362432,
        step_note="the step is the refusal scan of the 352,256 zero points (64 workgroups) and the repack kernel; "
                  "the bytes count the zero points once"),
    "gptq_dequant_bf16": dict(
        cfg=5, kind="dequant", unit="GB/s",
        desc="bulk dequant GPTQ (fp16 scales, u8 zeros, group 128) -> bf16 [K][N], K x N = 4096 x 11008",
        bytes=22544384 + 704512 + 352256 + 90177536),
    "int4_sym_encode": dict(
        cfg=10, kind="int4sym", unit="GB/s", dtype="f32",
        desc="signed INT4 symmetric encode of a bf16 11008x4096 weight, group 128 (s = amax / 7, q = clip(RNE(w/s), "
             "-8, 7)): read bf16, write two's-complement nibbles and binary32 scales",
        bytes=11008 * 4096 * 2 + 11008 * 2048 + 11008 * 32 * 4),
    "pack3_encode": dict(
        cfg=11, kind="pack", unit="GB/s", dtype="u8",
        desc="3-bit packing of 33,554,432 values (u8 in, one little-endian stream of 32-bit words out, fields "
             "straddling words)",
        bytes=33554432 + 33554432 * 3 // 8),
    "gptq_act_order": dict(
        cfg=12, kind="actorder", unit="GB/s", dtype="i32",
        desc="GPTQ act-order resolution, K x N = 4096 x 11008, group 128: rows ordered by group from g_idx, "
             "the packed int32 qweight permuted alike (two kernels: placement, then the row permute)",
        bytes=2 * 22544384 + 4096 * 4 + 4096 * 4 + 4),
}


def recorded_traffic(name):
    """Bytes per launch from profiles/traffic.json if the kernel sources are unchanged, else None."""
    import hashlib

    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(name)
    except (OSError, ValueError):
        return None
    if not rec:
        return None
    h = hashlib.sha256()
    for rel in rec["source"]:
        try:
            with open(os.path.join(ROOT, rel), "rb") as f:
                h.update(f.read())
        except OSError:
            return None
    return int(rec["traffic_bytes"]) if h.hexdigest() == rec["source_sha256"] else None


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=0, help="timed steps (default depends on the workload)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warmup steps, replayed from the captured graph (default 200; GEMMs 1500, "
                         "about 0.3 s, so their clocks have settled)")
    ap.add_argument("--workload", default="mxfp4_gemm", choices=sorted(WORKLOADS))
    ap.add_argument("--also", nargs="*", default=["q4k_gemv", "nvfp4_gemv"], choices=sorted(WORKLOADS),
                    help="further workloads timed in the same run and listed under \"also\"")
    ap.add_argument("--no-also", action="store_true", help="time only --workload")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the CPU oracle timing")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="CPU oracle time budget (half on one thread, half on all host cores)")
    return ap.parse_args()


def host_to_device(a, dev):
    import torch

    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev)
    if a.dtype == np.uint32:
        return torch.from_numpy(a.view(np.int32)).to(dev)
    return torch.from_numpy(a).to(dev)


def build_steps(name, spec, dev):
    """Return (step calls, one per weight copy; R; the inputs; the dominant
    kernel's own calls when a step launches more than one kernel, else None)."""
    import torch

    import bit_block_quantized_nibble_amd as qbn
    import workloads

    inp = workloads.workload(spec["cfg"])
    calls = []
    if spec["kind"] in ("w4a8", "a16q8"):
        n, k = inp["n"], inp["k"]
        wbytes = inp["data"].nbytes + (0 if inp["scales"] is None else inp["scales"].nbytes)
        R = max(1, math.ceil(ROTATE_BYTES / wbytes))
        d0 = host_to_device(inp["data"], dev)
        s0 = None if inp["scales"] is None else host_to_device(inp["scales"], dev)
        x = host_to_device(inp["x"], dev)
        if inp["x"].dtype == np.uint16:
            x = x.view(torch.bfloat16)
        q = torch.empty(k, dtype=torch.int8, device=dev)
        dx = torch.empty(k // 256, dtype=torch.float32, device=dev)
        bs = torch.empty(k // 32, dtype=torch.int32, device=dev)
        y = torch.empty(n, dtype=torch.float32 if spec["kind"] == "w4a8" else torch.float16, device=dev)
        quant = qbn.prepare_quantize_q8(x, q, dx, bs)
        gemvs = [qbn.prepare_gemv_q8(qbn.QTensor(inp["fmt"], n, k, d0.clone(), None if s0 is None else s0.clone(),
                                                 scale2=inp["scale2"]), q, dx, bs, y) for _ in range(R)]

        def step(g):
            def run():
                quant()
                g()
            return run

        return [step(g) for g in gemvs], R, inp, gemvs
    if spec["kind"] == "encode":
        n, k = inp["n"], inp["k"]
        # the weight to encode: the NVFP4 workload's dequantized values, as bf16 (generated on the device)
        w = qbn.QTensor("nvfp4", n, k, host_to_device(inp["data"], dev), host_to_device(inp["scales"], dev),
                        scale2=inp["scale2"])
        Wb = qbn.dequantize(w, dtype=torch.bfloat16)
        torch.cuda.synchronize()
        Wbits = Wb.view(torch.int16).cpu().numpy().view(np.uint16)  # the same weight on the host, for the oracle
        wbytes = Wb.numel() * 2
        R = max(1, math.ceil(ROTATE_BYTES / wbytes))
        srcs = [Wb.clone() for _ in range(R)]
        codes = torch.empty((n, k // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((n, k // 16), dtype=torch.uint8, device=dev)
        for W in srcs:
            calls.append(qbn.prepare_quantize_nvfp4(W, inp["scale2"], 0, codes, scales))
        return calls, R, dict(inp, Wbits=Wbits), None
    if spec["kind"] == "int4gemm":
        K, N, g, M = inp["K"], inp["N"], inp["group"], inp["M"]
        fmt = spec["fmt"]
        R = 2  # compute-bound: two weight copies suffice
        X = host_to_device(inp["X"], dev).view(torch.bfloat16)
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        if fmt == "q4_0":
            d0, s0, z0 = host_to_device(inp["q4_0"], dev), None, None
        else:
            d0 = host_to_device(inp["gptq"] if fmt == "gptq4" else inp["awq"], dev)
            s0 = host_to_device(inp["scales"].view(np.uint16), dev)
            z0 = host_to_device(inp["zeros"], dev)
        for _ in range(R):
            w = qbn.QTensor(fmt, N, K, d0.clone(), None if s0 is None else s0.clone(),
                            None if z0 is None else z0.clone(), group=g)
            calls.append(qbn.prepare_gemm(w, X, Y))
        return calls, R, inp, None
    if spec["kind"] == "int4gemv":
        K, N, g = inp["K"], inp["N"], inp["group"]
        fmt = spec["fmt"]
        x = host_to_device(inp["x"], dev)
        y = torch.empty(N, dtype=torch.float32, device=dev)
        if fmt == "q4_0":
            d0, s0, z0 = host_to_device(inp["q4_0"], dev), None, None
            wbytes = inp["q4_0"].nbytes
        else:
            d0 = host_to_device(inp["gptq"] if fmt == "gptq4" else inp["awq"], dev)
            s0 = host_to_device(inp["scales"].view(np.uint16), dev)
            z0 = host_to_device(inp["zeros"], dev)
            wbytes = d0.numel() * 4 + s0.numel() * 2 + z0.numel()
        R = max(1, math.ceil(ROTATE_BYTES / wbytes))
        for _ in range(R):
            w = qbn.QTensor(fmt, N, K, d0.clone(), None if s0 is None else s0.clone(),
                            None if z0 is None else z0.clone(), group=g)
            calls.append(qbn.prepare_gemv(w, x, y))
        return calls, R, inp, None
    if spec["kind"] == "gemv":
        n, k = inp["n"], inp["k"]
        wbytes = inp["data"].nbytes + (0 if inp["scales"] is None else inp["scales"].nbytes)
        R = max(1, math.ceil(ROTATE_BYTES / wbytes))
        d0 = host_to_device(inp["data"], dev)
        s0 = None if inp["scales"] is None else host_to_device(inp["scales"], dev)
        x = host_to_device(inp["x"], dev)
        if inp["x"].dtype == np.uint16:
            x = x.view(torch.bfloat16)
        y = torch.empty(n, dtype=torch.float32, device=dev)
        for _ in range(R):
            w = qbn.QTensor(inp["fmt"], n, k, d0.clone(), None if s0 is None else s0.clone(), scale2=inp["scale2"])
            calls.append(qbn.prepare_gemv(w, x, y))
        return calls, R, inp, None
    if spec["kind"] == "mxgemm":
        n, k, m = inp["n"], inp["k"], inp["m"]
        R = 2
        d0 = host_to_device(inp["data"], dev)
        s0 = host_to_device(inp["scales"], dev)
        X = host_to_device(inp["X"], dev).view(torch.bfloat16)
        xfmt = "mxfp4"
        xc = torch.empty((m, k // 2), dtype=torch.uint8, device=dev)
        xs = torch.empty((m, k // 32), dtype=torch.uint8, device=dev)
        Y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        quant = qbn.prepare_quantize_mx(X, xc, xs, xfmt)
        gemms = [qbn.prepare_gemm_mx(qbn.QTensor("mxfp4", n, k, d0.clone(), s0.clone()), xc, xs, Y, xfmt)
                 for _ in range(R)]

        def step(g):
            def run():
                quant()
                g()
            return run

        return [step(g) for g in gemms], R, inp, gemms
    if spec["kind"] == "gemm":
        n, k, m = inp["n"], inp["k"], inp["m"]
        R = 2
        d0 = host_to_device(inp["data"], dev)
        s0 = host_to_device(inp["scales"], dev)
        X = host_to_device(inp["X"], dev).view(torch.bfloat16)
        Y = torch.empty((m, n), dtype=torch.bfloat16, device=dev)
        for _ in range(R):
            w = qbn.QTensor("mxfp4", n, k, d0.clone(), s0.clone())
            calls.append(qbn.prepare_gemm(w, X, Y))
        return calls, R, inp, None
    if spec["kind"] in ("int4sym", "pack", "actorder"):
        lib = qbn._load()
        if spec["kind"] == "int4sym":
            m, k, g = inp["m"], inp["k"], inp["group"]
            W0 = host_to_device(inp["W"], dev).view(torch.bfloat16)
            R = max(1, math.ceil(ROTATE_BYTES / (m * k * 2)))
            codes = torch.empty((m, k // 2), dtype=torch.uint8, device=dev)
            scales = torch.empty((m, k // g), dtype=torch.float32, device=dev)
            for _ in range(R):
                W = W0.clone()
                calls.append(qbn.Prepared(lib.qbn_quantize_int4_sym,
                                          (qbn._ptr(W, "w"), qbn._DTYPES[torch.bfloat16], m, k, k, g,
                                           qbn._ptr(codes, "codes"), qbn._ptr(scales, "scales")),
                                          "qbn_quantize_int4_sym", dev, (W, codes, scales)))
        elif spec["kind"] == "pack":
            count, bits = inp["count"], inp["bits"]
            V0 = host_to_device(inp["values"], dev)
            R = max(1, math.ceil(ROTATE_BYTES / count))
            words = torch.empty((count * bits + 31) // 32, dtype=torch.int32, device=dev)
            for _ in range(R):
                V = V0.clone()
                calls.append(qbn.Prepared(lib.qbn_pack_bits,
                                          (qbn._ptr(V, "values"), count, bits, 0, qbn._ptr(words, "words"), None),
                                          "qbn_pack_bits", dev, (V, words)))
        else:
            K, N, g = inp["K"], inp["N"], inp["group"]
            Q0 = host_to_device(inp["qweight"], dev)
            gi = host_to_device(inp["g_idx"], dev)
            R = max(1, math.ceil(ROTATE_BYTES / (2 * Q0.numel() * 4)))
            out = torch.empty_like(Q0)
            perm = torch.empty(K, dtype=torch.int32, device=dev)
            status = torch.empty(1, dtype=torch.int32, device=dev)
            for _ in range(R):
                Q = Q0.clone()
                calls.append(qbn.Prepared(lib.qbn_gptq_resolve_g_idx,
                                          (qbn._ptr(Q, "qweight"), qbn._ptr(gi, "g_idx"), K, N, g, qbn._ptr(out, "out"),
                                           qbn._ptr(perm, "perm"), qbn._ptr(status, "status")),
                                          "qbn_gptq_resolve_g_idx", dev, (Q, gi, out, perm, status)))
        return calls, R, inp, None
    # cfg 5: repack / dequant from GPTQ (or from AWQ made by the library
    # itself). Q4_0 holds no zero point: its leg takes every zero point as 8.
    K, N, g = inp["K"], inp["N"], inp["group"]
    qw = host_to_device(inp["qweight"], dev)
    sc = host_to_device(inp["scales"].view(np.uint16), dev)
    zeros = np.full_like(inp["zeros"], 8) if spec.get("dst") == "q4_0" else inp["zeros"]
    zr = host_to_device(zeros, dev)
    per = spec["bytes"]
    R = max(1, math.ceil(ROTATE_BYTES / per))
    src_fmt = spec.get("src", "gptq4")
    base = qbn.QTensor("gptq4", N, K, qw, sc, zr, group=g)
    if src_fmt == "awq4":
        base = qbn.repack(base, "awq4")
        torch.cuda.synchronize()
    for _ in range(R):
        src = qbn.QTensor(src_fmt, N, K, base.data.clone(), sc.clone(), zr.clone(), group=g)
        if spec["kind"] == "dequant":
            out = torch.empty((K, N), dtype=torch.bfloat16, device=dev)
            calls.append(qbn.prepare_dequantize(src, out, layout="kn"))
        else:
            if spec["dst"] == "awq4":
                dst = qbn.QTensor("awq4", N, K, torch.empty((K, N // 8), dtype=torch.int32, device=dev), src.scales,
                                  src.zeros, group=g)
            else:
                dst = qbn.QTensor("q4_0", N, K, torch.empty((N, K // 32, 18), dtype=torch.uint8, device=dev))
            status = torch.empty(qbn.REPACK_STATUS_WORDS, dtype=torch.int64, device=dev)
            calls.append(qbn.prepare_repack(src, dst, status))
    return calls, R, inp, None


def oracle_unit(name, spec, inp):
    """One unit of oracle work on the workload's own inputs: a function
    f(rng) doing it and returning its amount in the metric's numerator (bytes
    or flops), and a description of the unit."""
    import oracle

    kind = spec["kind"]
    total = spec.get("flops", spec["bytes"])
    if kind in ("gemv", "w4a8", "a16q8", "encode"):
        n, k = inp["n"], inp["k"]
        rows = max(1, n // 64)

        def f(rng):
            r0 = int(rng.integers(0, n - rows + 1))
            rr = np.arange(r0, r0 + rows)
            if kind == "gemv":
                fmt = {"mxfp4": oracle.MXFP4, "nvfp4": oracle.NVFP4, "q4_k": oracle.Q4_K,
                       "nvfp4_cke": oracle.NVFP4_CKE}[inp["fmt"]]
                oracle.gemv_rows(fmt, inp["data"], inp["scales"], inp["scale2"], k, inp["x"], rr)
            elif kind == "w4a8":
                q, d, _ = oracle.q8_quantize(inp["x"])
                oracle.q4k_w4a8_rows(inp["data"], k, q, d, rr)
            elif kind == "a16q8":
                q, d, _ = oracle.q8_quantize(inp["x"])
                oracle.nvfp4_a16q8_rows(inp["data"], inp["scales"], inp["scale2"], k, q, d, rr)
            else:
                oracle.nvfp4_quantize(np.ascontiguousarray(inp["Wbits"][r0:r0 + rows]), inp["scale2"], 0)
            return total * rows / n
        return f, "slices of %d of the %d rows (activation quantization included where the step has it)" % (rows, n)
    if kind == "int4gemv":
        K, N, g, fmt = inp["K"], inp["N"], inp["group"], spec["fmt"]
        cols = max(1, N // 64)

        def f(rng):
            c0 = int(rng.integers(0, N - cols + 1))
            cc = np.arange(c0, c0 + cols)
            if fmt == "q4_0":
                oracle.gemv_rows(oracle.Q4_0, inp["q4_0"], None, 1.0, K, inp["x"], cc)
            else:
                oracle.int4_gemv(fmt, inp["gptq"] if fmt == "gptq4" else inp["awq"], inp["scales"], inp["zeros"], g,
                                 inp["x"], cc)
            return total * cols / N
        return f, "slices of %d of the %d outputs" % (cols, N)
    if kind == "gemm":
        n, k, m = inp["n"], inp["k"], inp["m"]

        def f(rng):
            mm = rng.integers(0, m, 16)
            nn = np.full(16, rng.integers(0, n))
            oracle.gemm_entries(oracle.MXFP4, inp["data"], inp["scales"], 1.0, k, inp["X"], mm, nn)
            return 2.0 * k * 16
        return f, "16 output entries of one column of the %dx%d output per call (2k flops each)" % (m, n)
    if kind == "mxgemm":
        n, k, m = inp["n"], inp["k"], inp["m"]

        def f(rng):
            i = int(rng.integers(0, m))
            xc, xs = oracle.mx_quantize(inp["X"][i:i + 1], oracle.MXFP4)
            oracle.mx_gemm_entries(inp["data"], inp["scales"], k, oracle.MXFP4, xc, xs, np.zeros(16, np.int64),
                                   rng.integers(0, n, 16))
            return 2.0 * k * 16
        return f, "one X row quantized and 16 of its output entries per call (2k flops each)"
    if kind == "int4gemm":
        K, N, g, M, fmt = inp["K"], inp["N"], inp["group"], inp["M"], spec["fmt"]
        data = inp["q4_0"] if fmt == "q4_0" else (inp["gptq"] if fmt == "gptq4" else inp["awq"])

        def f(rng):
            nn = rng.integers(0, N, 2)
            oracle.int4_gemm_entries(fmt, data, inp["scales"], inp["zeros"], g, inp["X"], np.repeat(np.arange(M), 2),
                                     np.tile(nn, M))
            return 2.0 * K * M * 2
        return f, "2 whole columns of the %dx%d output per call (2k flops per entry)" % (M, N)
    if kind == "int4sym":
        m, g = inp["m"], inp["group"]
        rows = max(1, m // 64)

        def f(rng):
            r0 = int(rng.integers(0, m - rows + 1))
            oracle.int4_sym_quantize(np.ascontiguousarray(inp["W"][r0:r0 + rows]), g)
            return total * rows / m
        return f, "slices of %d of the %d rows" % (rows, m)
    if kind == "pack":
        count, bits = inp["count"], inp["bits"]
        span = count // 64

        def f(rng):
            i0 = 32 * int(rng.integers(0, (count - span) // 32 + 1))
            oracle.pack_bits(inp["values"][i0:i0 + span], bits)
            return total * span / count
        return f, "slices of %d of the %d values" % (span, count)
    if kind == "actorder":
        K, N, g = inp["K"], inp["N"], inp["group"]
        cols = max(1, N // 64)

        def f(rng):
            c0 = int(rng.integers(0, N - cols + 1))
            _, perm = oracle.resolve_g_idx(inp["g_idx"], g)
            q = oracle.gptq_unpack(np.ascontiguousarray(inp["qweight"][:, c0:c0 + cols]))
            oracle.gptq_pack(np.ascontiguousarray(q[perm]))
            return total * cols / N
        return f, "the row order for all of K and the permuted rows of a slice of %d of the %d columns" % (cols, N)
    # repack / dequant through the oracle's logical matrix, on a slice of the
    # K x N matrix (whole groups, whole 8-column words)
    K, N, g = inp["K"], inp["N"], inp["group"]
    cols = 8 * max(1, N // 8 // 64)
    qw, sc, zr = inp["qweight"], inp["scales"].view(np.uint16), inp["zeros"]

    def f(rng):
        c0 = 8 * int(rng.integers(0, (N - cols) // 8 + 1))
        q = oracle.gptq_unpack(np.ascontiguousarray(qw[:, c0:c0 + cols]))
        if kind == "dequant":
            oracle.bf16_rne_array(oracle.affine_dequant(q, np.ascontiguousarray(sc[:, c0:c0 + cols]),
                                                        np.ascontiguousarray(zr[:, c0:c0 + cols]), g))
        elif spec["dst"] == "awq4":
            oracle.awq_pack(q)
        else:
            oracle.q4_0_pack(q, np.ascontiguousarray(np.repeat(sc[:, c0:c0 + cols].T, g // 32, axis=1)))
        return total * cols / N
    return f, "slices of %d of the %d columns of the %dx%d matrix" % (cols, N, K, N)


def _oracle_rate(f, seconds, threads):
    """Run f repeatedly on `threads` host threads for about `seconds` (the
    oracle's C calls release the interpreter lock); returns (amount done,
    elapsed seconds, calls)."""
    import concurrent.futures as cf

    t0 = time.perf_counter()
    deadline = t0 + seconds

    def worker(seed):
        rng = np.random.default_rng(seed)
        amount, calls = 0.0, 0
        while True:
            amount += f(rng)
            calls += 1
            if time.perf_counter() >= deadline:
                return amount, calls, time.perf_counter()

    with cf.ThreadPoolExecutor(threads) as ex:
        res = list(ex.map(worker, range(threads)))
    return sum(r[0] for r in res), max(r[2] for r in res) - t0, sum(r[1] for r in res)


def host_cores():
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(name, spec, inp, budget_s):
    """The oracle as it stands, timed on the host: first on one thread, then
    on every core this process may use (rows / columns / entries dealt to
    threads), each for half the budget, on the workload's own inputs."""
    f, what = oracle_unit(name, spec, inp)
    unit = spec["unit"]
    scale = 1e9 if unit == "GB/s" else 1e12
    amount1, t1, calls1 = _oracle_rate(f, budget_s / 2, 1)
    cores = host_cores()
    amount, t, calls = _oracle_rate(f, budget_s / 2, cores)
    return dict(value=round(amount / t / scale, 6), unit=unit, cores=cores, kind="oracle",
                sample="%s: %d calls in %.1f s on %d threads" % (what, calls, t, cores),
                one_core=dict(value=round(amount1 / t1 / scale, 6), cores=1,
                              sample="%d calls in %.1f s on one thread" % (calls1, t1)),
                cpu=cpu_model())


def environment():
    """What the numbers were taken on: GPU, clocks (rocm-smi, read right after the
    timed replays), ROCm and build flags."""
    import subprocess

    import torch

    from bit_block_quantized_nibble_amd import build as qbn_build

    props = torch.cuda.get_device_properties(0)
    env = {"gpu": props.name, "gcn_arch": getattr(props, "gcnArchName", ""),
           "compute_units": props.multi_processor_count, "torch": torch.__version__, "hip": torch.version.hip,
           "hipcc_flags": " ".join(f for f in qbn_build.CFLAGS if not f.startswith("-I")),
           "host_cpu": cpu_model(), "host_cores": host_cores()}
    try:
        with open("/opt/rocm/.info/version") as fh:
            env["rocm"] = fh.read().strip()
    except OSError:
        env["rocm"] = None
    try:
        r = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=20)
        clocks = [ln.strip() for ln in r.stdout.splitlines() if "clock level" in ln.lower() or "sclk" in ln.lower()
                  or "mclk" in ln.lower()]
        env["clocks"] = clocks[:8] if clocks else None
    except (OSError, subprocess.SubprocessError):
        env["clocks"] = None
    return env


def default_steps(kind):
    return 50 if kind in ("gemm", "int4gemm") else 200 if kind == "mxgemm" else 2000


def default_warmup(kind):
    return 1500 if kind in ("gemm", "mxgemm", "int4gemm") else 200


def measure(name, steps, warmup, dev):
    """Capture `steps` steps of the workload in one HIP graph, warm up by
    replaying it, time one replay between events (plus four more for the
    spread), and take the context figures (one weight copy; device copy)."""
    import torch

    spec = WORKLOADS[name]
    steps = steps or default_steps(spec["kind"])
    warmup = warmup if warmup is not None else default_warmup(spec["kind"])
    calls, R, inp, kcalls = build_steps(name, spec, dev)
    torch.cuda.synchronize()

    for i in range(min(R, 3)):
        calls[i]()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(steps):
            calls[i % R]()
    for _ in range(max(1, math.ceil(warmup / steps))):
        graph.replay()
    torch.cuda.synchronize()

    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = e0.elapsed_time(e1) / steps

    spread = []
    for _ in range(4):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        graph.replay()
        b.record()
        torch.cuda.synchronize()
        spread.append(a.elapsed_time(b) / steps)
    kernel_ms = ms_step
    if kcalls is not None:
        # the dominant kernel alone: K launches of it, captured and replayed
        # the same way (its inputs were written by the step graph above)
        kg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(kg):
            for i in range(steps):
                kcalls[i % R]()
        kg.replay()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        kg.replay()
        b.record()
        torch.cuda.synchronize()
        kernel_ms = a.elapsed_time(b) / steps
        del kg

    warm = torch.cuda.CUDAGraph()
    with torch.cuda.graph(warm):
        for i in range(steps):
            calls[0]()
    warm.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    warm.replay()
    b.record()
    torch.cuda.synchronize()
    warm_ms = a.elapsed_time(b) / steps
    del warm
    half = max(1 << 20, int(spec["bytes"]) // 2)
    nbuf = max(2, math.ceil(ROTATE_BYTES / (2 * half)))
    bufs = [(torch.empty(half, dtype=torch.uint8, device=dev), torch.empty(half, dtype=torch.uint8, device=dev))
            for _ in range(nbuf)]
    cg = torch.cuda.CUDAGraph()
    csteps = 200
    with torch.cuda.graph(cg):
        for i in range(csteps):
            dst, src = bufs[i % nbuf]
            dst.copy_(src)
    cg.replay()
    torch.cuda.synchronize()
    a.record()
    cg.replay()
    b.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * half / (a.elapsed_time(b) / csteps * 1e-3) / 1e9
    del cg, bufs, graph, calls, kcalls
    torch.cuda.synchronize()
    torch.cuda.empty_cache()

    if spec["kind"] in ("gemm", "mxgemm", "int4gemm"):
        peak = BF16_MFMA_PEAK_TFLOPS if spec["kind"] in ("gemm", "int4gemm") else FP4_MFMA_PEAK_TFLOPS
        value = spec["flops"] / (ms_step * 1e-3) / 1e12
        achieved = spec["flops"] / (kernel_ms * 1e-3) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 2), peak=peak, unit="TFLOP/s",
                    frac=round(achieved / peak, 4), traffic=recorded_traffic(name))
        metric = "int4 GEMM TFLOP/s (% MFMA peak)" if spec["kind"] == "int4gemm" else "FP4 GEMM TFLOP/s (% MFMA peak)"
    else:
        value = spec["bytes"] / (ms_step * 1e-3) / 1e9
        achieved = spec.get("kernel_bytes", spec["bytes"]) / (kernel_ms * 1e-3) / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved / HBM_PEAK_GBS, 4), traffic=recorded_traffic(name))
        metric = "quantized GEMV GB/s (% HBM peak)" if spec["kind"] in ("gemv", "w4a8", "a16q8", "int4gemv") else \
            "NVFP4 encode GB/s (% HBM peak)" if spec["kind"] == "encode" else \
            "INT4 encode GB/s (% HBM peak)" if spec["kind"] == "int4sym" else \
            "b-bit packing GB/s (% HBM peak)" if spec["kind"] == "pack" else \
            "act-order resolution GB/s (% HBM peak)" if spec["kind"] == "actorder" else (
            "int4 repack GB/s (% HBM peak)" if spec["kind"] == "repack" else "bulk dequant GB/s (% HBM peak)")
    config = {
        "workload": spec["desc"],
        "name": name,
        "seed": int(inp["seed"]),
        "rotating_copies": R,
        "step_bytes": spec["bytes"],
        **({"step_flops": spec["flops"]} if "flops" in spec else {}),
        **({"kernel_bytes": spec["kernel_bytes"], "kernel_note": spec.get("kernel_note", "roofline is the dominant "
            "kernel alone, timed in its own graph of K launches; value is the whole step")}
           if "kernel_bytes" in spec else {}),
        **({"step_note": spec["step_note"]} if "step_note" in spec else {}),
        "kernel_ms_per_launch": round(kernel_ms, 6),
        "kernel_ms_other_replays": [round(v, 6) for v in spread],
        "cache_resident_ms_per_launch": round(warm_ms, 6),
        "cache_resident_note": "one weight copy reused: served from MALL/L2, not HBM (context only)",
        "device_copy_gbs": round(copy_gbs, 1),
        "device_copy_note": "plain device-to-device copy of the step's byte count, read + write (context only)",
        **({"fp4_peak_frac": round(spec["flops"] / (kernel_ms * 1e-3) / 1e12 / FP4_MFMA_PEAK_TFLOPS, 4)}
           if spec["kind"] == "gemm" else {}),
        "timed_wall_s": round(wall, 4),
    }
    return dict(name=name, spec=spec, inp=inp, steps=steps, warmup=warmup, ms_step=ms_step, value=value,
                metric=metric, roofline=roof, config=config)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: nothing in this library uses a second GPU "
              "(the GEMV would shard by output rows, the GEMM by output columns). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    import torch

    import bit_block_quantized_nibble_amd as qbn

    if not os.path.exists(qbn.lib_path()):
        import __graft_entry__

        __graft_entry__.build()
    dev = torch.device("cuda:0")
    main_r = measure(args.workload, args.steps, args.warmup, dev)
    env = environment()  # after the timed replays, so the clock reading is that of a loaded GPU
    also = []
    for other in ([] if args.no_also else args.also):
        if other == args.workload:
            continue
        r = measure(other, 0, None, dev)
        also.append({"name": other, "metric": r["metric"], "value": round(r["value"], 2), "unit": r["spec"]["unit"],
                     "steps": r["steps"], "ms_per_step": round(r["ms_step"], 6), "roofline": r["roofline"],
                     "workload": r["spec"]["desc"]})
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(args.workload, main_r["spec"], main_r["inp"], args.cpu_seconds)
    spec = main_r["spec"]
    line = {
        "metric": main_r["metric"],
        "value": round(main_r["value"], 2),
        "unit": spec["unit"],
        "n_gpus": 1,
        "steps": main_r["steps"],
        "warmup": main_r["warmup"],
        "ms_per_step": round(main_r["ms_step"], 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.get("dtype", "f32"),
        "data": "synthetic",
        "config": {**main_r["config"], "environment": env},
        "roofline": main_r["roofline"],
        "cpu_baseline": cpu,
        "also": also,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
