"""Seeded synthetic inputs for the twelve workloads (host numpy arrays).

This module holds no decoding, dot-product or repacking arithmetic: it only
draws random bytes and numbers with the distributions below and lays them
out in the documented buffer layouts. Both the CPU oracle and the HIP
library consume what it returns.

Generator: numpy.random.default_rng(seed), seed = 1000 + workload number by
default, draws in the order listed per workload. Packed 4-bit payloads are
drawn as uniform bytes: two independent codes uniform over 0..15 packed into
one byte give exactly a uniform byte, and eight such codes packed into a
32-bit word give a uniform word, so no packing step is needed here. Likewise
the 12 Q4_K metadata bytes are a bijective packing of eight 6-bit (scale, min)
pairs, so uniform bytes give every pair uniform over 0..63.
bfloat16 activations are rounded from binary32 by torch (round to nearest
even); fp16 scales are rounded by numpy (round to nearest even).

Workloads (n = output rows, k = reduction length):
  1  MXFP4 GEMV 256 x 1024: codes u8 [n][k/2]; E8M0 = 127 + U{-4..4} [n][k/32];
     x f32 N(0,1) [k].
  2  NVFP4 GEMV 4096 x 4096: codes u8 [n][k/2]; E4M3FN bytes U{0x18..0x50}
     (the 57 positive encodings with magnitude in [2^-4, 8]) [n][k/16];
     scale2 = float32(0.01); x bf16 N(0,1) [k].
  3  Q4_K GEMV 14336 x 4096: blocks [n][k/256][144] with fp16 d ~ U[1e-4,1e-3],
     fp16 dmin ~ U[0,1e-3], 12 uniform metadata bytes, 128 uniform code bytes;
     x f32 N(0,1) [k].
  4  MXFP4 GEMM, W 8192 x 8192 with E8M0 = 127 + U{-6..2}; X bf16 N(0,1)
     [2048][8192]; Y bf16 [2048][8192].
  5  int4 repack / dequant, K x N = 4096 x 11008, group 128: GPTQ qweight
     uniform u32 [K/8][N]; fp16 scales ~ U[1e-3,1e-2] [K/128][N]; zero points
     U{0..15} u8 [K/128][N].
  6  W4A8 decode GEMV, Q4_K 14336 x 4096 times int8-quantized activations:
     blocks and x drawn exactly as workload 3 (x f32 N(0,1) [k]); the
     activation codes are made from x by the library / the oracle.
  7  int4 decode GEMV, K x N = 4096 x 11008, group 128 (the weights of
     workload 5 in each int4 layout, drawn independently): GPTQ qweight
     uniform u32 [K/8][N]; AWQ qweight uniform u32 [K][N/8]; fp16 scales
     ~ U[1e-3,1e-2] [K/128][N]; zero points U{0..15} u8 [K/128][N]; Q4_0
     blocks [N][K/32][18] with fp16 d ~ U[1e-3,1e-2] and 16 uniform code
     bytes; x f32 N(0,1) [K].
  8  NVFP4 GEMV 4096 x 4096 in CKE's 36-byte split-half blocks: per block the
     four subscale bytes U{0x18..0x50} (drawn for all blocks first, as
     workload 2's scales), then 32 uniform code bytes; scale2 =
     float32(0.01); x bf16 N(0,1) [k].
  9  int4 prefill GEMM, K x N = 4096 x 11008, group 128, M = 2048: the
     weights drawn exactly as workload 7 (GPTQ, AWQ, scales, zero points,
     Q4_0 blocks, in that order, then workload 7's x, unused), then X bf16
     N(0,1) [M][K].
 10  INT4 symmetric encode, W bf16 N(0,1) [m][k] = [11008][4096], group 128.
 11  3-bit packing: values U{0..7} u8 [33554432].
 12  GPTQ act-order resolution, K x N = 4096 x 11008, group 128: qweight
     uniform u32 [K/8][N]; g_idx int32 [K] = (a uniform permutation of
     0..K-1) // 128, so every group holds exactly 128 rows, scattered as
     desc_act orders them.
"""
from __future__ import annotations

import numpy as np

SCALE2_NVFP4 = np.float32(0.01)

SHAPES = {
    1: dict(fmt="mxfp4", n=256, k=1024),
    2: dict(fmt="nvfp4", n=4096, k=4096),
    3: dict(fmt="q4_k", n=14336, k=4096),
    4: dict(fmt="mxfp4", n=8192, k=8192, m=2048),
    5: dict(fmt="gptq4", K=4096, N=11008, group=128),
    6: dict(fmt="q4_k", n=14336, k=4096),
    7: dict(fmt="int4", K=4096, N=11008, group=128),
    8: dict(fmt="nvfp4_cke", n=4096, k=4096),
    9: dict(fmt="int4", K=4096, N=11008, group=128, M=2048),
    10: dict(fmt="int4_sym", m=11008, k=4096, group=128),
    11: dict(fmt="pack", count=33554432, bits=3),
    12: dict(fmt="gptq4", K=4096, N=11008, group=128),
}


def _rng(seed):
    return np.random.default_rng(seed)


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round binary32 values to bfloat16 with torch (RNE); returns uint16 bits."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def mxfp4_weights(rng, n: int, k: int, exp_lo: int, exp_hi: int):
    codes = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    scales = (127 + rng.integers(exp_lo, exp_hi + 1, size=(n, k // 32))).astype(np.uint8)
    return codes, scales


def nvfp4_weights(rng, n: int, k: int):
    codes = rng.integers(0, 256, size=(n, k // 2), dtype=np.uint8)
    scales = rng.integers(0x18, 0x51, size=(n, k // 16)).astype(np.uint8)
    return codes, scales


def q4k_weights(rng, n: int, k: int):
    nb = n * (k // 256)
    d = rng.uniform(1e-4, 1e-3, size=nb).astype(np.float16)
    dmin = rng.uniform(0.0, 1e-3, size=nb).astype(np.float16)
    meta = rng.integers(0, 256, size=(nb, 12), dtype=np.uint8)
    qs = rng.integers(0, 256, size=(nb, 128), dtype=np.uint8)
    blocks = np.empty((nb, 144), dtype=np.uint8)
    blocks[:, 0:2] = d.view(np.uint8).reshape(nb, 2)
    blocks[:, 2:4] = dmin.view(np.uint8).reshape(nb, 2)
    blocks[:, 4:16] = meta
    blocks[:, 16:144] = qs
    return blocks.reshape(n, k // 256, 144)


def q4_0_weights(rng, n: int, k: int):
    nb = n * (k // 32)
    d = rng.uniform(1e-3, 1e-2, size=nb).astype(np.float16)
    qs = rng.integers(0, 256, size=(nb, 16), dtype=np.uint8)
    blocks = np.empty((nb, 18), dtype=np.uint8)
    blocks[:, 0:2] = d.view(np.uint8).reshape(nb, 2)
    blocks[:, 2:18] = qs
    return blocks.reshape(n, k // 32, 18)


def layout_probes(K: int, N: int):
    """Three K x N code matrices for checking a 4-bit layout both ways
    ("Bit Packing Architecture", Verification): a pattern whose value changes
    with the row and the column at different rates, so that reading the
    wrong axis or the wrong slot order gives different codes; seeded random
    codes; and every code 15, which sets the int32 sign bit of each word."""
    kk = np.arange(K, dtype=np.int64)[:, None]
    nn = np.arange(N, dtype=np.int64)[None, :]
    pattern = ((5 * kk + 11 * nn + kk // 16) % 16).astype(np.uint8)
    rand = _rng(4242).integers(0, 16, size=(K, N)).astype(np.uint8)
    return [pattern, rand, np.full((K, N), 15, np.uint8)]


def int4_affine(rng, K: int, N: int, group: int):
    qweight = rng.integers(0, 2**32, size=(K // 8, N), dtype=np.uint32)
    scales = rng.uniform(1e-3, 1e-2, size=(K // group, N)).astype(np.float16)
    zeros = rng.integers(0, 16, size=(K // group, N)).astype(np.uint8)
    return qweight, scales, zeros


def cke_blocks(rng, n: int, k: int):
    """CKE NVFP4 blocks u8 [n][k/64][36]: bytes 0-3 subscales U{0x18..0x50},
    bytes 4-35 uniform code bytes."""
    sub = rng.integers(0x18, 0x51, size=(n, k // 64, 4)).astype(np.uint8)
    codes = rng.integers(0, 256, size=(n, k // 64, 32), dtype=np.uint8)
    return np.ascontiguousarray(np.concatenate([sub, codes], axis=2))


def q4_0_blocks(rng, n: int, k: int):
    """Q4_0 blocks u8 [n][k/32][18]: fp16 d ~ U[1e-3, 1e-2] in bytes 0-1
    (little-endian), 16 uniform code bytes."""
    d = rng.uniform(1e-3, 1e-2, size=(n, k // 32)).astype(np.float16)
    blocks = np.zeros((n, k // 32, 18), np.uint8)
    blocks[:, :, :2] = d.view(np.uint8).reshape(n, k // 32, 2)
    blocks[:, :, 2:] = rng.integers(0, 256, size=(n, k // 32, 16), dtype=np.uint8)
    return blocks


def x_f32(rng, k: int):
    return rng.standard_normal(k).astype(np.float32)


def x_bf16(rng, k: int):
    return bf16_bits_from_f32(rng.standard_normal(k).astype(np.float32))


def workload(c: int, seed: int | None = None, n: int | None = None, k: int | None = None,
             m: int | None = None) -> dict:
    """Inputs of workload c (1..12). n / k / m override the shape (same
    distributions) so that tests can run the same recipe at small sizes."""
    seed = 1000 + c if seed is None else seed
    rng = _rng(seed)
    sh = dict(SHAPES[c])
    if c == 1:
        n = n or sh["n"]
        k = k or sh["k"]
        codes, scales = mxfp4_weights(rng, n, k, -4, 4)
        return dict(fmt="mxfp4", n=n, k=k, data=codes, scales=scales, scale2=1.0, x=x_f32(rng, k), seed=seed)
    if c == 2:
        n = n or sh["n"]
        k = k or sh["k"]
        codes, scales = nvfp4_weights(rng, n, k)
        return dict(fmt="nvfp4", n=n, k=k, data=codes, scales=scales, scale2=float(SCALE2_NVFP4),
                    x=x_bf16(rng, k), seed=seed)
    if c in (3, 6):
        n = n or sh["n"]
        k = k or sh["k"]
        blocks = q4k_weights(rng, n, k)
        return dict(fmt="q4_k", n=n, k=k, data=blocks, scales=None, scale2=1.0, x=x_f32(rng, k), seed=seed)
    if c == 4:
        n = n or sh["n"]
        k = k or sh["k"]
        m = m or sh["m"]
        codes, scales = mxfp4_weights(rng, n, k, -6, 2)
        X = bf16_bits_from_f32(rng.standard_normal((m, k)).astype(np.float32))
        return dict(fmt="mxfp4", n=n, k=k, m=m, data=codes, scales=scales, scale2=1.0, X=X, seed=seed)
    if c == 5:
        K = k or sh["K"]
        N = n or sh["N"]
        g = sh["group"]
        qweight, scales, zeros = int4_affine(rng, K, N, g)
        return dict(fmt="gptq4", K=K, N=N, group=g, qweight=qweight, scales=scales, zeros=zeros, seed=seed)
    if c in (7, 9):
        K = k or sh["K"]
        N = n or sh["N"]
        g = sh["group"]
        gptq = rng.integers(0, 2**32, size=(K // 8, N), dtype=np.uint32)
        awq = rng.integers(0, 2**32, size=(K, N // 8), dtype=np.uint32)
        scales = rng.uniform(1e-3, 1e-2, size=(K // g, N)).astype(np.float16)
        zeros = rng.integers(0, 16, size=(K // g, N)).astype(np.uint8)
        q4_0 = q4_0_blocks(rng, N, K)
        x = x_f32(rng, K)
        out = dict(fmt="int4", K=K, N=N, group=g, gptq=gptq, awq=awq, scales=scales, zeros=zeros, q4_0=q4_0, x=x,
                   seed=seed)
        if c == 9:
            M = m or sh["M"]
            out["M"] = M
            out["X"] = bf16_bits_from_f32(rng.standard_normal((M, K)).astype(np.float32))
        return out
    if c == 8:
        n = n or sh["n"]
        k = k or sh["k"]
        blocks = cke_blocks(rng, n, k)
        return dict(fmt="nvfp4_cke", n=n, k=k, data=blocks, scales=None, scale2=float(SCALE2_NVFP4),
                    x=x_bf16(rng, k), seed=seed)
    if c == 10:
        m = n or sh["m"]
        k = k or sh["k"]
        W = bf16_bits_from_f32(rng.standard_normal((m, k)).astype(np.float32))
        return dict(fmt="int4_sym", m=m, k=k, group=sh["group"], W=W, seed=seed)
    if c == 11:
        count = n or sh["count"]
        values = rng.integers(0, 1 << sh["bits"], size=count).astype(np.uint8)
        return dict(fmt="pack", count=count, bits=sh["bits"], values=values, seed=seed)
    if c == 12:
        K = k or sh["K"]
        N = n or sh["N"]
        g = sh["group"]
        qweight = rng.integers(0, 2**32, size=(K // 8, N), dtype=np.uint32)
        g_idx = (rng.permutation(K) // g).astype(np.int32)
        return dict(fmt="gptq4", K=K, N=N, group=g, qweight=qweight, g_idx=g_idx, seed=seed)
    raise ValueError("workload must be 1..12")
