"""CPU oracle for 4-bit block-quantized weights (test infrastructure only).

Plain, slow reference definitions of the MXFP4, NVFP4 (also in CKE's split-half
blocks), Q4_K and Q4_0 decoders,
of the GPTQ / AWQ / Q4_0 int4 layouts, of the dot products and GEMM entries built on them, and
of the W4A8 route (int8 activation quantization, Q4_K x int8 dot) and of the
integer-exact NVFP4 x Q8_K decode.
The arithmetic lives in ``qbn_oracle.c`` (plain C, gcc -O2, no SIMD
intrinsics, no fast-math); this module only compiles it and marshals numpy
arrays.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package. The library under ``bit_block_quantized_nibble_amd``
never imports it and shares no code with it.

Every function with an arithmetic definition is pinned by ``tests/test_oracle_*``
against facts the source pages fix (printed worked values, closed forms,
exhaustive enumeration against torch's float8 dtypes, brute force on tiny
inputs). No function here is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qbn_oracle.c")
_BUILD = os.path.join(_HERE, "_build")
_LIB_PATH = os.path.join(_BUILD, "liboracle.so")

MXFP4, NVFP4, Q4_K, Q4_0 = 1, 2, 3, 4
MXFP8 = 7  # activation format: E4M3FN elements, E8M0 scale per 32
NVFP4_CKE = 8  # NVFP4 in CKE's 36-byte split-half blocks of 64 weights

_lock = threading.Lock()
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle into oracle/_build/liboracle.so with gcc -O2."""
    os.makedirs(_BUILD, exist_ok=True)
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
               "-fvisibility=hidden", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.oracle_e2m1.argtypes = [ctypes.c_uint]
        lib.oracle_e2m1.restype = ctypes.c_double
        lib.oracle_e8m0.argtypes = [ctypes.c_uint]
        lib.oracle_e8m0.restype = ctypes.c_double
        lib.oracle_e4m3fn.argtypes = [ctypes.c_uint]
        lib.oracle_e4m3fn.restype = ctypes.c_double
        lib.oracle_f16.argtypes = [ctypes.c_uint]
        lib.oracle_f16.restype = ctypes.c_double
        lib.oracle_bf16_value.argtypes = [ctypes.c_uint]
        lib.oracle_bf16_value.restype = ctypes.c_double
        lib.oracle_bf16_rne.argtypes = [ctypes.c_float]
        lib.oracle_bf16_rne.restype = ctypes.c_uint
        lib.oracle_q4k_unpack_scales.argtypes = [P, P, P]
        lib.oracle_q4k_pack_scales.argtypes = [P, P, P]
        lib.oracle_pack_bits.argtypes = [P, I64, ctypes.c_int, P]
        lib.oracle_unpack_bits.argtypes = [P, I64, ctypes.c_int, P]
        for name in ("oracle_gptq_pack", "oracle_gptq_unpack", "oracle_awq_pack", "oracle_awq_unpack"):
            getattr(lib, name).argtypes = [P, I64, I64, P]
        lib.oracle_q4_0_pack.argtypes = [P, P, I64, I64, P]
        lib.oracle_cke_pack.argtypes = [P, P, I64, I64, P]
        lib.oracle_cke_unpack.argtypes = [P, I64, I64, P, P]
        lib.oracle_q4_0_unpack.argtypes = [P, I64, I64, P, P]
        lib.oracle_affine_dequant.argtypes = [P, P, P, I64, I64, I64, P]
        lib.oracle_gemv_kn.argtypes = [P, I64, I64, P, ctypes.c_int, P, I64, P, P, P]
        lib.oracle_qzeros_unpack.argtypes = [P, I64, I64, ctypes.c_int, P]
        lib.oracle_qzeros_unpack.restype = ctypes.c_int
        lib.oracle_qzeros_pack.argtypes = [P, I64, I64, ctypes.c_int, P]
        lib.oracle_qzeros_pack.restype = ctypes.c_int
        lib.oracle_resolve_g_idx.argtypes = [P, I64, I64, P]
        lib.oracle_resolve_g_idx.restype = ctypes.c_int
        lib.oracle_e2m1_round.argtypes = [ctypes.c_double, ctypes.c_int]
        lib.oracle_e2m1_round.restype = ctypes.c_uint
        lib.oracle_nvfp4_quantize.argtypes = [P, ctypes.c_int, I64, I64, I64, ctypes.c_float, ctypes.c_int, P, P]
        lib.oracle_nvfp4_quantize.restype = ctypes.c_int
        lib.oracle_int4_sym_quantize.argtypes = [P, ctypes.c_int, I64, I64, I64, I64, P, P]
        lib.oracle_pack_planes.argtypes = [P, I64, ctypes.c_int, ctypes.c_int, P, P, P]
        lib.oracle_unpack_planes.argtypes = [P, P, I64, ctypes.c_int, ctypes.c_int, P, P]
        lib.oracle_dequant_rows.argtypes = [ctypes.c_int, P, P, ctypes.c_float, I64, P, I64, P]
        lib.oracle_dequant_rows.restype = ctypes.c_int
        lib.oracle_gemv_rows.argtypes = [ctypes.c_int, P, P, ctypes.c_float, I64, P, ctypes.c_int, P, I64,
                                         P, P, P, P]
        lib.oracle_gemv_rows.restype = ctypes.c_int
        lib.oracle_gemm_entries.argtypes = [ctypes.c_int, P, P, ctypes.c_float, I64, P, I64, P, P, I64,
                                            P, P, P, P]
        lib.oracle_gemm_entries.restype = ctypes.c_int
        lib.oracle_e2m1_nearest.argtypes = [ctypes.c_double, ctypes.c_double]
        lib.oracle_e2m1_nearest.restype = ctypes.c_uint
        lib.oracle_int4_sym_code.argtypes = [ctypes.c_double, ctypes.c_double]
        lib.oracle_int4_sym_code.restype = ctypes.c_uint
        lib.oracle_int4_sym_value.argtypes = [ctypes.c_uint]
        lib.oracle_int4_sym_value.restype = ctypes.c_int
        lib.oracle_q8_code.argtypes = [ctypes.c_float, ctypes.c_float]
        lib.oracle_q8_code.restype = ctypes.c_int
        lib.oracle_q8_quantize.argtypes = [P, ctypes.c_int, I64, P, P, P]
        lib.oracle_w4a8_term.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_double, P, P, ctypes.c_int,
                                         ctypes.POINTER(I64), ctypes.POINTER(I64)]
        lib.oracle_w4a8_term.restype = ctypes.c_double
        lib.oracle_q4k_w4a8_rows.argtypes = [P, I64, P, P, P, I64, P, P]
        lib.oracle_e2m1_q1.argtypes = [ctypes.c_uint]
        lib.oracle_e2m1_q1.restype = ctypes.c_int
        lib.oracle_e4m3fn_q9.argtypes = [ctypes.c_uint]
        lib.oracle_e4m3fn_q9.restype = I64
        lib.oracle_f16_rne.argtypes = [ctypes.c_float]
        lib.oracle_f16_rne.restype = ctypes.c_uint
        lib.oracle_nvfp4_a16q8_rows.argtypes = [P, P, ctypes.c_float, I64, P, P, P, I64, P, P]
        lib.oracle_e2m1_rne.argtypes = [ctypes.c_double]
        lib.oracle_e2m1_rne.restype = ctypes.c_uint
        lib.oracle_e4m3fn_rne.argtypes = [ctypes.c_double]
        lib.oracle_e4m3fn_rne.restype = ctypes.c_uint
        lib.oracle_mx_quantize.argtypes = [P, ctypes.c_int, I64, I64, I64, ctypes.c_int, P, P]
        lib.oracle_mx_quantize.restype = ctypes.c_int
        lib.oracle_mx_gemm_entries.argtypes = [P, P, I64, ctypes.c_int, P, P, P, P, I64, P, P]
        lib.oracle_mx_gemm_entries.restype = ctypes.c_int
        _lib = lib
        return lib


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(a.ctypes.data)


# ---------------------------------------------------------------- scalars

def e2m1(code: int) -> float:
    return _load().oracle_e2m1(code)


def e8m0(byte: int) -> float:
    return _load().oracle_e8m0(byte)


def e4m3fn(byte: int) -> float:
    return _load().oracle_e4m3fn(byte)


def f16(bits: int) -> float:
    return _load().oracle_f16(bits)


def bf16_value(bits: int) -> float:
    return _load().oracle_bf16_value(bits)


def bf16_rne(values) -> np.ndarray:
    """binary32 values -> bfloat16 bit patterns (uint16), round to nearest even."""
    lib = _load()
    v = np.ascontiguousarray(values, dtype=np.float32).ravel()
    out = np.empty(v.shape, dtype=np.uint16)
    for i, f in enumerate(v.tolist()):
        out[i] = lib.oracle_bf16_rne(f)
    return out.reshape(np.shape(values))


def bf16_rne_array(values: np.ndarray) -> np.ndarray:
    """Vector form of bf16_rne for large arrays; same rule, written with numpy
    integer operations so that big outputs can be compared in seconds."""
    u = np.ascontiguousarray(values, dtype=np.float32).view(np.uint32)
    is_nan = ((u & 0x7F800000) == 0x7F800000) & ((u & 0x007FFFFF) != 0)
    lsb = (u >> 16) & 1
    r = ((u + np.uint32(0x7FFF) + lsb) >> 16).astype(np.uint16)
    r = np.where(is_nan, ((u >> 16) | 0x40).astype(np.uint16), r)
    return r.astype(np.uint16)


def e2m1_nearest(w: float, s: float) -> int:
    return _load().oracle_e2m1_nearest(w, s)


def int4_sym_code(w: float, s: float) -> int:
    return _load().oracle_int4_sym_code(w, s)


def int4_sym_value(code: int) -> int:
    return _load().oracle_int4_sym_value(code)


# ---------------------------------------------------------------- Q4_K metadata

def q4k_unpack_scales(B) -> tuple[list[int], list[int]]:
    b = np.ascontiguousarray(np.asarray(B, dtype=np.uint8))
    assert b.size == 12
    s = np.zeros(8, dtype=np.uint32)
    m = np.zeros(8, dtype=np.uint32)
    _load().oracle_q4k_unpack_scales(_ptr(b), _ptr(s), _ptr(m))
    return s.tolist(), m.tolist()


def q4k_pack_scales(s, m) -> np.ndarray:
    sa = np.ascontiguousarray(np.asarray(s, dtype=np.uint32))
    ma = np.ascontiguousarray(np.asarray(m, dtype=np.uint32))
    out = np.zeros(12, dtype=np.uint8)
    _load().oracle_q4k_pack_scales(_ptr(sa), _ptr(ma), _ptr(out))
    return out


# ---------------------------------------------------------------- bit streams and layouts

def pack_bits(vals, bits: int) -> np.ndarray:
    v = np.ascontiguousarray(np.asarray(vals, dtype=np.uint32))
    words = np.zeros((v.size * bits + 31) // 32, dtype=np.uint32)
    _load().oracle_pack_bits(_ptr(v), v.size, bits, _ptr(words))
    return words


def unpack_bits(words, bits: int, count: int) -> np.ndarray:
    w = np.ascontiguousarray(np.asarray(words, dtype=np.uint32))
    out = np.zeros(count, dtype=np.uint32)
    _load().oracle_unpack_bits(_ptr(w), count, bits, _ptr(out))
    return out


def gptq_pack(q: np.ndarray) -> np.ndarray:
    """q u8 [K][N] codes -> GPTQ qweight as uint32 [K/8][N]."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    K, N = q.shape
    out = np.zeros((K // 8, N), dtype=np.uint32)
    _load().oracle_gptq_pack(_ptr(q), K, N, _ptr(out))
    return out


def gptq_unpack(qw: np.ndarray) -> np.ndarray:
    qw = np.ascontiguousarray(qw).view(np.uint32)
    K8, N = qw.shape
    out = np.zeros((K8 * 8, N), dtype=np.uint8)
    _load().oracle_gptq_unpack(_ptr(qw), K8 * 8, N, _ptr(out))
    return out


def awq_pack(q: np.ndarray) -> np.ndarray:
    """q u8 [K][N] codes -> AWQ qweight as uint32 [K][N/8]."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    K, N = q.shape
    out = np.zeros((K, N // 8), dtype=np.uint32)
    _load().oracle_awq_pack(_ptr(q), K, N, _ptr(out))
    return out


def awq_unpack(qw: np.ndarray) -> np.ndarray:
    qw = np.ascontiguousarray(qw).view(np.uint32)
    K, N8 = qw.shape
    out = np.zeros((K, N8 * 8), dtype=np.uint8)
    _load().oracle_awq_unpack(_ptr(qw), K, N8 * 8, _ptr(out))
    return out


def cke_pack(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Logical E2M1 codes u8 [n][k] and E4M3FN subscales u8 [n][k/16] ->
    CKE split-half NVFP4 blocks u8 [n][k/64][36] ("Why 4-Bit Quantization Is
    King", section 5: four subscales, then 32 code bytes; inside a 16-weight
    subblock the low nibbles of its eight bytes are weights 0-7 and the high
    nibbles weights 8-15)."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    n, k = c.shape
    assert k % 64 == 0
    s = np.ascontiguousarray(scales, dtype=np.uint8)
    assert s.shape == (n, k // 16)
    out = np.zeros((n, k // 64, 36), dtype=np.uint8)
    _load().oracle_cke_pack(_ptr(c), _ptr(s), n, k, _ptr(out))
    return out


def cke_unpack(blocks: np.ndarray, n: int, k: int) -> tuple[np.ndarray, np.ndarray]:
    """CKE blocks -> (logical codes u8 [n][k], subscales u8 [n][k/16])."""
    b = np.ascontiguousarray(blocks, dtype=np.uint8)
    assert b.size == n * (k // 64) * 36
    codes = np.zeros((n, k), dtype=np.uint8)
    scales = np.zeros((n, k // 16), dtype=np.uint8)
    _load().oracle_cke_unpack(_ptr(b), n, k, _ptr(codes), _ptr(scales))
    return codes, scales


def q4_0_pack(q: np.ndarray, d_bits: np.ndarray) -> np.ndarray:
    """q u8 [K][N], d_bits u16 [N][K/32] -> Q4_0 blocks u8 [N][K/32][18]."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    K, N = q.shape
    d = np.ascontiguousarray(d_bits, dtype=np.uint16)
    assert d.shape == (N, K // 32)
    out = np.zeros((N, K // 32, 18), dtype=np.uint8)
    _load().oracle_q4_0_pack(_ptr(q), _ptr(d), K, N, _ptr(out))
    return out


def q4_0_unpack(blocks: np.ndarray, K: int, N: int) -> tuple[np.ndarray, np.ndarray]:
    b = np.ascontiguousarray(blocks, dtype=np.uint8)
    assert b.size == N * (K // 32) * 18
    q = np.zeros((K, N), dtype=np.uint8)
    d = np.zeros((N, K // 32), dtype=np.uint16)
    _load().oracle_q4_0_unpack(_ptr(b), K, N, _ptr(q), _ptr(d))
    return q, d


def affine_dequant(q: np.ndarray, scale_bits: np.ndarray, zeros: np.ndarray, group: int) -> np.ndarray:
    """w[k][n] = s[k/g][n] * (q[k][n] - z[k/g][n]) as binary32, [K][N]."""
    q = np.ascontiguousarray(q, dtype=np.uint8)
    K, N = q.shape
    s = np.ascontiguousarray(scale_bits, dtype=np.uint16)
    z = np.ascontiguousarray(zeros, dtype=np.uint8)
    assert s.shape == (K // group, N) and z.shape == (K // group, N)
    out = np.zeros((K, N), dtype=np.float32)
    _load().oracle_affine_dequant(_ptr(q), _ptr(s), _ptr(z), K, N, group, _ptr(out))
    return out


def qzeros_unpack(qz: np.ndarray, version: int) -> np.ndarray:
    """GPTQ qzeros uint32 [G][N/8] -> logical zero points u8 [G][N]."""
    q = np.ascontiguousarray(qz).view(np.uint32)
    G, N8 = q.shape
    out = np.zeros((G, N8 * 8), np.uint8)
    if _load().oracle_qzeros_unpack(_ptr(q), G, N8 * 8, version, _ptr(out)):
        raise ValueError("qzeros version must be 1 or 2")
    return out


def qzeros_pack(zeros: np.ndarray, version: int) -> np.ndarray:
    """Logical zero points u8 [G][N] -> GPTQ qzeros uint32 [G][N/8]."""
    z = np.ascontiguousarray(zeros, dtype=np.uint8)
    G, N = z.shape
    out = np.zeros((G, N // 8), np.uint32)
    if _load().oracle_qzeros_pack(_ptr(z), G, N, version, _ptr(out)):
        raise ValueError("qzeros version must be 1 or 2")
    return out


def resolve_g_idx(g_idx: np.ndarray, group: int):
    """(status, perm int32 [K]): rows ordered by group, stable; status 0,
    -1 (a g_idx out of range) or -2 (a group without exactly `group` rows)."""
    g = np.ascontiguousarray(g_idx, dtype=np.int32)
    perm = np.zeros(g.size, np.int32)
    rc = _load().oracle_resolve_g_idx(_ptr(g), g.size, group, _ptr(perm))
    return rc, perm


def gemv_kn(W: np.ndarray, x: np.ndarray, cols):
    """(y, S) in binary64 for columns cols of a [K][N] binary32 weight:
    y = x @ W[:, cols], S = |x| @ |W[:, cols]|. x float32 or bfloat16 bits."""
    Wc = np.ascontiguousarray(W, dtype=np.float32)
    K, N = Wc.shape
    xa = np.ascontiguousarray(x)
    if xa.dtype == np.float32:
        xdt = 0
    elif xa.dtype == np.uint16:
        xdt = 1
    else:
        raise TypeError("x must be float32 or bfloat16 bits (uint16)")
    assert xa.size == K
    c = np.ascontiguousarray(np.asarray(cols, dtype=np.int64))
    y = np.zeros(c.size, np.float64)
    sa = np.zeros(c.size, np.float64)
    xscr = np.zeros(K, np.float64)
    _load().oracle_gemv_kn(_ptr(Wc), K, N, _ptr(xa), xdt, _ptr(c), c.size, _ptr(y), _ptr(sa), _ptr(xscr))
    return y, sa


def int4_gemv(fmt: str, data: np.ndarray, scale_bits: np.ndarray, zeros: np.ndarray, group: int, x: np.ndarray,
              cols):
    """(y, S) for an int4 K x N weight: fmt "gptq4" (int32 [K/8][N]) or
    "awq4" (int32 [K][N/8]), unpacked to the logical matrix, dequantized as
    s * (q - z), then y[c] = sum_k w[k][c] x[k]."""
    q = gptq_unpack(data) if fmt == "gptq4" else awq_unpack(data)
    sb = np.asarray(scale_bits)
    sb = sb.view(np.uint16) if sb.dtype == np.float16 else sb
    return gemv_kn(affine_dequant(q, sb, zeros, group), x, cols)


def int4_gemm_entries(fmt: str, data: np.ndarray, scale_bits, zeros, group: int, X_bits: np.ndarray, ms, ns):
    """(Y, S) in binary64 for entries (ms[i], ns[i]) of Y = X @ W_hat with X
    bfloat16 bits [M][K] and an int4 K x N weight: "gptq4" / "awq4" (data as
    for int4_gemv, w = s * (q - z)) or "q4_0" (blocks u8 [N][K/32][18],
    w = d * (q - 8)). Entry (m, n) is the dot of row m of X with column n of
    W_hat, the same sum as the GEMV of that row."""
    X = np.ascontiguousarray(X_bits, dtype=np.uint16)
    K = X.shape[1]
    ms = np.asarray(ms, dtype=np.int64)
    ns = np.asarray(ns, dtype=np.int64)
    if fmt == "q4_0":
        return gemm_entries(Q4_0, data, None, 1.0, K, X, ms, ns)
    q = gptq_unpack(data) if fmt == "gptq4" else awq_unpack(data)
    sb = np.asarray(scale_bits)
    sb = sb.view(np.uint16) if sb.dtype == np.float16 else sb
    W = affine_dequant(q, sb, zeros, group)
    y = np.zeros(ms.size, np.float64)
    sa = np.zeros(ms.size, np.float64)
    for m in np.unique(ms):
        sel = np.nonzero(ms == m)[0]
        y[sel], sa[sel] = gemv_kn(W, X[m], ns[sel])
    return y, sa


# ---------------------------------------------------------------- dequant and dots

def _scales_or_null(scales):
    if scales is None:
        return None, ctypes.c_void_p(0)
    s = np.ascontiguousarray(scales, dtype=np.uint8)
    return s, _ptr(s)


def dequant_rows(fmt: int, data: np.ndarray, scales, scale2: float, k: int, rows) -> np.ndarray:
    """Dequantized rows [len(rows)][k] (binary32) of an n x k weight."""
    d = np.ascontiguousarray(data).view(np.uint8)
    s_keep, s_ptr = _scales_or_null(scales)
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    out = np.zeros((r.size, k), dtype=np.float32)
    rc = _load().oracle_dequant_rows(fmt, _ptr(d), s_ptr, scale2, k, _ptr(r), r.size, _ptr(out))
    if rc:
        raise ValueError("oracle: unsupported format %r" % fmt)
    return out


def gemv_rows(fmt: int, data, scales, scale2: float, k: int, x: np.ndarray, rows):
    """(y, S) in binary64 for the chosen rows: y = W_hat[rows] @ x and
    S = |W_hat[rows]| @ |x|. x is float32 or bfloat16 bits (uint16)."""
    d = np.ascontiguousarray(data).view(np.uint8)
    s_keep, s_ptr = _scales_or_null(scales)
    xa = np.ascontiguousarray(x)
    if xa.dtype == np.float32:
        xdt = 0
    elif xa.dtype == np.uint16:
        xdt = 1
    else:
        raise TypeError("x must be float32 or bfloat16 bits (uint16)")
    assert xa.size == k
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    y = np.zeros(r.size, dtype=np.float64)
    sa = np.zeros(r.size, dtype=np.float64)
    wscr = np.zeros(k, dtype=np.float32)
    xscr = np.zeros(k, dtype=np.float64)
    rc = _load().oracle_gemv_rows(fmt, _ptr(d), s_ptr, scale2, k, _ptr(xa), xdt, _ptr(r), r.size,
                                  _ptr(y), _ptr(sa), _ptr(wscr), _ptr(xscr))
    if rc:
        raise ValueError("oracle: unsupported format %r" % fmt)
    return y, sa


def gemm_entries(fmt: int, data, scales, scale2: float, k: int, X_bits: np.ndarray, ms, ns):
    """(Y, S) in binary64 for entries (ms[i], ns[i]) of X @ W_hat^T, X bf16 bits [M][k]."""
    d = np.ascontiguousarray(data).view(np.uint8)
    s_keep, s_ptr = _scales_or_null(scales)
    X = np.ascontiguousarray(X_bits, dtype=np.uint16)
    ms = np.asarray(ms, dtype=np.int64)
    ns = np.asarray(ns, dtype=np.int64)
    order = np.argsort(ns, kind="stable")
    ms_o = np.ascontiguousarray(ms[order])
    ns_o = np.ascontiguousarray(ns[order])
    y = np.zeros(ms.size, dtype=np.float64)
    sa = np.zeros(ms.size, dtype=np.float64)
    wscr = np.zeros(k, dtype=np.float32)
    xscr = np.zeros(k, dtype=np.float64)
    rc = _load().oracle_gemm_entries(fmt, _ptr(d), s_ptr, scale2, k, _ptr(X), X.shape[1], _ptr(ms_o),
                                     _ptr(ns_o), ms.size, _ptr(y), _ptr(sa), _ptr(wscr), _ptr(xscr))
    if rc:
        raise ValueError("oracle: unsupported format %r" % fmt)
    y_out = np.empty_like(y)
    s_out = np.empty_like(sa)
    y_out[order] = y
    s_out[order] = sa
    return y_out, s_out


# ---------------------------------------------------------------- W4A8 (Q4_K x int8 activations)

def q8_code(x: float, inv: float) -> int:
    """One int8 activation code: RNE(binary32(x * inv)) limited to [-127, 127]."""
    return _load().oracle_q8_code(x, inv)


def q8_quantize(x: np.ndarray):
    """(q int8 [k], d float32 [k/256], bsums int32 [k/32]) of f32 or bf16-bit x."""
    xa = np.ascontiguousarray(x)
    if xa.dtype == np.float32:
        xdt = 0
    elif xa.dtype == np.uint16:
        xdt = 1
    else:
        raise TypeError("x must be float32 or bfloat16 bits (uint16)")
    k = xa.size
    if k % 256:
        raise ValueError("k must be a multiple of 256")
    q = np.zeros(k, np.int8)
    d = np.zeros(k // 256, np.float32)
    bs = np.zeros(k // 32, np.int32)
    _load().oracle_q8_quantize(_ptr(xa), xdt, k, _ptr(q), _ptr(d), _ptr(bs))
    return q, d, bs


def w4a8_term(step: float, offset: float, sx: float, qw, qx):
    """(value, integer dot, code sum) of one sub-block in the W4A8 identity."""
    a = np.ascontiguousarray(np.asarray(qw, dtype=np.int32))
    b = np.ascontiguousarray(np.asarray(qx, dtype=np.int32))
    assert a.size == b.size
    idot = ctypes.c_int64()
    csum = ctypes.c_int64()
    v = _load().oracle_w4a8_term(step, offset, sx, _ptr(a), _ptr(b), a.size, ctypes.byref(idot), ctypes.byref(csum))
    return v, idot.value, csum.value


def q4k_w4a8_rows(blocks, k: int, q: np.ndarray, d: np.ndarray, rows):
    """(y, S) in binary64 for the chosen rows of a Q4_K weight times the
    int8-quantized activation d[i // 256] * q[i]."""
    blk = np.ascontiguousarray(blocks).view(np.uint8)
    qa = np.ascontiguousarray(q, dtype=np.int8)
    da = np.ascontiguousarray(d, dtype=np.float32)
    assert qa.size == k and da.size == k // 256
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    y = np.zeros(r.size, np.float64)
    sa = np.zeros(r.size, np.float64)
    _load().oracle_q4k_w4a8_rows(_ptr(blk), k, _ptr(qa), _ptr(da), _ptr(r), r.size, _ptr(y), _ptr(sa))
    return y, sa


# ---------------------------------------------------------------- NVFP4 x Q8_K, integer-exact

def e2m1_q1(code: int) -> int:
    return _load().oracle_e2m1_q1(code)


def e4m3fn_q9(byte: int) -> int:
    return _load().oracle_e4m3fn_q9(byte)


def f16_rne(values) -> np.ndarray:
    """binary16 bits (uint16) of binary32 values, round to nearest even."""
    lib = _load()
    v = np.ascontiguousarray(values, dtype=np.float32).ravel()
    return np.array([lib.oracle_f16_rne(float(t)) for t in v], dtype=np.uint16)


def nvfp4_a16q8_rows(codes, scales, scale2: float, k: int, q: np.ndarray, d: np.ndarray, rows):
    """(y binary32, y binary16 bits) of the integer-exact NVFP4 x Q8_K decode."""
    c = np.ascontiguousarray(codes).view(np.uint8)
    s = np.ascontiguousarray(scales).view(np.uint8)
    qa = np.ascontiguousarray(q, dtype=np.int8)
    da = np.ascontiguousarray(d, dtype=np.float32)
    assert qa.size == k and da.size == k // 256 and k % 256 == 0
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    y32 = np.zeros(r.size, np.float32)
    y16 = np.zeros(r.size, np.uint16)
    _load().oracle_nvfp4_a16q8_rows(_ptr(c), _ptr(s), scale2, k, _ptr(qa), _ptr(da), _ptr(r), r.size, _ptr(y32),
                                    _ptr(y16))
    return y32, y16


# ---------------------------------------------------------------- MX activations and the MX x MX product

def e2m1_rne(v: float) -> int:
    return _load().oracle_e2m1_rne(v)


def e4m3fn_rne(v: float) -> int:
    return _load().oracle_e4m3fn_rne(v)


def mx_quantize(X: np.ndarray, xfmt: int):
    """(codes, scales) of X [m][k] (float32, or bfloat16 bits as uint16) quantized
    to MX: xfmt MXFP4 -> E2M1 codes u8 [m][k/2]; MXFP8 -> E4M3FN bytes u8 [m][k];
    E8M0 scales u8 [m][k/32]."""
    Xa = np.ascontiguousarray(X)
    if Xa.ndim == 1:
        Xa = Xa[None, :]
    xdt = 1 if Xa.dtype == np.uint16 else 0
    if xdt == 0:
        Xa = np.ascontiguousarray(Xa, dtype=np.float32)
    m, k = Xa.shape
    assert k % 32 == 0
    codes = np.zeros((m, k // 2 if xfmt == MXFP4 else k), np.uint8)
    scales = np.zeros((m, k // 32), np.uint8)
    rc = _load().oracle_mx_quantize(_ptr(Xa), xdt, m, k, k, xfmt, _ptr(codes), _ptr(scales))
    if rc:
        raise ValueError("oracle: unsupported MX element format %r" % xfmt)
    return codes, scales


def mx_gemm_entries(wcodes, wscales, k: int, xfmt: int, xcodes, xscales, ms, ns):
    """(Y, S) in binary64 for entries (ms[i], ns[i]) of X_hat @ W_hat^T."""
    wc = np.ascontiguousarray(wcodes).view(np.uint8)
    ws = np.ascontiguousarray(wscales).view(np.uint8)
    xc = np.ascontiguousarray(xcodes).view(np.uint8)
    xs = np.ascontiguousarray(xscales).view(np.uint8)
    ms = np.ascontiguousarray(np.asarray(ms, dtype=np.int64))
    ns = np.ascontiguousarray(np.asarray(ns, dtype=np.int64))
    y = np.zeros(ms.size, np.float64)
    sa = np.zeros(ms.size, np.float64)
    rc = _load().oracle_mx_gemm_entries(_ptr(wc), _ptr(ws), k, xfmt, _ptr(xc), _ptr(xs), _ptr(ms), _ptr(ns), ms.size,
                                        _ptr(y), _ptr(sa))
    if rc:
        raise ValueError("oracle: unsupported MX element format %r" % xfmt)
    return y, sa


# ---------------------------------------------------------------- encode side

TIE_EVEN, TIE_LOWEST = 0, 1


def e2m1_round(v: float, tie: int) -> int:
    """Nearest E2M1 code, ties to the even code (0) or the lowest code (1)."""
    return int(_load().oracle_e2m1_round(float(v), int(tie)))


def _rows(X):
    Xa = np.ascontiguousarray(X)
    if Xa.dtype == np.float32:
        return Xa, 0
    if Xa.dtype == np.uint16:
        return Xa, 1
    raise TypeError("X must be float32 or bfloat16 bits (uint16)")


def nvfp4_quantize(X: np.ndarray, scale2: float, tie: int):
    """NVFP4 codes u8 [m][k/2] and E4M3FN scale bytes [m][k/16] of X [m][k]."""
    Xa, dt = _rows(X)
    m, k = Xa.shape
    codes = np.zeros((m, k // 2), np.uint8)
    scales = np.zeros((m, k // 16), np.uint8)
    if _load().oracle_nvfp4_quantize(_ptr(Xa), dt, m, k, k, float(np.float32(scale2)), int(tie), _ptr(codes),
                                     _ptr(scales)):
        raise ValueError("tie must be 0 or 1")
    return codes, scales


def int4_sym_quantize(W: np.ndarray, group: int):
    """Signed INT4 codes u8 [m][k/2] (two's complement nibbles, low = even)
    and binary32 scales [m][k/group] of W [m][k]."""
    Wa, dt = _rows(W)
    m, k = Wa.shape
    codes = np.zeros((m, k // 2), np.uint8)
    scales = np.zeros((m, k // group), np.float32)
    _load().oracle_int4_sym_quantize(_ptr(Wa), dt, m, k, k, group, _ptr(codes), _ptr(scales))
    return codes, scales


def pack_planes(vals, bits: int, lo: int):
    v = np.ascontiguousarray(vals, dtype=np.uint32)
    n = v.size
    lo_w = np.zeros((n * lo + 31) // 32, np.uint32)
    hi_w = np.zeros((n * (bits - lo) + 31) // 32, np.uint32)
    scr = np.zeros(n, np.uint32)
    _load().oracle_pack_planes(_ptr(v), n, bits, lo, _ptr(lo_w), _ptr(hi_w), _ptr(scr))
    return lo_w, hi_w


def unpack_planes(lo_w, hi_w, count: int, bits: int, lo: int) -> np.ndarray:
    a = np.ascontiguousarray(lo_w, dtype=np.uint32)
    b = np.ascontiguousarray(hi_w, dtype=np.uint32)
    out = np.zeros(count, np.uint32)
    scr = np.zeros(count, np.uint32)
    _load().oracle_unpack_planes(_ptr(a), _ptr(b), count, bits, lo, _ptr(out), _ptr(scr))
    return out
