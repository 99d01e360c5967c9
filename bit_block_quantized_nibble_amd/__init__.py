"""Python binding of libqbn: fused dequantize-and-dot over packed 4-bit
block-quantized weights (MXFP4, NVFP4, Q4_K), bulk dequantization of six
formats and bit-exact int4 layout repacks, on AMD MI355X (gfx950).

This module only marshals arguments: it checks that every tensor is a
device tensor holding at least the bytes the call will touch (the C ABI
takes raw pointers and cannot), turns the tensors into raw pointers, passes
torch's current HIP stream, and raises on a nonzero status.
Every step of the computation runs in the HIP kernels of libqbn.so; there is
no CPU or PyTorch fallback. The names mirror the C ABI in include/qbn.h
(``qbn_quantized_gemv`` -> ``quantized_gemv`` and so on).
"""
from __future__ import annotations

import ctypes
import os
import threading
from dataclasses import dataclass
from typing import Optional

import torch

__all__ = [
    "QTensor", "QbnError", "RepackRefused", "quantized_gemv", "quantized_gemm", "dequantize", "repack", "validate",
    "validate_async", "nbytes", "status_string", "lib_path", "FORMATS", "Prepared", "prepare_gemv", "prepare_gemm",
    "prepare_dequantize", "prepare_repack",
]

FORMATS = {"mxfp4": 1, "nvfp4": 2, "q4_k": 3, "q4_0": 4, "gptq4": 5, "awq4": 6, "nvfp4_cke": 8}
_F32, _BF16, _F16 = 0, 1, 2
REPACK_STATUS_WORDS = 65  # QBN_REPACK_STATUS_WORDS: the result word and the refusal scan's 64 partial results
_DTYPES = {torch.float32: _F32, torch.bfloat16: _BF16, torch.float16: _F16}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libqbn.so")
_lock = threading.Lock()
_lib = None

EXPORTED = (
    "qbn_abi_version", "qbn_tensor_struct_size", "qbn_status_string", "qbn_last_hip_error", "qbn_bytes",
    "qbn_quantized_gemv", "qbn_quantized_gemm", "qbn_dequantize", "qbn_repack", "qbn_repack_noalloc", "qbn_validate",
    "qbn_validate_async",
    "qbn_quantize_q8", "qbn_quantized_gemv_q8", "qbn_quantize_mx", "qbn_quantized_gemm_mx",
    "qbn_gptq_qzeros", "qbn_gptq_resolve_g_idx", "qbn_permute",
    "qbn_quantize_nvfp4", "qbn_quantize_int4_sym", "qbn_pack_bits", "qbn_unpack_bits",
)


class QbnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        detail = _load().qbn_status_string(status).decode()
        if status == 9:
            detail += " (hipError %d)" % _load().qbn_last_hip_error()
        super().__init__("%s: qbn status %d: %s" % (where, status, detail))


class RepackRefused(ValueError):
    """A Q4_0 repack found a weight the target cannot hold exactly (a zero
    point other than 8, or a group whose Q4_0 blocks disagree on d); nothing
    was written to the destination. `index` is the first offending index."""

    def __init__(self, index: int, what: str):
        self.index = index
        super().__init__("repack refused: %s (first offending index %d); the destination is untouched"
                         % (what, index))


class _CTensor(ctypes.Structure):
    _fields_ = [
        ("format", ctypes.c_int32), ("group", ctypes.c_int32), ("n", ctypes.c_int64), ("k", ctypes.c_int64),
        ("data", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("zeros", ctypes.c_void_p),
        ("scale2", ctypes.c_float), ("reserved", ctypes.c_int32),
    ]


def lib_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError("libqbn.so is not built; run `python -m bit_block_quantized_nibble_amd.build` "
                               "(or __graft_entry__.build()) first")
        lib = ctypes.CDLL(_LIB_PATH)
        P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        T = ctypes.POINTER(_CTensor)
        lib.qbn_abi_version.restype = I32
        lib.qbn_tensor_struct_size.restype = ctypes.c_size_t
        lib.qbn_status_string.argtypes = [I32]
        lib.qbn_status_string.restype = ctypes.c_char_p
        lib.qbn_last_hip_error.restype = I32
        lib.qbn_bytes.argtypes = [I32, I64, I64, I32, I32]
        lib.qbn_bytes.restype = I64
        lib.qbn_quantized_gemv.argtypes = [T, P, I32, P, I32, P]
        lib.qbn_quantized_gemv.restype = I32
        lib.qbn_quantized_gemm.argtypes = [T, I64, P, I32, I64, P, I32, I64, P]
        lib.qbn_quantized_gemm.restype = I32
        lib.qbn_dequantize.argtypes = [T, P, I32, I32, P]
        lib.qbn_dequantize.restype = I32
        lib.qbn_repack.argtypes = [T, T, P, P]
        lib.qbn_repack.restype = I32
        lib.qbn_repack_noalloc.argtypes = [T, T, P, P]
        lib.qbn_repack_noalloc.restype = I32
        lib.qbn_gptq_qzeros.argtypes = [P, P, I64, I64, I32, I32, P]
        lib.qbn_gptq_qzeros.restype = I32
        lib.qbn_gptq_resolve_g_idx.argtypes = [P, P, I64, I64, I32, P, P, P, P]
        lib.qbn_gptq_resolve_g_idx.restype = I32
        lib.qbn_permute.argtypes = [P, P, I64, I32, P, P]
        lib.qbn_permute.restype = I32
        lib.qbn_quantize_nvfp4.argtypes = [P, I32, I64, I64, I64, ctypes.c_float, I32, P, P, P]
        lib.qbn_quantize_nvfp4.restype = I32
        lib.qbn_quantize_int4_sym.argtypes = [P, I32, I64, I64, I64, I32, P, P, P]
        lib.qbn_quantize_int4_sym.restype = I32
        lib.qbn_pack_bits.argtypes = [P, I64, I32, I32, P, P, P]
        lib.qbn_pack_bits.restype = I32
        lib.qbn_unpack_bits.argtypes = [P, P, I64, I32, I32, P, P]
        lib.qbn_unpack_bits.restype = I32
        lib.qbn_validate.argtypes = [T, ctypes.POINTER(ctypes.c_int64), P]
        lib.qbn_validate.restype = I32
        lib.qbn_validate_async.argtypes = [T, P, P]
        lib.qbn_validate_async.restype = I32
        lib.qbn_quantize_q8.argtypes = [P, I32, I64, P, P, P, P]
        lib.qbn_quantize_q8.restype = I32
        lib.qbn_quantized_gemv_q8.argtypes = [T, P, P, P, P, I32, P]
        lib.qbn_quantized_gemv_q8.restype = I32
        lib.qbn_quantize_mx.argtypes = [P, I32, I64, I64, I64, I32, P, P, P]
        lib.qbn_quantize_mx.restype = I32
        lib.qbn_quantized_gemm_mx.argtypes = [T, I64, I32, P, P, P, I32, I64, P]
        lib.qbn_quantized_gemm_mx.restype = I32
        if lib.qbn_abi_version() != 2 or lib.qbn_tensor_struct_size() != ctypes.sizeof(_CTensor):
            raise RuntimeError("libqbn ABI mismatch: rebuild the library")
        _lib = lib
        return lib


def _ptr(t: Optional[torch.Tensor], name: str):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("%s must be a device (cuda) tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return ctypes.c_void_p(t.data_ptr())


def _ptr_rows(t: torch.Tensor, name: str):
    """Pointer to a 2-D matrix whose rows are contiguous but may sit inside a
    wider one (row stride >= columns, passed to the library as its leading
    dimension)."""
    if not t.is_cuda:
        raise ValueError("%s must be a device (cuda) tensor" % name)
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1) or (t.shape[0] > 1 and t.stride(0) < t.shape[1]):
        raise ValueError("%s must be 2-D with contiguous rows" % name)
    return ctypes.c_void_p(t.data_ptr())


def _need(t: Optional[torch.Tensor], nbytes: int, name: str):
    """Refuse, before any launch, a tensor that holds fewer bytes than the
    call will read or write through its pointer."""
    if nbytes <= 0:
        return
    if t is None:
        raise ValueError("%s is required" % name)
    have = t.numel() * t.element_size()
    if have < nbytes:
        raise ValueError("%s holds %d bytes; the call needs %d" % (name, have, nbytes))


def _need_dtype(t: torch.Tensor, dtypes, name: str):
    if t.dtype not in dtypes:
        raise TypeError("%s dtype %s (expected %s)" % (name, t.dtype, ", ".join(str(d) for d in dtypes)))


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


@dataclass
class QTensor:
    """A quantized weight W (n output rows x k inputs) in device memory.

    Buffers follow include/qbn.h: MXFP4 / NVFP4 data u8 [n][k/2] with scale
    bytes [n][k/32] / [n][k/16] (NVFP4 also takes scale2); Q4_K data u8
    [n][k/256][144]; Q4_0 data u8 [n][k/32][18]; GPTQ4 data int32 [k/8][n],
    AWQ4 data int32 [k][n/8], both with fp16 scales and u8 logical zero points
    [k/group][n]; NVFP4_CKE data u8 [n][k/64][36] split-half blocks (subscales
    inside the blocks, no scales tensor) with scale2.
    """
    format: str
    n: int
    k: int
    data: torch.Tensor
    scales: Optional[torch.Tensor] = None
    zeros: Optional[torch.Tensor] = None
    scale2: float = 1.0
    group: int = 0

    def check_sizes(self):
        """Every buffer must hold the bytes of its part (the library reads
        them through raw pointers and cannot check)."""
        if self.format not in FORMATS:
            raise ValueError("unknown format %r" % self.format)
        grp = int(self.group) if self.format in ("gptq4", "awq4") else 0
        for part, t, name in ((0, self.data, "data"), (1, self.scales, "scales"), (2, self.zeros, "zeros")):
            need = nbytes(self.format, int(self.n), int(self.k), grp, part)
            if need < 0:
                break  # invalid shape or group: the library reports it
            if t is not None or need > 0:
                _need(t, need, name)

    def _c(self) -> _CTensor:
        self.check_sizes()
        c = _CTensor()
        c.format = FORMATS[self.format]
        c.group = int(self.group)
        c.n = int(self.n)
        c.k = int(self.k)
        c.data = _ptr(self.data, "data")
        c.scales = _ptr(self.scales, "scales")
        c.zeros = _ptr(self.zeros, "zeros")
        c.scale2 = float(self.scale2)
        c.reserved = 0
        return c

    @property
    def device(self) -> torch.device:
        return self.data.device


def _check(status: int, where: str):
    if status != 0:
        raise QbnError(status, where)


def status_string(status: int) -> str:
    return _load().qbn_status_string(status).decode()


def nbytes(format: str, n: int, k: int, group: int = 0, part: int = 0) -> int:
    """Bytes of part 0 (data), 1 (scales) or 2 (zeros); -1 if invalid."""
    return int(_load().qbn_bytes(FORMATS[format], n, k, group, part))


def gptq_qzeros(src: torch.Tensor, version: int, to_logical: bool, n: int,
                dst: Optional[torch.Tensor] = None) -> torch.Tensor:
    """GPTQ qzeros int32 [groups][n/8] <-> logical zero points uint8 [groups][n]
    (version 1 stores z - 1, version 2 stores z)."""
    lib = _load()
    groups = src.shape[0]
    if dst is None:
        dst = (torch.empty((groups, n), dtype=torch.uint8, device=src.device) if to_logical
               else torch.empty((groups, n // 8), dtype=torch.int32, device=src.device))
    _need(src, groups * (n // 2 if to_logical else n), "src")
    _need(dst, groups * (n if to_logical else n // 2), "dst")
    _check(lib.qbn_gptq_qzeros(_ptr(src, "src"), _ptr(dst, "dst"), groups, n, int(version), int(bool(to_logical)),
                               _stream(src.device)), "qbn_gptq_qzeros")  # sizes checked above
    return dst


def gptq_resolve_g_idx(qweight: torch.Tensor, g_idx: torch.Tensor, group: int):
    """Act-order resolution: returns (qweight_out int32 [k/8][n], perm int32 [k],
    status int32 [1]) on the device; apply perm to the activations with permute()."""
    lib = _load()
    k, n = g_idx.numel(), qweight.shape[1]
    out = torch.empty_like(qweight)
    perm = torch.empty(k, dtype=torch.int32, device=qweight.device)
    status = torch.empty(1, dtype=torch.int32, device=qweight.device)
    _need(qweight, (k // 8) * n * 4, "qweight")
    _need(g_idx, 4 * k, "g_idx")
    _check(lib.qbn_gptq_resolve_g_idx(_ptr(qweight, "qweight"), _ptr(g_idx, "g_idx"), k, n, int(group),
                                      _ptr(out, "qweight_out"), _ptr(perm, "perm"), _ptr(status, "status"),
                                      _stream(qweight.device)), "qbn_gptq_resolve_g_idx")
    return out, perm, status


def permute(src: torch.Tensor, perm: torch.Tensor, dst: Optional[torch.Tensor] = None) -> torch.Tensor:
    """dst[i] = src[perm[i]] (float32, bfloat16 or float16 vectors)."""
    lib = _load()
    if src.dtype not in _DTYPES:
        raise TypeError("src dtype %s" % src.dtype)
    if dst is None:
        dst = torch.empty_like(src)
    _need(perm, 4 * src.numel(), "perm")
    _need(dst, src.numel() * src.element_size(), "dst")
    _check(lib.qbn_permute(_ptr(src, "src"), _ptr(perm, "perm"), src.numel(), _DTYPES[src.dtype], _ptr(dst, "dst"),
                           _stream(src.device)), "qbn_permute")
    return dst


def quantize_nvfp4(x: torch.Tensor, scale2: float, tie: int = 0):
    """NVFP4 encode of x [m][k] (float32 or bfloat16): (codes uint8 [m][k/2],
    E4M3FN scale bytes uint8 [m][k/16]); tie 0 ties-to-even, 1 lowest code."""
    lib = _load()
    m, k = x.shape if x.dim() == 2 else (0, 0)
    xp = _ptr_rows(x, "x")
    codes = torch.empty((m, k // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((m, k // 16), dtype=torch.uint8, device=x.device)
    ldx = x.stride(0) if m > 1 else k
    _check(lib.qbn_quantize_nvfp4(xp, _DTYPES.get(x.dtype, -1), m, k, ldx, float(scale2), int(tie),
                                  _ptr(codes, "codes"), _ptr(scales, "scales"), _stream(x.device)),
           "qbn_quantize_nvfp4")
    return codes, scales


def quantize_int4_sym(w: torch.Tensor, group: int):
    """Signed INT4 symmetric encode of w [m][k]: (codes uint8 [m][k/2],
    scales float32 [m][k/group])."""
    lib = _load()
    m, k = w.shape if w.dim() == 2 else (0, 0)
    wp = _ptr_rows(w, "w")
    codes = torch.empty((m, k // 2), dtype=torch.uint8, device=w.device)
    scales = torch.empty((m, k // group), dtype=torch.float32, device=w.device)
    ldw = w.stride(0) if m > 1 else k
    _check(lib.qbn_quantize_int4_sym(wp, _DTYPES.get(w.dtype, -1), m, k, ldw, int(group),
                                     _ptr(codes, "codes"), _ptr(scales, "scales"), _stream(w.device)),
           "qbn_quantize_int4_sym")
    return codes, scales


def pack_bits(values: torch.Tensor, bits: int, lo_bits: int = 0):
    """Pack uint8 values (one per element) into int32 word streams: one
    stream (lo_bits 0) or two bit planes. Returns (words_lo, words_hi or None)."""
    lib = _load()
    n = values.numel()
    w0 = lo_bits if lo_bits else bits
    lo = torch.empty((n * w0 + 31) // 32, dtype=torch.int32, device=values.device)
    hi = (torch.empty((n * (bits - lo_bits) + 31) // 32, dtype=torch.int32, device=values.device) if lo_bits
          else None)
    _check(lib.qbn_pack_bits(_ptr(values, "values"), n, int(bits), int(lo_bits), _ptr(lo, "words_lo"),
                             _ptr(hi, "words_hi"), _stream(values.device)), "qbn_pack_bits")
    return lo, hi


def unpack_bits(words_lo: torch.Tensor, words_hi: Optional[torch.Tensor], count: int, bits: int,
                lo_bits: int = 0) -> torch.Tensor:
    lib = _load()
    out = torch.empty(count, dtype=torch.uint8, device=words_lo.device)
    w0 = lo_bits if lo_bits else bits
    _need(words_lo, 4 * ((count * w0 + 31) // 32), "words_lo")
    if lo_bits:
        _need(words_hi, 4 * ((count * (bits - lo_bits) + 31) // 32), "words_hi")
    _check(lib.qbn_unpack_bits(_ptr(words_lo, "words_lo"), _ptr(words_hi, "words_hi"), count, int(bits),
                               int(lo_bits), _ptr(out, "values"), _stream(words_lo.device)), "qbn_unpack_bits")
    return out


def quantized_gemv(w: QTensor, x: torch.Tensor, y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """y = W_hat @ x (float32 [n]) for x float32 or bfloat16 [k]."""
    lib = _load()
    _need_dtype(x, (torch.float32, torch.bfloat16), "x")
    if y is None:
        y = torch.empty(w.n, dtype=torch.float32, device=w.device)
    _need_dtype(y, (torch.float32,), "y")
    _need(x, w.k * x.element_size(), "x")
    _need(y, w.n * 4, "y")
    ct = w._c()
    _check(lib.qbn_quantized_gemv(ctypes.byref(ct), _ptr(x, "x"), _DTYPES[x.dtype], _ptr(y, "y"),
                                  _DTYPES.get(y.dtype, -1), _stream(w.device)), "qbn_quantized_gemv")
    return y


def quantize_q8(x: torch.Tensor, q: Optional[torch.Tensor] = None, d: Optional[torch.Tensor] = None,
                bsums: Optional[torch.Tensor] = None):
    """int8 activation quantization of x (float32 or bfloat16 [k], k % 256 == 0):
    returns (q int8 [k], d float32 [k/256], bsums int32 [k/32])."""
    lib = _load()
    if x.dtype not in _DTYPES:
        raise TypeError("x dtype %s" % x.dtype)
    k = x.numel()
    if q is None:
        q = torch.empty(k, dtype=torch.int8, device=x.device)
    if d is None:
        d = torch.empty(k // 256, dtype=torch.float32, device=x.device)
    if bsums is None:
        bsums = torch.empty(k // 32, dtype=torch.int32, device=x.device)
    _need(q, k, "q")
    _need(d, 4 * (k // 256), "d")
    _need(bsums, 4 * (k // 32), "bsums")
    _check(lib.qbn_quantize_q8(_ptr(x, "x"), _DTYPES[x.dtype], k, _ptr(q, "q"), _ptr(d, "d"), _ptr(bsums, "bsums"),
                               _stream(x.device)), "qbn_quantize_q8")
    return q, d, bsums


def quantized_gemv_q8(w: QTensor, q: torch.Tensor, d: torch.Tensor, bsums: Optional[torch.Tensor] = None,
                      y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """GEMV against Q8_K activations from quantize_q8. Q4_K: y = W_hat @ (d * q),
    float32 [n] (bsums required). NVFP4: the integer-exact decode with the
    pinned binary32 epilogue, rounded to binary16; y float16 or float32 [n]
    (default float32)."""
    lib = _load()
    if y is None:
        y = torch.empty(w.n, dtype=torch.float32, device=w.device)
    _check_gemv_q8(w, q, d, bsums, y)
    ct = w._c()
    _check(lib.qbn_quantized_gemv_q8(ctypes.byref(ct), _ptr(q, "q"), _ptr(d, "d"), _ptr(bsums, "bsums"),
                                     _ptr(y, "y"), _DTYPES.get(y.dtype, -1), _stream(w.device)),
           "qbn_quantized_gemv_q8")
    return y


def _check_gemv_q8(w, q, d, bsums, y):
    _need(q, w.k, "q")
    _need(d, 4 * (w.k // 256), "d")
    if w.format == "q4_k":
        _need(bsums, 4 * (w.k // 32), "bsums")
    _need_dtype(y, (torch.float32, torch.float16), "y")
    _need(y, w.n * y.element_size(), "y")


MX_FORMATS = {"mxfp4": 1, "mxfp8": 7}


def quantize_mx(x: torch.Tensor, fmt: str = "mxfp4", codes: Optional[torch.Tensor] = None,
                scales: Optional[torch.Tensor] = None):
    """OCP MX quantization of x (float32 or bfloat16 [m][k], rows contiguous):
    returns (codes u8 [m][k/2] for mxfp4 or [m][k] for mxfp8, E8M0 scales u8 [m][k/32])."""
    lib = _load()
    if x.dtype not in _DTYPES:
        raise TypeError("x dtype %s" % x.dtype)
    if x.dim() == 1:
        x = x.unsqueeze(0)
    m, k = x.shape
    if codes is None:
        codes = torch.empty((m, k // 2 if fmt == "mxfp4" else k), dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty((m, k // 32), dtype=torch.uint8, device=x.device)
    _need(codes, m * (k // 2 if fmt == "mxfp4" else k), "codes")
    _need(scales, m * (k // 32), "scales")
    if not x.is_cuda or x.stride(1) != 1:
        raise ValueError("x must be a device tensor with contiguous rows")
    _check(lib.qbn_quantize_mx(ctypes.c_void_p(x.data_ptr()), _DTYPES[x.dtype], m, k, x.stride(0), MX_FORMATS[fmt],
                               _ptr(codes, "codes"), _ptr(scales, "scales"), _stream(x.device)), "qbn_quantize_mx")
    return codes, scales


def quantized_gemm_mx(w: QTensor, xcodes: torch.Tensor, xscales: torch.Tensor, fmt: str = "mxfp4",
                      y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = X_hat @ W_hat^T for MXFP4 activations (from quantize_mx) and an
    MXFP4 weight (W4A4), on the block-scaled matrix cores. Y bfloat16 (default)
    or float32 [m][n]. fmt "mxfp8" (W4A8) is refused by the library with
    QBN_ERR_UNSUPPORTED: the FP8 x FP4 matrix instruction drops product bits
    below a 13-bit window of each run of 8, so the tolerance would not hold."""
    lib = _load()
    m = xcodes.shape[0]
    if y is None:
        y = torch.empty((m, w.n), dtype=torch.bfloat16, device=w.device)
    _check_gemm_mx(w, m, xcodes, xscales, y, fmt)
    if not y.is_cuda or y.stride(1) != 1:
        raise ValueError("y must be a device tensor with contiguous rows")
    ct = w._c()
    _check(lib.qbn_quantized_gemm_mx(ctypes.byref(ct), m, MX_FORMATS[fmt], _ptr(xcodes, "xcodes"),
                                     _ptr(xscales, "xscales"), ctypes.c_void_p(y.data_ptr()), _DTYPES.get(y.dtype, -1),
                                     y.stride(0), _stream(w.device)), "qbn_quantized_gemm_mx")
    return y


def _check_gemm_mx(w, m, xcodes, xscales, y, fmt):
    _need(xcodes, m * (w.k // 2 if fmt == "mxfp4" else w.k), "xcodes")
    _need(xscales, m * (w.k // 32), "xscales")
    _check_rows(y, m, w.n, "y")


def _check_rows(t: torch.Tensor, rows: int, cols: int, name: str):
    """A [rows][>= cols] matrix with contiguous rows (leading dimension = stride 0)."""
    if rows == 0 or cols == 0:
        return
    if t.dim() != 2 or t.shape[0] < rows or t.shape[1] < cols:
        raise ValueError("%s must be at least [%d][%d], got %s" % (name, rows, cols, tuple(t.shape)))


def quantized_gemm(w: QTensor, x: torch.Tensor, y: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = X @ W_hat^T, X bfloat16 [m][k] -> Y bfloat16 [m][n] (MXFP4, GPTQ4,
    AWQ4, Q4_0; the int4 layouts also write a float32 y passed in)."""
    lib = _load()
    if x.dim() != 2:
        raise ValueError("x must be 2-D [m][k]")
    m = x.shape[0]
    if y is None:
        y = torch.empty((m, w.n), dtype=torch.bfloat16, device=w.device)
    _check_rows(x, m, w.k, "x")
    _check_rows(y, m, w.n, "y")
    if not (x.is_cuda and y.is_cuda):
        raise ValueError("x and y must be device (cuda) tensors")
    ct = w._c()
    ldx = x.stride(0) if x.shape[0] > 1 else x.shape[1]
    ldy = y.stride(0) if y.shape[0] > 1 else y.shape[1]
    if x.stride(1) != 1 or y.stride(1) != 1:
        raise ValueError("rows of x and y must be contiguous")
    _check(lib.qbn_quantized_gemm(ctypes.byref(ct), m, ctypes.c_void_p(x.data_ptr()), _DTYPES.get(x.dtype, -1), ldx,
                                  ctypes.c_void_p(y.data_ptr()), _DTYPES.get(y.dtype, -1), ldy, _stream(w.device)),
           "qbn_quantized_gemm")
    return y


def dequantize(w: QTensor, out: Optional[torch.Tensor] = None, dtype: torch.dtype = torch.float32,
               layout: str = "nk") -> torch.Tensor:
    """W_hat as float32 or bfloat16, layout "nk" ([n][k]) or "kn" ([k][n])."""
    lib = _load()
    lay = {"nk": 0, "kn": 1}[layout]
    if out is None:
        shape = (w.n, w.k) if lay == 0 else (w.k, w.n)
        out = torch.empty(shape, dtype=dtype, device=w.device)
    _need_dtype(out, (torch.float32, torch.bfloat16), "out")
    _need(out, w.n * w.k * out.element_size(), "out")
    ct = w._c()
    _check(lib.qbn_dequantize(ctypes.byref(ct), _ptr(out, "out"), _DTYPES.get(out.dtype, -1), lay,
                              _stream(w.device)), "qbn_dequantize")
    return out


def repack_target(src: QTensor, dst_format: str, dst_group: Optional[int] = None,
                  data: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None,
                  zeros: Optional[torch.Tensor] = None) -> QTensor:
    """The destination tensor of a repack of src into dst_format: the given
    buffers, the others allocated (GPTQ4 <-> AWQ4 share src's scales and zero
    points unless new ones are given)."""
    n, k, dev = src.n, src.k, src.device
    if dst_format in ("nvfp4", "nvfp4_cke"):
        if data is None:
            data = (torch.empty((n, k // 2), dtype=torch.uint8, device=dev) if dst_format == "nvfp4"
                    else torch.empty((n, k // 64, 36), dtype=torch.uint8, device=dev))
        if dst_format == "nvfp4" and scales is None:
            scales = torch.empty((n, k // 16), dtype=torch.uint8, device=dev)
        return QTensor(dst_format, n, k, data, scales if dst_format == "nvfp4" else None, scale2=src.scale2)
    if dst_format not in ("gptq4", "awq4", "q4_0"):
        raise ValueError("repack target must be gptq4, awq4, q4_0, nvfp4 or nvfp4_cke")
    if data is None:
        if dst_format == "gptq4":
            data = torch.empty((k // 8, n), dtype=torch.int32, device=dev)
        elif dst_format == "awq4":
            data = torch.empty((k, n // 8), dtype=torch.int32, device=dev)
        else:
            data = torch.empty((n, k // 32, 18), dtype=torch.uint8, device=dev)
    if dst_format == "q4_0":
        return QTensor("q4_0", n, k, data)
    g = dst_group if dst_group is not None else src.group
    if src.format == "q4_0":
        if scales is None:
            scales = torch.empty((k // g, n), dtype=torch.float16, device=dev)
        if zeros is None:
            zeros = torch.empty((k // g, n), dtype=torch.uint8, device=dev)
    else:
        scales = src.scales if scales is None else scales
        zeros = src.zeros if zeros is None else zeros
    return QTensor(dst_format, n, k, data, scales, zeros, group=g)


def repack(src: QTensor, dst_format: str, dst_group: Optional[int] = None, data: Optional[torch.Tensor] = None,
           scales: Optional[torch.Tensor] = None, zeros: Optional[torch.Tensor] = None) -> QTensor:
    """Repack int4 codes between GPTQ4, AWQ4 and Q4_0, or NVFP4 codes between
    the adjacent-pair and CKE split-half layouts (bit-exact). The Q4_0
    directions fail closed: if a weight cannot be held exactly by the target
    (a zero point other than 8; Q4_0 blocks of one target group with
    different d) nothing is written and RepackRefused is raised; this waits
    for the stream to read the device-side verdict."""
    lib = _load()
    dst = repack_target(src, dst_format, dst_group, data, scales, zeros)
    src.check_sizes()
    dst.check_sizes()
    status = torch.empty(REPACK_STATUS_WORDS, dtype=torch.int64, device=src.device)
    cs, cd = src._c(), dst._c()
    _check(lib.qbn_repack(ctypes.byref(cs), ctypes.byref(cd), _ptr(status, "status"), _stream(src.device)),
           "qbn_repack")
    if "q4_0" in (src.format, dst_format):
        bad = int(status[0].item())
        if bad >= 0:
            raise RepackRefused(bad, "a zero point other than 8" if dst_format == "q4_0"
                                else "Q4_0 blocks of one target group with different d")
    return dst


def validate(w: QTensor) -> int:
    """Fail-closed load-time scan (synchronous): -1 if the tensor is clean,
    else the index of its first invalid element."""
    lib = _load()
    first = ctypes.c_int64(-1)
    ct = w._c()
    st = lib.qbn_validate(ctypes.byref(ct), ctypes.byref(first), _stream(w.device))
    if st not in (0, 7):  # 7: QBN_ERR_NAN_SCALE, an invalid element was found
        raise QbnError(st, "qbn_validate")
    return int(first.value)


def validate_async(w: QTensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The same scan without waiting: out (int64 [1] on the device) receives
    the result when the stream reaches it."""
    lib = _load()
    if out is None:
        out = torch.empty(1, dtype=torch.int64, device=w.device)
    _need_dtype(out, (torch.int64,), "out")
    ct = w._c()
    _check(lib.qbn_validate_async(ctypes.byref(ct), _ptr(out, "first_bad"), _stream(w.device)), "qbn_validate_async")
    return out


class Prepared:
    """A library call with its arguments marshalled once, for tight loops and
    HIP-graph capture: calling it issues the C entry point on the current
    stream of the tensors' device and raises on a nonzero status."""

    def __init__(self, fn, args, where, device, keep):
        self._fn, self._args, self._where, self._device = fn, args, where, device
        self._keep = keep  # tensors and structs referenced by raw pointers

    def __call__(self):
        st = self._fn(*self._args, _stream(self._device))
        if st != 0:
            raise QbnError(st, self._where)


def prepare_gemv(w: QTensor, x: torch.Tensor, y: torch.Tensor) -> Prepared:
    lib = _load()
    _need_dtype(x, (torch.float32, torch.bfloat16), "x")
    _need_dtype(y, (torch.float32,), "y")
    _need(x, w.k * x.element_size(), "x")
    _need(y, w.n * 4, "y")
    ct = w._c()
    args = (ctypes.byref(ct), _ptr(x, "x"), _DTYPES[x.dtype], _ptr(y, "y"), _DTYPES.get(y.dtype, -1))
    return Prepared(lib.qbn_quantized_gemv, args, "qbn_quantized_gemv", w.device, (w, x, y, ct))


def prepare_quantize_q8(x: torch.Tensor, q: torch.Tensor, d: torch.Tensor, bsums: torch.Tensor) -> Prepared:
    lib = _load()
    k = x.numel()
    _need(q, k, "q")
    _need(d, 4 * (k // 256), "d")
    _need(bsums, 4 * (k // 32), "bsums")
    args = (_ptr(x, "x"), _DTYPES[x.dtype], x.numel(), _ptr(q, "q"), _ptr(d, "d"), _ptr(bsums, "bsums"))
    return Prepared(lib.qbn_quantize_q8, args, "qbn_quantize_q8", x.device, (x, q, d, bsums))


def prepare_gemv_q8(w: QTensor, q: torch.Tensor, d: torch.Tensor, bsums: Optional[torch.Tensor],
                    y: torch.Tensor) -> Prepared:
    lib = _load()
    _check_gemv_q8(w, q, d, bsums, y)
    ct = w._c()
    args = (ctypes.byref(ct), _ptr(q, "q"), _ptr(d, "d"), _ptr(bsums, "bsums"), _ptr(y, "y"),
            _DTYPES.get(y.dtype, -1))
    return Prepared(lib.qbn_quantized_gemv_q8, args, "qbn_quantized_gemv_q8", w.device, (w, q, d, bsums, y, ct))


def prepare_quantize_mx(x: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor, fmt: str = "mxfp4") -> Prepared:
    lib = _load()
    m, k = x.shape
    _need(codes, m * (k // 2 if fmt == "mxfp4" else k), "codes")
    _need(scales, m * (k // 32), "scales")
    args = (ctypes.c_void_p(x.data_ptr()), _DTYPES[x.dtype], m, k, x.stride(0), MX_FORMATS[fmt], _ptr(codes, "codes"),
            _ptr(scales, "scales"))
    return Prepared(lib.qbn_quantize_mx, args, "qbn_quantize_mx", x.device, (x, codes, scales))


def prepare_gemm_mx(w: QTensor, xcodes: torch.Tensor, xscales: torch.Tensor, y: torch.Tensor,
                    fmt: str = "mxfp4") -> Prepared:
    lib = _load()
    _check_gemm_mx(w, xcodes.shape[0], xcodes, xscales, y, fmt)
    ct = w._c()
    args = (ctypes.byref(ct), xcodes.shape[0], MX_FORMATS[fmt], _ptr(xcodes, "xcodes"), _ptr(xscales, "xscales"),
            ctypes.c_void_p(y.data_ptr()), _DTYPES.get(y.dtype, -1), y.stride(0))
    return Prepared(lib.qbn_quantized_gemm_mx, args, "qbn_quantized_gemm_mx", w.device, (w, xcodes, xscales, y, ct))


def prepare_quantize_nvfp4(x: torch.Tensor, scale2: float, tie: int, codes: torch.Tensor,
                           scales: torch.Tensor) -> Prepared:
    lib = _load()
    m, k = x.shape
    _need(codes, m * (k // 2), "codes")
    _need(scales, m * (k // 16), "scales")
    args = (ctypes.c_void_p(x.data_ptr()), _DTYPES.get(x.dtype, -1), m, k, x.stride(0) if m > 1 else k,
            ctypes.c_float(scale2), int(tie), _ptr(codes, "codes"), _ptr(scales, "scales"))
    return Prepared(lib.qbn_quantize_nvfp4, args, "qbn_quantize_nvfp4", x.device, (x, codes, scales))


def prepare_gemm(w: QTensor, x: torch.Tensor, y: torch.Tensor) -> Prepared:
    lib = _load()
    m = x.shape[0]
    _check_rows(x, m, w.k, "x")
    _check_rows(y, m, w.n, "y")
    if not (x.is_cuda and y.is_cuda) or x.stride(1) != 1 or y.stride(1) != 1:
        raise ValueError("x and y must be device tensors with contiguous rows")
    ct = w._c()
    args = (ctypes.byref(ct), m, ctypes.c_void_p(x.data_ptr()), _DTYPES.get(x.dtype, -1), x.stride(0),
            ctypes.c_void_p(y.data_ptr()), _DTYPES.get(y.dtype, -1), y.stride(0))
    return Prepared(lib.qbn_quantized_gemm, args, "qbn_quantized_gemm", w.device, (w, x, y, ct))


def prepare_dequantize(w: QTensor, out: torch.Tensor, layout: str = "nk") -> Prepared:
    lib = _load()
    _need_dtype(out, (torch.float32, torch.bfloat16), "out")
    _need(out, w.n * w.k * out.element_size(), "out")
    ct = w._c()
    args = (ctypes.byref(ct), _ptr(out, "out"), _DTYPES.get(out.dtype, -1), {"nk": 0, "kn": 1}[layout])
    return Prepared(lib.qbn_dequantize, args, "qbn_dequantize", w.device, (w, out, ct))


def prepare_repack(src: QTensor, dst: QTensor, status: torch.Tensor) -> Prepared:
    """Repack src into the buffers of dst (same n, k). status (int64
    [REPACK_STATUS_WORDS] on the device): status[0] receives -1, or the
    refusal index of a Q4_0 direction (then dst is left untouched)."""
    lib = _load()
    _need_dtype(status, (torch.int64,), "status")
    _need(status, 8 * REPACK_STATUS_WORDS, "status")
    src.check_sizes()
    dst.check_sizes()
    cs, cd = src._c(), dst._c()
    args = (ctypes.byref(cs), ctypes.byref(cd), _ptr(status, "status"))
    return Prepared(lib.qbn_repack, args, "qbn_repack", src.device, (src, dst, status, cs, cd))
