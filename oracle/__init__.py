"""CPU oracle for the FP4 block-scaled quantizer and GEMM.

TEST INFRASTRUCTURE ONLY.  This package is imported by ``tests/``, by the
``smoke()`` check and by the benchmark's ``cpu_baseline`` leg -- never by the
product library, which must fail loudly when its HIP build is missing rather
than fall back to anything here.  It shares no code with the GPU path.

The arithmetic lives in ``fp4_oracle.c`` (plain scalar C, binary32 without FMA
contraction, built by ``oracle/build.py``); this module only marshals numpy
arrays through ctypes and, for the GEMM reference, multiplies the dequantized
operands with a float64 library matmul (numpy), which is the one library
primitive the oracle uses.

Every function here is pinned by the CPU tests against closed forms,
exhaustive enumeration, a second formulation, brute force or rocRAND.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

AXIS_ROWS, AXIS_COLS = 0, 1
ROUND_RNE, ROUND_SR = 0, 1
NV_GLOBAL, NV_TILE128 = 0, 1


class OracleInputError(ValueError):
    """Input outside the quantizer contract (non-finite, degenerate NV domain)."""


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from oracle import build as _b

        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    u8p = ctypes.POINTER(ctypes.c_uint8)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    u32p = ctypes.POINTER(ctypes.c_uint32)
    f32p = ctypes.POINTER(ctypes.c_float)
    f64p = ctypes.POINTER(ctypes.c_double)
    i64, u64, u32, i32 = ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int

    def sig(name, res, *args):
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = list(args)

    sig("oc_e2m1_value", ctypes.c_double, ctypes.c_uint8)
    sig("oc_e2m1_rne", ctypes.c_uint8, ctypes.c_float)
    sig("oc_e2m1_sr", ctypes.c_uint8, ctypes.c_float, u32)
    sig("oc_e4m3_value", ctypes.c_double, ctypes.c_uint8)
    sig("oc_e4m3_rne_satfinite", ctypes.c_uint8, ctypes.c_float)
    sig("oc_philox4x32_10", None, u32p, u32p, u32p)
    sig("oc_r16", u32, u64, u32, u32, u32)
    sig("oc_mx_shared_exponent", i32, ctypes.c_float)
    sig("oc_hadamard32", None, f32p, u32)
    sig("oc_quantize_mx", i32, u16p, i64, i64, i64, i32, i32, u64, u32, u8p, u8p)
    sig("oc_hadamard32_quantize", i32, u16p, i64, i64, i64, i32, u32, i32, u64, u32, u8p, u8p)
    sig("oc_nv_tensor_scale", ctypes.c_float, ctypes.c_float)
    sig("oc_nv_block_scale", ctypes.c_uint8, ctypes.c_float, ctypes.c_float)
    sig("oc_quantize_nv", i32, u16p, i64, i64, i64, i32, i32, u64, u32, i32, u8p, u8p, f32p)
    sig("oc_hadamard32_quantize_nv", i32, u16p, i64, i64, i64, i32, u32, i32, u64, u32, i32, u8p, u8p, f32p)
    sig("oc_dequant_mx", None, u8p, u8p, i64, i64, f64p)
    sig("oc_dequant_nv", None, u8p, u8p, f32p, i32, i64, i64, f64p)
    sig("oc_gemm_bruteforce", None, f64p, f64p, i64, i64, i64, ctypes.c_double, f64p, f64p)
    sig("oc_float_to_bf16", ctypes.c_uint16, ctypes.c_float)
    sig("oc_double_to_bf16", ctypes.c_uint16, ctypes.c_double)
    sig("oc_double_to_bf16_array", None, f64p, i64, u16p)
    sig("oc_swiglu_f64", ctypes.c_double, ctypes.c_float, ctypes.c_float)
    sig("oc_swiglu_bf16", i32, u16p, i64, i64, i64, i64, u16p, f64p)
    _lib = lib
    return lib


def _ptr(a, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _as_bf16_bits(x):
    """Accept a 2-D uint16 array of bf16 bit patterns (C-contiguous rows)."""
    x = np.asarray(x)
    if x.dtype != np.uint16 or x.ndim != 2:
        raise TypeError("expected a 2-D uint16 array of bf16 bit patterns")
    return np.ascontiguousarray(x)


# ---------------------------------------------------------------- scalars


def e2m1_value(code: int) -> float:
    return _load().oc_e2m1_value(code)


def e2m1_rne(y: float) -> int:
    return _load().oc_e2m1_rne(y)


def e2m1_sr(y: float, r16: int) -> int:
    return _load().oc_e2m1_sr(y, r16)


def e4m3_value(code: int) -> float:
    return _load().oc_e4m3_value(code)


def e4m3_rne_satfinite(z: float) -> int:
    return _load().oc_e4m3_rne_satfinite(z)


def philox4x32_10(ctr, key):
    c = np.asarray(ctr, dtype=np.uint32)
    k = np.asarray(key, dtype=np.uint32)
    out = np.zeros(4, dtype=np.uint32)
    _load().oc_philox4x32_10(_ptr(c, ctypes.c_uint32), _ptr(k, ctypes.c_uint32), _ptr(out, ctypes.c_uint32))
    return [int(v) for v in out]


def r16(seed: int, stream: int, row: int, col: int) -> int:
    return _load().oc_r16(seed, stream, row, col)


def mx_shared_exponent(amax: float) -> int:
    return _load().oc_mx_shared_exponent(amax)


def hadamard32(v, sign_mask: int) -> np.ndarray:
    a = np.array(v, dtype=np.float32).copy()
    assert a.shape == (32,)
    _load().oc_hadamard32(_ptr(a, ctypes.c_float), sign_mask)
    return a


def nv_tensor_scale(amax: float) -> float:
    return _load().oc_nv_tensor_scale(amax)


def nv_block_scale(b: float, S: float) -> int:
    return _load().oc_nv_block_scale(b, S)


# ---------------------------------------------------------------- operands


def _logical_shape(x, cols, axis):
    rows = x.shape[0]
    return (rows, cols) if axis == AXIS_ROWS else (cols, rows)


def quantize_mx(x, cols=None, axis=AXIS_ROWS, sr=False, seed=0, stream=0):
    """MXFP4-quantize bf16 bits ``x`` [rows x ld] (first ``cols`` columns).

    Returns ``(codes [R, K/2] uint8, scales [R, K/32] uint8)`` in the linear
    layout of the logical operand (R, K) = (rows, cols) for AXIS_ROWS and
    (cols, rows) for AXIS_COLS.
    """
    x = _as_bf16_bits(x)
    rows, ld = x.shape
    cols = ld if cols is None else cols
    R, K = _logical_shape(x, cols, axis)
    codes = np.zeros((R, K // 2), dtype=np.uint8)
    scales = np.zeros((R, K // 32), dtype=np.uint8)
    st = _load().oc_quantize_mx(_ptr(x, ctypes.c_uint16), rows, cols, ld, axis, int(bool(sr)), seed, stream,
                                _ptr(codes, ctypes.c_uint8), _ptr(scales, ctypes.c_uint8))
    if st != 0:
        raise OracleInputError(f"oc_quantize_mx status {st}")
    return codes, scales


def hadamard32_quantize(x, sign_mask, cols=None, axis=AXIS_COLS, sr=False, seed=0, stream=0):
    """Fixed-sign Hadamard-32 along K, then MXFP4 (same outputs as quantize_mx)."""
    x = _as_bf16_bits(x)
    rows, ld = x.shape
    cols = ld if cols is None else cols
    R, K = _logical_shape(x, cols, axis)
    codes = np.zeros((R, K // 2), dtype=np.uint8)
    scales = np.zeros((R, K // 32), dtype=np.uint8)
    st = _load().oc_hadamard32_quantize(_ptr(x, ctypes.c_uint16), rows, cols, ld, axis, sign_mask,
                                        int(bool(sr)), seed, stream,
                                        _ptr(codes, ctypes.c_uint8), _ptr(scales, ctypes.c_uint8))
    if st != 0:
        raise OracleInputError(f"oc_hadamard32_quantize status {st}")
    return codes, scales


def nv_tensor_scale_shape(R, K, domain):
    return (1,) if domain == NV_GLOBAL else ((R + 127) // 128, (K + 127) // 128)


def quantize_nv(x, cols=None, axis=AXIS_ROWS, sr=False, seed=0, stream=0, domain=NV_GLOBAL):
    """NVFP4-quantize; returns ``(codes [R, K/2], scales [R, K/16] E4M3 bytes,
    tensor_scale float32 [1] or [ceil(R/128), ceil(K/128)])``."""
    x = _as_bf16_bits(x)
    rows, ld = x.shape
    cols = ld if cols is None else cols
    R, K = _logical_shape(x, cols, axis)
    codes = np.zeros((R, K // 2), dtype=np.uint8)
    scales = np.zeros((R, K // 16), dtype=np.uint8)
    ts = np.zeros(nv_tensor_scale_shape(R, K, domain), dtype=np.float32)
    st = _load().oc_quantize_nv(_ptr(x, ctypes.c_uint16), rows, cols, ld, axis, int(bool(sr)), seed, stream,
                                domain, _ptr(codes, ctypes.c_uint8), _ptr(scales, ctypes.c_uint8),
                                _ptr(ts, ctypes.c_float))
    if st != 0:
        raise OracleInputError(f"oc_quantize_nv status {st}")
    return codes, scales, ts


def hadamard32_quantize_nv(x, sign_mask, cols=None, axis=AXIS_COLS, sr=False, seed=0, stream=0, domain=NV_GLOBAL):
    """Fixed-sign Hadamard-32 along K, then NVFP4 (K % 32 == 0); outputs as
    quantize_nv."""
    x = _as_bf16_bits(x)
    rows, ld = x.shape
    cols = ld if cols is None else cols
    R, K = _logical_shape(x, cols, axis)
    codes = np.zeros((R, K // 2), dtype=np.uint8)
    scales = np.zeros((R, K // 16), dtype=np.uint8)
    ts = np.zeros(nv_tensor_scale_shape(R, K, domain), dtype=np.float32)
    st = _load().oc_hadamard32_quantize_nv(_ptr(x, ctypes.c_uint16), rows, cols, ld, axis, sign_mask & 0xFFFFFFFF,
                                           int(bool(sr)), seed, stream, domain, _ptr(codes, ctypes.c_uint8),
                                           _ptr(scales, ctypes.c_uint8), _ptr(ts, ctypes.c_float))
    if st != 0:
        raise OracleInputError(f"oc_hadamard32_quantize_nv status {st}")
    return codes, scales, ts


def tile_mx(codes, scales):
    """The tiled consumer layout of an MX operand, as a pure index map of the
    linear one (definition in the library header): with Rp = 32 * ceil(R/32),
    codes become [Rp/32][K/64][64 lanes][16 bytes] where lane l of block
    (g, kb) holds row 32 g + l mod 32, K elements 64 kb + 32 (l / 32) .. +31;
    scales become [K/128][Rp][4] (byte q of (s, r) = scale of row r, block
    4 s + q).  Padding rows are zero.  Returns (codes [Rp, K/2], scales
    [K/128, Rp, 4]) as uint8 arrays."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    R, K2 = codes.shape
    K = 2 * K2
    assert K % 128 == 0 and scales.shape == (R, K // 32)
    Rp = (R + 31) // 32 * 32
    c = np.zeros((Rp, K2), dtype=np.uint8)
    c[:R] = codes
    # [g, row in group, kb, half, 16 bytes] -> [g, kb, half, row in group, 16 bytes]
    tiled = c.reshape(Rp // 32, 32, K // 64, 2, 16).transpose(0, 2, 3, 1, 4).reshape(Rp, K2)
    s = np.zeros((Rp, K // 32), dtype=np.uint8)
    s[:R] = scales
    ts = s.reshape(Rp, K // 128, 4).transpose(1, 0, 2)
    return np.ascontiguousarray(tiled), np.ascontiguousarray(ts)


def tile_nv(codes, scales):
    """The tiled consumer layout of an NV operand (K % 128 == 0), as a pure
    index map of the linear one (definition in the library header): with
    Rp = 32 * ceil(R/32) and S = K/128 steps, codes become [Rp/32][S][32][64]
    (the 64 code bytes of row 32 g + f for K elements 128 s .. 128 s + 127 at
    (g, s, f)) and scales [Rp/32][S][32][8] (the eight E4M3 bytes of the same
    row and step).  Padding rows are zero.  Returns (codes [Rp, K/2], scales
    [Rp, K/16]) as uint8 arrays holding those bytes in order."""
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    R, K2 = codes.shape
    K = 2 * K2
    assert K % 128 == 0 and scales.shape == (R, K // 16)
    Rp = (R + 31) // 32 * 32
    c = np.zeros((Rp, K2), dtype=np.uint8)
    c[:R] = codes
    s = np.zeros((Rp, K // 16), dtype=np.uint8)
    s[:R] = scales
    # [g, f, step, bytes] -> [g, step, f, bytes]
    tc = c.reshape(Rp // 32, 32, K // 128, 64).transpose(0, 2, 1, 3).reshape(Rp, K2)
    tsc = s.reshape(Rp // 32, 32, K // 128, 8).transpose(0, 2, 1, 3).reshape(Rp, K // 16)
    return np.ascontiguousarray(tc), np.ascontiguousarray(tsc)


def dequant_mx(codes, scales):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    R, K = codes.shape[0], codes.shape[1] * 2
    assert scales.shape == (R, K // 32)
    out = np.zeros((R, K), dtype=np.float64)
    _load().oc_dequant_mx(_ptr(codes, ctypes.c_uint8), _ptr(scales, ctypes.c_uint8), R, K,
                          _ptr(out, ctypes.c_double))
    return out


def dequant_nv(codes, scales, tensor_scale, domain):
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    ts = np.ascontiguousarray(tensor_scale, dtype=np.float32)
    R, K = codes.shape[0], codes.shape[1] * 2
    assert scales.shape == (R, K // 16)
    assert ts.shape == nv_tensor_scale_shape(R, K, domain)
    out = np.zeros((R, K), dtype=np.float64)
    _load().oc_dequant_nv(_ptr(codes, ctypes.c_uint8), _ptr(scales, ctypes.c_uint8), _ptr(ts, ctypes.c_float),
                          domain, R, K, _ptr(out, ctypes.c_double))
    return out


def gemm_bruteforce(a_dq, b_dq, alpha=1.0):
    """C = alpha * A @ B^T and W = |alpha| * |A| @ |B|^T by a plain fp64 triple loop."""
    A = np.ascontiguousarray(a_dq, dtype=np.float64)
    B = np.ascontiguousarray(b_dq, dtype=np.float64)
    M, K = A.shape
    N = B.shape[0]
    assert B.shape[1] == K
    C = np.zeros((M, N), dtype=np.float64)
    W = np.zeros((M, N), dtype=np.float64)
    _load().oc_gemm_bruteforce(_ptr(A, ctypes.c_double), _ptr(B, ctypes.c_double), M, N, K, alpha,
                               _ptr(C, ctypes.c_double), _ptr(W, ctypes.c_double))
    return C, W


def gemm_ref(a_dq, b_dq, alpha=1.0, weights=True):
    """C = alpha * A @ B^T and the tolerance weight W = |alpha| * |A| @ |B|^T
    (None with weights=False), with a float64 library matmul (numpy) as the
    contraction step."""
    A = np.asarray(a_dq, dtype=np.float64)
    B = np.asarray(b_dq, dtype=np.float64)
    C = alpha * (A @ B.T)
    W = abs(alpha) * (np.abs(A) @ np.abs(B).T) if weights else None
    return C, W


def float_to_bf16(f: float) -> int:
    """binary32 -> bf16 bits, round to nearest even."""
    return int(_load().oc_float_to_bf16(float(f)))


def double_to_bf16(v: float) -> int:
    """binary64 -> bf16 bits, rounded once to nearest even (no binary32 step)."""
    return int(_load().oc_double_to_bf16(float(v)))


def double_to_bf16_array(v):
    """bf16 bits (uint16, same shape) of a float64 array, each element
    rounded once to nearest even."""
    a = np.ascontiguousarray(v, dtype=np.float64)
    out = np.zeros(a.shape, dtype=np.uint16)
    if a.size:
        _load().oc_double_to_bf16_array(_ptr(a, ctypes.c_double), a.size, _ptr(out, ctypes.c_uint16))
    return out


def swiglu_f64(g: float, u: float) -> float:
    """SiLU(g) * u = g u / (1 + e^-g) in binary64 (for g, u binary32 values):
    the value the oracle's bf16 H is rounded from."""
    return float(_load().oc_swiglu_f64(float(g), float(u)))


def swiglu_bf16(c, F, pair=32, with_f64=False):
    """H = bf16(SiLU(gate) * up), the real value rounded once, from a bf16
    GEMM output C [M x >= 2F] whose columns interleave gate and up in groups
    of `pair` (pair = 32: the layout of the fused GEMM's weight; pair = F:
    [gate | up]).  c: a 2-D uint16 array of bf16 bit patterns.  Returns
    uint16 bits [M x F]; with ``with_f64`` also the float64 values H was
    rounded from (to bound a kernel's deviation).  H is the binary64 value of
    SiLU(g) u rounded once to nearest even."""
    cb = _as_bf16_bits(c)
    M, ldc = cb.shape
    if ldc < 2 * F:
        raise ValueError("C needs at least 2F columns")
    h = np.zeros((M, F), dtype=np.uint16)
    hv = np.zeros((M, F), dtype=np.float64) if with_f64 else None
    if M and F:
        rc = _load().oc_swiglu_bf16(_ptr(cb, ctypes.c_uint16), M, F, ldc, pair, _ptr(h, ctypes.c_uint16),
                                    _ptr(hv, ctypes.c_double) if with_f64 else None)
        if rc != 0:
            raise ValueError("pair must divide F")
    return (h, hv) if with_f64 else h
