"""ctypes binding of ``libfp4q.so`` with the C ABI's entry-point names.

Argument marshalling only: every step of the quantizers and GEMMs runs in the
library's HIP kernels.  PyTorch supplies device memory (``data_ptr()``) and the
stream (``torch.cuda.current_stream()``).  If the library has not been built
this module raises -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp4q.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "fp4q.h")

# enums of include/fp4q.h
OK, EINVAL, ESHAPE, EALIGN, ELAUNCH, EUNSUPPORTED = 0, 1, 2, 3, 4, 5
ALONG_ROWS, ALONG_COLS = 0, 1
RNE, SR = 0, 1
NV_GLOBAL, NV_TILE128 = 0, 1
LAYOUT_LINEAR, LAYOUT_TILED = 0, 1
OUT_F32, OUT_BF16 = 0, 1

_lib = None


class Fp4qError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed with status {status}: {status_str(status)}")
        self.status = status


def declared_functions():
    """Names of the functions include/fp4q.h declares."""
    with open(HEADER) as f:
        text = f.read()
    return re.findall(r"^FP4Q_API\s+[\w\s\*]*?\b(\w+)\s*\(", text, flags=re.MULTILINE)


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise FileNotFoundError(
            f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
            "(hipcc, gfx950); libfp4q has no CPU fallback")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, u64, u32, i32, f32 = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32,
                                   ctypes.c_int, ctypes.c_float)
    L.fp4_quantize_mx.argtypes = [vp, i64, i64, i64, i32, i32, u64, u32, vp, vp, i32, vp]
    L.fp4_hadamard32_quantize.argtypes = [vp, i64, i64, i64, i32, u32, i32, u64, u32, vp, vp, i32, vp]
    L.fp4_quantize_mx_dual.argtypes = [vp, i64, i64, i64, i32, u32, vp, vp, i32, u32, i32, u32, vp, vp, u64, i32,
                                       vp]
    L.fp4q_nv_workspace_bytes.argtypes = [i64, i64, i32, i32]
    L.fp4q_nv_workspace_bytes.restype = ctypes.c_size_t
    L.fp4_quantize_nv.argtypes = [vp, i64, i64, i64, i32, i32, u64, u32, i32, vp, vp, vp, vp, ctypes.c_size_t,
                                  i32, vp]
    L.fp4_gemm_mx.argtypes = [vp, vp, vp, vp, i64, i64, i64, f32, i32, vp, i32, i64, vp]
    L.fp4_gemm_nv.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i64, i64, f32, i32, vp, i32, i64, vp]
    L.fp4_gemm_mx_amax.argtypes = [vp, vp, vp, vp, i64, i64, i64, f32, i32, vp, i32, i64, vp, vp]
    L.fp4_gemm_mx_quant.argtypes = [vp, vp, vp, vp, i64, i64, i64, f32, i32, vp, vp, i32, vp]
    L.fp4_gemm_mx_swiglu_quant.argtypes = [vp, vp, vp, vp, i64, i64, i64, f32, i32, vp, vp, i32, vp]
    L.fp4_swiglu_bf16.argtypes = [vp, i64, i64, i64, i64, vp, i64, vp]
    L.fp4_gemm_nv_amax.argtypes = [vp, vp, vp, vp, vp, vp, i32, i64, i64, i64, f32, i32, vp, i32, i64, vp, vp]
    L.fp4_quantize_nv_amax.argtypes = [vp, i64, i64, i64, i32, u64, u32, vp, vp, vp, vp, vp]
    L.fp4_quantize_nv_noalloc.argtypes = [vp, i64, i64, i64, i32, i32, u64, u32, i32, vp, vp, vp, i32, vp]
    L.fp4_hadamard32_quantize_nv.argtypes = [vp, i64, i64, i64, i32, u32, i32, u64, u32, i32, vp, vp, vp, vp,
                                             ctypes.c_size_t, i32, vp]
    for fn in ("fp4_quantize_mx", "fp4_hadamard32_quantize", "fp4_quantize_mx_dual", "fp4_quantize_nv",
               "fp4_quantize_nv_noalloc",
               "fp4_quantize_nv_amax", "fp4_hadamard32_quantize_nv", "fp4_gemm_mx", "fp4_gemm_nv",
               "fp4_gemm_mx_amax", "fp4_gemm_nv_amax", "fp4_gemm_mx_quant"):
        getattr(L, fn).restype = i32
    L.fp4q_status_str.argtypes = [i32]
    L.fp4q_status_str.restype = ctypes.c_char_p
    L.fp4q_abi_version.argtypes = []
    L.fp4q_abi_version.restype = i32
    _lib = L
    return L


def status_str(status: int) -> str:
    return lib().fp4q_status_str(status).decode()


def abi_version() -> int:
    return lib().fp4q_abi_version()


def _check(fn: str, status: int):
    if status != OK:
        raise Fp4qError(fn, status)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check_out(t: torch.Tensor, name: str, dtype, shape, device) -> torch.Tensor:
    """A caller-supplied output: the library cannot see buffer sizes, so a
    wrong one would be written past its end.  It must be a contiguous tensor
    of `dtype` on the input's device with exactly `shape`."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if t.device != torch.device(device):
        raise ValueError(f"{name} is on {t.device}, the input on {device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, not {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _amax_ptr(t: torch.Tensor, device) -> int:
    if t.dtype != torch.float32 or t.numel() < 1 or t.device != torch.device(device):
        raise ValueError("c_amax must be a float32 tensor with at least one element on the operands' device")
    return t.data_ptr()


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _input(x: torch.Tensor, cols: Optional[int]):
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D bf16 tensor with unit column stride")
    rows = x.shape[0]
    cols = x.shape[1] if cols is None else cols
    ld = x.stride(0) if rows > 1 else x.shape[1]
    return rows, cols, ld


def _logical(rows: int, cols: int, axis: int):
    return (rows, cols) if axis == ALONG_ROWS else (cols, rows)


def mx_output_shapes(R: int, K: int, layout: int):
    """(codes shape, scales shape) of an MX operand [R x K] in `layout`."""
    if layout == LAYOUT_TILED:
        Rp = (R + 31) // 32 * 32
        return (Rp, K // 2), (K // 128, Rp, 4)
    return (R, K // 2), (R, K // 32)


def _mx_outputs(R, K, layout, codes, scales, device):
    cshape, sshape = mx_output_shapes(R, K, layout)
    if codes is None:
        codes = torch.empty(cshape, dtype=torch.uint8, device=device)
    if scales is None:
        scales = torch.empty(sshape, dtype=torch.uint8, device=device)
    return (_check_out(codes, "codes", torch.uint8, cshape, device),
            _check_out(scales, "scales", torch.uint8, sshape, device))


def fp4_quantize_mx(x: torch.Tensor, *, cols: Optional[int] = None, axis: int = ALONG_ROWS, round: int = RNE,
                    seed: int = 0, stream_id: int = 0, layout: int = LAYOUT_LINEAR,
                    codes: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None,
                    stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    rows, cols, ld = _input(x, cols)
    R, K = _logical(rows, cols, axis)
    codes, scales = _mx_outputs(R, K, layout, codes, scales, x.device)
    _check("fp4_quantize_mx", lib().fp4_quantize_mx(x.data_ptr(), rows, cols, ld, axis, round, seed, stream_id,
                                                    codes.data_ptr(), scales.data_ptr(), layout, _stream(stream)))
    return codes, scales


def fp4_quantize_mx_dual(x: torch.Tensor, *, round_rows: int = RNE, stream_id_rows: int = 0,
                         hadamard_cols: bool = True, sign_mask: int = 0, round_cols: int = RNE,
                         stream_id_cols: int = 0, seed: int = 0, layout: int = LAYOUT_LINEAR,
                         codes_rows: Optional[torch.Tensor] = None, scales_rows: Optional[torch.Tensor] = None,
                         codes_cols: Optional[torch.Tensor] = None, scales_cols: Optional[torch.Tensor] = None,
                         stream=None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor, torch.Tensor]:
    """x along rows and x^T along columns (optionally Hadamard) from one read
    of x: (codes_rows, scales_rows, codes_cols, scales_cols)."""
    rows, cols, ld = _input(x, None)
    codes_rows, scales_rows = _mx_outputs(rows, cols, layout, codes_rows, scales_rows, x.device)
    codes_cols, scales_cols = _mx_outputs(cols, rows, layout, codes_cols, scales_cols, x.device)
    _check("fp4_quantize_mx_dual",
           lib().fp4_quantize_mx_dual(x.data_ptr(), rows, cols, ld, round_rows, stream_id_rows, codes_rows.data_ptr(),
                                      scales_rows.data_ptr(), int(bool(hadamard_cols)), sign_mask & 0xFFFFFFFF,
                                      round_cols, stream_id_cols, codes_cols.data_ptr(), scales_cols.data_ptr(),
                                      seed, layout, _stream(stream)))
    return codes_rows, scales_rows, codes_cols, scales_cols


def fp4_hadamard32_quantize(x: torch.Tensor, sign_mask: int, *, cols: Optional[int] = None, axis: int = ALONG_COLS,
                            round: int = RNE, seed: int = 0, stream_id: int = 0, layout: int = LAYOUT_LINEAR,
                            codes: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None,
                            stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    rows, cols, ld = _input(x, cols)
    R, K = _logical(rows, cols, axis)
    codes, scales = _mx_outputs(R, K, layout, codes, scales, x.device)
    _check("fp4_hadamard32_quantize",
           lib().fp4_hadamard32_quantize(x.data_ptr(), rows, cols, ld, axis, sign_mask & 0xFFFFFFFF, round, seed,
                                         stream_id, codes.data_ptr(), scales.data_ptr(), layout, _stream(stream)))
    return codes, scales


def fp4q_nv_workspace_bytes(rows: int, cols: int, axis: int, domain: int) -> int:
    return lib().fp4q_nv_workspace_bytes(rows, cols, axis, domain)


def nv_tensor_scale_shape(R: int, K: int, domain: int):
    return (1,) if domain == NV_GLOBAL else ((R + 127) // 128, (K + 127) // 128)


def nv_output_shapes(R: int, K: int, layout: int = LAYOUT_LINEAR):
    """(codes shape, scales shape) of an NV operand [R x K] in `layout`: the
    tiled layout stores Rp = 32 ceil(R/32) rows (same bytes per row)."""
    Rs = (R + 31) // 32 * 32 if layout == LAYOUT_TILED else R
    return (Rs, K // 2), (Rs, K // 16)


def fp4_quantize_nv(x: torch.Tensor, domain: int = NV_GLOBAL, *, cols: Optional[int] = None, axis: int = ALONG_ROWS,
                    round: int = RNE, seed: int = 0, stream_id: int = 0, codes: Optional[torch.Tensor] = None,
                    scales: Optional[torch.Tensor] = None, tensor_scale: Optional[torch.Tensor] = None,
                    workspace: Optional[torch.Tensor] = None, amax: Optional[torch.Tensor] = None,
                    hadamard_mask: Optional[int] = None, layout: int = LAYOUT_LINEAR, stream=None):
    """NVFP4; with `amax` (a device float32 tensor holding max |x|, global
    domain only) the producer runs in one pass (fp4_quantize_nv_amax); with
    `hadamard_mask` the fixed-sign Hadamard-32 runs first
    (fp4_hadamard32_quantize_nv, along columns)."""
    rows, cols, ld = _input(x, cols)
    R, K = _logical(rows, cols, axis)
    cshape, sshape = nv_output_shapes(R, K, layout)
    if codes is None:
        codes = torch.empty(cshape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(sshape, dtype=torch.uint8, device=x.device)
    if tensor_scale is None:
        tensor_scale = torch.empty(nv_tensor_scale_shape(R, K, domain), dtype=torch.float32, device=x.device)
    _check_out(codes, "codes", torch.uint8, cshape, x.device)
    _check_out(scales, "scales", torch.uint8, sshape, x.device)
    _check_out(tensor_scale, "tensor_scale", torch.float32, nv_tensor_scale_shape(R, K, domain), x.device)
    if amax is not None:
        if (domain != NV_GLOBAL or axis != ALONG_ROWS or amax.dtype != torch.float32 or amax.device != x.device
                or layout != LAYOUT_LINEAR):
            raise ValueError("a given amax is a float32 tensor on x's device, for the global domain along rows, "
                             "linear layout")
        _check("fp4_quantize_nv_amax",
               lib().fp4_quantize_nv_amax(x.data_ptr(), rows, cols, ld, round, seed, stream_id, amax.data_ptr(),
                                          codes.data_ptr(), scales.data_ptr(), tensor_scale.data_ptr(),
                                          _stream(stream)))
        return codes, scales, tensor_scale
    need = fp4q_nv_workspace_bytes(rows, cols, axis, domain)
    if workspace is None and need > 0:
        workspace = torch.empty((need,), dtype=torch.uint8, device=x.device)
    if workspace is not None and (workspace.device != x.device or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor on x's device")
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if hadamard_mask is not None:
        _check("fp4_hadamard32_quantize_nv",
               lib().fp4_hadamard32_quantize_nv(x.data_ptr(), rows, cols, ld, axis, hadamard_mask & 0xFFFFFFFF, round,
                                                seed, stream_id, domain, codes.data_ptr(), scales.data_ptr(),
                                                tensor_scale.data_ptr(), _ptr(workspace), wbytes, layout,
                                                _stream(stream)))
        return codes, scales, tensor_scale
    _check("fp4_quantize_nv",
           lib().fp4_quantize_nv(x.data_ptr(), rows, cols, ld, axis, round, seed, stream_id, domain,
                                 codes.data_ptr(), scales.data_ptr(), tensor_scale.data_ptr(), _ptr(workspace),
                                 wbytes, layout, _stream(stream)))
    return codes, scales, tensor_scale


def fp4_quantize_nv_noalloc(x: torch.Tensor, domain: int = NV_GLOBAL, *, cols: Optional[int] = None,
                            axis: int = ALONG_ROWS, round: int = RNE, seed: int = 0, stream_id: int = 0,
                            codes: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None,
                            tensor_scale: Optional[torch.Tensor] = None, layout: int = LAYOUT_LINEAR, stream=None):
    """fp4_quantize_nv with the library's own workspace: the call allocates
    no device memory (pass every output to allocate none here either)."""
    rows, cols, ld = _input(x, cols)
    R, K = _logical(rows, cols, axis)
    cshape, sshape = nv_output_shapes(R, K, layout)
    if codes is None:
        codes = torch.empty(cshape, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(sshape, dtype=torch.uint8, device=x.device)
    if tensor_scale is None:
        tensor_scale = torch.empty(nv_tensor_scale_shape(R, K, domain), dtype=torch.float32, device=x.device)
    _check_out(codes, "codes", torch.uint8, cshape, x.device)
    _check_out(scales, "scales", torch.uint8, sshape, x.device)
    _check_out(tensor_scale, "tensor_scale", torch.float32, nv_tensor_scale_shape(R, K, domain), x.device)
    _check("fp4_quantize_nv_noalloc",
           lib().fp4_quantize_nv_noalloc(x.data_ptr(), rows, cols, ld, axis, round, seed, stream_id, domain,
                                         codes.data_ptr(), scales.data_ptr(), tensor_scale.data_ptr(), layout,
                                         _stream(stream)))
    return codes, scales, tensor_scale


def _gemm_out(M: int, N: int, out_dtype, device, c: Optional[torch.Tensor]):
    if c is None:
        c = torch.empty((M, N), dtype=out_dtype, device=device)
    if c.dtype not in (torch.float32, torch.bfloat16) or c.dim() != 2 or c.stride(1) != 1:
        raise ValueError("c must be a 2-D fp32 or bf16 tensor with unit column stride")
    if tuple(c.shape) != (M, N) or c.device != torch.device(device):
        raise ValueError(f"c must be a [{M} x {N}] tensor on {device}, not {tuple(c.shape)} on {c.device}")
    if M > 1 and c.stride(0) < N:
        raise ValueError("c's rows overlap (row stride below N)")
    ldc = c.stride(0) if M > 1 else N
    return c, (OUT_F32 if c.dtype == torch.float32 else OUT_BF16), ldc


def fp4_gemm_mx(a_codes: torch.Tensor, a_scales: torch.Tensor, b_codes: torch.Tensor, b_scales: torch.Tensor, *,
                alpha: float = 1.0, out_dtype=torch.float32, c: Optional[torch.Tensor] = None,
                layout: int = LAYOUT_LINEAR, m: Optional[int] = None, n: Optional[int] = None,
                c_amax: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """C = alpha * A B^T.  In the tiled layout the code tensors carry rows
    padded to a multiple of 32, so pass the logical m and n.  With `c_amax`
    (a device float32 tensor) max |C| is folded into it (fp4_gemm_mx_amax)."""
    M = a_codes.shape[0] if m is None else m
    N = b_codes.shape[0] if n is None else n
    K = a_codes.shape[1] * 2
    if b_codes.shape[1] * 2 != K:
        raise ValueError("A and B must have the same K")
    c, ctype, ldc = _gemm_out(M, N, out_dtype, a_codes.device, c)
    if c_amax is not None:
        _check("fp4_gemm_mx_amax",
               lib().fp4_gemm_mx_amax(a_codes.data_ptr(), a_scales.data_ptr(), b_codes.data_ptr(), b_scales.data_ptr(),
                                      M, N, K, float(alpha), layout, c.data_ptr(), ctype, ldc, _amax_ptr(c_amax, a_codes.device),
                                      _stream(stream)))
        return c
    _check("fp4_gemm_mx", lib().fp4_gemm_mx(a_codes.data_ptr(), a_scales.data_ptr(), b_codes.data_ptr(),
                                            b_scales.data_ptr(), M, N, K, float(alpha), layout,
                                            c.data_ptr(), ctype, ldc, _stream(stream)))
    return c


def fp4_gemm_mx_quant(a_codes: torch.Tensor, a_scales: torch.Tensor, b_codes: torch.Tensor, b_scales: torch.Tensor,
                      *, alpha: float = 1.0, layout: int = LAYOUT_LINEAR, m: Optional[int] = None,
                      n: Optional[int] = None, c_layout: int = LAYOUT_LINEAR, codes: Optional[torch.Tensor] = None,
                      scales: Optional[torch.Tensor] = None, stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """C = alpha * A B^T written as an MXFP4 operand along rows (RNE of the
    bf16 C) in c_layout: returns (codes, scales)."""
    M = a_codes.shape[0] if m is None else m
    N = b_codes.shape[0] if n is None else n
    K = a_codes.shape[1] * 2
    if b_codes.shape[1] * 2 != K:
        raise ValueError("A and B must have the same K")
    codes, scales = _mx_outputs(M, N, c_layout, codes, scales, a_codes.device)
    _check("fp4_gemm_mx_quant",
           lib().fp4_gemm_mx_quant(a_codes.data_ptr(), a_scales.data_ptr(), b_codes.data_ptr(), b_scales.data_ptr(),
                                   M, N, K, float(alpha), layout, codes.data_ptr(), scales.data_ptr(), c_layout,
                                   _stream(stream)))
    return codes, scales


def fp4_gemm_mx_swiglu_quant(a_codes: torch.Tensor, a_scales: torch.Tensor, b_codes: torch.Tensor,
                             b_scales: torch.Tensor, *, alpha: float = 1.0, layout: int = LAYOUT_LINEAR,
                             m: Optional[int] = None, n: Optional[int] = None, h_layout: int = LAYOUT_LINEAR,
                             codes: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None,
                             stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """H = SwiGLU(alpha * A B^T) written as an MXFP4 operand along rows in
    h_layout; B's n = 2F rows interleave gate and up rows in groups of 32
    (pair_gate_up).  Returns (codes, scales) of H [m x F]."""
    M = a_codes.shape[0] if m is None else m
    N = b_codes.shape[0] if n is None else n
    K = a_codes.shape[1] * 2
    if b_codes.shape[1] * 2 != K:
        raise ValueError("A and B must have the same K")
    codes, scales = _mx_outputs(M, N // 2, h_layout, codes, scales, a_codes.device)
    _check("fp4_gemm_mx_swiglu_quant",
           lib().fp4_gemm_mx_swiglu_quant(a_codes.data_ptr(), a_scales.data_ptr(), b_codes.data_ptr(),
                                          b_scales.data_ptr(), M, N, K, float(alpha), layout, codes.data_ptr(),
                                          scales.data_ptr(), h_layout, _stream(stream)))
    return codes, scales


def fp4_swiglu_bf16(c: torch.Tensor, f: int, *, pair: int = 32, h: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """h = bf16(SiLU(gate) * up) from a bf16 C [M x >= 2f] whose columns
    interleave gate and up in groups of `pair` columns."""
    if c.dtype != torch.bfloat16 or c.dim() != 2 or c.stride(1) != 1:
        raise ValueError("c must be a 2-D bf16 tensor with contiguous rows")
    M = c.shape[0]
    if h is None:
        h = torch.empty((M, f), dtype=torch.bfloat16, device=c.device)
    if (h.dtype != torch.bfloat16 or h.dim() != 2 or h.stride(1) != 1 or tuple(h.shape) != (M, f)
            or h.device != c.device or (M > 1 and h.stride(0) < f)):
        raise ValueError(f"h must be a [{M} x {f}] bf16 tensor on {c.device} with unit column stride")
    _check("fp4_swiglu_bf16", lib().fp4_swiglu_bf16(c.data_ptr(), M, f, c.stride(0), pair, h.data_ptr(),
                                                    h.stride(0), _stream(stream)))
    return h


def pair_gate_up(w_gate: torch.Tensor, w_up: torch.Tensor, pair: int = 32) -> torch.Tensor:
    """The gate/up weight in the row order fp4_gemm_mx_swiglu_quant takes:
    rows 2 pair b .. + pair-1 = gate rows pair b .., the next pair rows the
    up rows of the same units (a one-time layout of the weight, like the
    tiled operand layout)."""
    F, K = w_gate.shape
    if w_up.shape != (F, K) or F % pair != 0:
        raise ValueError("gate and up must have the same [F x K] shape, F a multiple of pair")
    return torch.stack([w_gate.reshape(F // pair, pair, K), w_up.reshape(F // pair, pair, K)], dim=1).reshape(2 * F, K)


def fp4_gemm_nv(a_codes: torch.Tensor, a_scales: torch.Tensor, a_tensor_scale: torch.Tensor, b_codes: torch.Tensor,
                b_scales: torch.Tensor, b_tensor_scale: torch.Tensor, domain: int = NV_GLOBAL, *, alpha: float = 1.0,
                out_dtype=torch.float32, c: Optional[torch.Tensor] = None, c_amax: Optional[torch.Tensor] = None,
                layout: int = LAYOUT_LINEAR, m: Optional[int] = None, n: Optional[int] = None,
                stream=None) -> torch.Tensor:
    """With `c_amax` (a device float32 tensor) max |C| is folded into it
    (fp4_gemm_nv_amax).  In the tiled layout the code tensors carry rows
    padded to a multiple of 32, so pass the logical m and n."""
    M = a_codes.shape[0] if m is None else m
    N = b_codes.shape[0] if n is None else n
    K = a_codes.shape[1] * 2
    if b_codes.shape[1] * 2 != K:
        raise ValueError("A and B must have the same K")
    c, ctype, ldc = _gemm_out(M, N, out_dtype, a_codes.device, c)
    if c_amax is not None:
        _check("fp4_gemm_nv_amax",
               lib().fp4_gemm_nv_amax(a_codes.data_ptr(), a_scales.data_ptr(), a_tensor_scale.data_ptr(),
                                      b_codes.data_ptr(), b_scales.data_ptr(), b_tensor_scale.data_ptr(), domain, M, N,
                                      K, float(alpha), layout, c.data_ptr(), ctype, ldc, _amax_ptr(c_amax, a_codes.device),
                                      _stream(stream)))
        return c
    _check("fp4_gemm_nv", lib().fp4_gemm_nv(a_codes.data_ptr(), a_scales.data_ptr(), a_tensor_scale.data_ptr(),
                                            b_codes.data_ptr(), b_scales.data_ptr(), b_tensor_scale.data_ptr(),
                                            domain, M, N, K, float(alpha), layout, c.data_ptr(), ctype, ldc,
                                            _stream(stream)))
    return c
