"""The C-ABI library loads, exports every function include/fp4q.h declares,
and rejects bad arguments with the documented status before any HIP call
(so these run without a GPU; the pointers below are never dereferenced)."""
import ctypes

import pytest
import torch

from fp4_block_scaled_quantizer_amd import binding as B

L = None
X = 0x7F0000000000  # fake, 16-byte aligned device addresses far apart
CODES = 0x7F1000000000
SCALES = 0x7F2000000000
TS = 0x7F3000000000
WS = 0x7F4000000000
C = 0x7F5000000000


@pytest.fixture(scope="module", autouse=True)
def lib():
    global L
    L = B.lib()
    return L


def test_exports_every_declared_function():
    names = B.declared_functions()
    assert set(names) >= {"fp4_quantize_mx", "fp4_quantize_nv", "fp4_hadamard32_quantize", "fp4_quantize_mx_dual",
                          "fp4_quantize_nv_amax", "fp4_hadamard32_quantize_nv", "fp4_gemm_mx", "fp4_gemm_nv",
                          "fp4_gemm_mx_amax", "fp4_gemm_nv_amax", "fp4_gemm_mx_quant", "fp4_gemm_mx_swiglu_quant",
                          "fp4_swiglu_bf16"}
    for n in names:
        assert hasattr(L, n), n
    assert B.abi_version() == 1
    for s in range(6):
        assert B.status_str(s)


def q_mx(x=X, rows=64, cols=64, ld=64, axis=0, rnd=0, codes=CODES, scales=SCALES, layout=0):
    return L.fp4_quantize_mx(x, rows, cols, ld, axis, rnd, 7, 0, codes, scales, layout, None)


def test_quantize_mx_status_codes():
    assert q_mx(axis=2) == B.EINVAL
    assert q_mx(rnd=5) == B.EINVAL
    assert q_mx(layout=3) == B.EINVAL
    assert q_mx(x=None) == B.EINVAL
    assert q_mx(codes=None) == B.EINVAL
    assert q_mx(scales=None) == B.EINVAL
    assert q_mx(cols=48, ld=48) == B.ESHAPE          # K % 32
    assert q_mx(axis=1, rows=48) == B.ESHAPE         # K = rows % 32
    assert q_mx(axis=1, cols=62, ld=64) == B.ESHAPE  # column axis needs cols % 4
    assert q_mx(ld=32) == B.ESHAPE                   # ld < cols
    assert q_mx(rows=-1) == B.ESHAPE
    assert q_mx(rows=2**31) == B.ESHAPE
    assert q_mx(x=X + 8) == B.EALIGN
    assert q_mx(codes=CODES + 4) == B.EALIGN
    assert q_mx(ld=68) == B.EALIGN
    assert q_mx(codes=X + 64) == B.EINVAL            # output overlaps input
    assert q_mx(scales=CODES + 16) == B.EINVAL       # outputs overlap
    # empty operands are valid and enqueue nothing
    assert q_mx(rows=0) == B.OK
    assert q_mx(axis=1, rows=0) == B.OK


def test_hadamard_status_codes():
    f = L.fp4_hadamard32_quantize
    assert f(X, 64, 64, 64, 1, 0xFFFF, 0, 0, 0, CODES, SCALES, 2, None) == B.EINVAL
    assert f(X, 40, 64, 64, 1, 0xFFFF, 0, 0, 0, CODES, SCALES, 0, None) == B.ESHAPE
    assert f(X, 0, 64, 64, 1, 0xFFFF, 0, 0, 0, CODES, SCALES, 0, None) == B.OK


def q_nv(rows=64, cols=64, ld=64, axis=0, dom=0, ts=TS, ws=WS, wbytes=None, x=X):
    if wbytes is None:
        wbytes = L.fp4q_nv_workspace_bytes(rows, cols, axis, dom)
    return L.fp4_quantize_nv(x, rows, cols, ld, axis, 0, 0, 0, dom, CODES, SCALES, ts, ws, wbytes, 0, None)


def test_quantize_nv_status_codes():
    assert L.fp4q_nv_workspace_bytes(64, 64, 0, 0) > 0
    assert L.fp4q_nv_workspace_bytes(64, 64, 0, 1) == 0
    assert q_nv(dom=2) == B.EINVAL
    assert q_nv(axis=1) in (B.OK, B.ELAUNCH)         # along columns is valid (no GPU here: the launch fails)
    assert q_nv(axis=1, rows=40) == B.ESHAPE         # K = rows % 16
    assert q_nv(axis=1, cols=62, ld=64) == B.ESHAPE  # column axis needs cols % 4
    assert q_nv(cols=40, ld=48) == B.ESHAPE
    assert q_nv(ts=None) == B.EINVAL
    assert q_nv(ws=None) == B.EINVAL
    assert q_nv(wbytes=4) == B.EINVAL
    assert q_nv(ts=TS + 2) == B.EALIGN
    assert q_nv(ws=X) == B.EINVAL                    # workspace overlaps input
    assert q_nv(dom=1, ws=None, wbytes=0, rows=0) == B.OK


def g_mx(M=256, N=256, K=256, layout=0, ctype=0, ldc=None, c=C, a_codes=CODES, a_scales=SCALES):
    ldc = N if ldc is None else ldc
    return L.fp4_gemm_mx(a_codes, a_scales, 0x7F6000000000, 0x7F7000000000, M, N, K, 1.0, layout, c, ctype, ldc,
                         None)


def test_gemm_mx_status_codes():
    assert g_mx(layout=2) == B.EINVAL
    assert g_mx(ctype=3) == B.EINVAL
    assert g_mx(c=None) == B.EINVAL
    assert g_mx(a_codes=None) == B.EINVAL
    assert g_mx(K=96) == B.ESHAPE
    assert g_mx(ldc=100) == B.ESHAPE
    assert g_mx(M=-3) == B.ESHAPE
    assert g_mx(a_codes=CODES + 8) == B.EALIGN
    assert g_mx(a_scales=SCALES + 2) == B.EALIGN
    assert g_mx(c=C + 2) == B.EALIGN
    assert g_mx(c=CODES) == B.EINVAL                 # C overlaps A codes
    assert g_mx(M=0) == B.OK and g_mx(N=0) == B.OK


def test_gemm_nv_status_codes():
    f = L.fp4_gemm_nv
    args = (CODES, SCALES, TS, 0x7F6000000000, 0x7F7000000000, 0x7F8000000000)
    assert f(*args, 2, 256, 256, 256, 1.0, 0, C, 0, 256, None) == B.EINVAL
    assert f(*args, 0, 256, 256, 200, 1.0, 0, C, 0, 256, None) == B.ESHAPE
    assert f(CODES, SCALES, None, 0x7F6000000000, 0x7F7000000000, 0x7F8000000000, 1, 256, 256, 256, 1.0, 0, C, 0,
             256, None) == B.EINVAL
    assert f(*args, 1, 256, 256, 256, 1.0, 0, TS, 0, 256, None) == B.EINVAL  # C overlaps a tensor scale
    assert f(*args, 0, 0, 256, 256, 1.0, 0, C, 0, 256, None) == B.OK


def test_binding_has_no_cpu_fallback(monkeypatch, tmp_path):
    # the binding refuses to run when the library is absent
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(FileNotFoundError):
        B.lib()


def test_tiled_layout_status_codes():
    assert q_mx(layout=1, cols=96, ld=96) == B.ESHAPE             # tiled needs K % 128
    assert q_mx(layout=1, cols=128, ld=128, scales=SCALES + 4) == B.EALIGN
    assert q_mx(layout=2) == B.EINVAL
    # NVFP4 tiled: K % 128 (the 64-column operand has K = 64), 16-byte aligned scales
    assert L.fp4_quantize_nv(X, 64, 64, 64, 0, 0, 0, 0, 0, CODES, SCALES, TS, WS, 4096, 1, None) == B.ESHAPE
    assert L.fp4_quantize_nv(X, 32, 128, 128, 0, 0, 0, 0, 0, CODES, SCALES + 4, TS, WS, 4096, 1, None) == B.EALIGN
    assert L.fp4_quantize_nv_noalloc(X, 64, 64, 64, 0, 0, 0, 0, 0, CODES, SCALES, TS, 1, None) == B.ESHAPE
    assert g_mx(layout=1, K=96) == B.ESHAPE
    assert g_mx(layout=3) == B.EINVAL


CODES2 = 0x7F6000000000
SCALES2 = 0x7F7000000000


def q_dual(x=X, rows=64, cols=64, ld=64, rr=0, had=1, rc=0, codes_r=CODES, scales_r=SCALES, codes_c=CODES2,
           scales_c=SCALES2, layout=0):
    return L.fp4_quantize_mx_dual(x, rows, cols, ld, rr, 0, codes_r, scales_r, had, 0xF0F0F0F0, rc, 1, codes_c,
                                  scales_c, 7, layout, None)


def test_quantize_mx_dual_status_codes():
    assert q_dual(rr=2) == B.EINVAL
    assert q_dual(rc=3) == B.EINVAL
    assert q_dual(had=2) == B.EINVAL
    assert q_dual(layout=2) == B.EINVAL
    assert q_dual(x=None) == B.EINVAL
    assert q_dual(codes_r=None) == B.EINVAL
    assert q_dual(scales_c=None) == B.EINVAL
    assert q_dual(cols=48, ld=48) == B.ESHAPE            # K of the row operand % 32
    assert q_dual(rows=48) == B.ESHAPE                   # K of the column operand % 32
    assert q_dual(rows=96, layout=1) == B.ESHAPE         # tiled: rows % 128
    assert q_dual(rows=128, cols=96, ld=96, layout=1) == B.ESHAPE
    assert q_dual(ld=32) == B.ESHAPE
    assert q_dual(rows=-1) == B.ESHAPE
    assert q_dual(x=X + 8) == B.EALIGN
    assert q_dual(codes_c=CODES2 + 4) == B.EALIGN
    assert q_dual(codes_c=CODES + 512) == B.EINVAL       # the two operands' codes overlap
    assert q_dual(scales_c=SCALES + 16) == B.EINVAL      # the two operands' scales overlap
    assert q_dual(codes_r=X + 64) == B.EINVAL            # output overlaps input
    assert q_dual(rows=0) == B.OK                        # empty: nothing enqueued
    assert q_dual(cols=0, ld=0) == B.OK


AMAX = 0x7F8000000000


def test_amax_entry_points_status_codes():
    def g_mx(amax=AMAX, c=C):
        return L.fp4_gemm_mx_amax(CODES, SCALES, CODES2, SCALES2, 64, 64, 128, 1.0, 0, c, 1, 64, amax, None)

    def g_nv(amax=AMAX, c=C):
        return L.fp4_gemm_nv_amax(CODES, SCALES, TS, CODES2, SCALES2, TS + 64, 0, 64, 64, 128, 1.0, 0, c, 1, 64,
                                  amax, None)

    def q_nv1(amax=AMAX, cols=64):
        return L.fp4_quantize_nv_amax(X, 64, cols, 64, 0, 7, 0, amax, CODES, SCALES, TS, None)

    for g in (g_mx, g_nv):
        assert g(amax=None) == B.EINVAL
        assert g(amax=AMAX + 2) == B.EALIGN
        assert g(amax=C + 64) == B.EINVAL        # inside C
    assert q_nv1(amax=None) == B.EINVAL
    assert q_nv1(amax=AMAX + 1) == B.EALIGN
    assert q_nv1(amax=CODES + 16) == B.EINVAL    # overlaps an output
    assert q_nv1(cols=24) == B.ESHAPE            # K % 16


def test_hadamard_nv_status_codes():
    def q(axis=1, rows=64, cols=64, ld=64, dom=0, rnd=0):
        wb = L.fp4q_nv_workspace_bytes(rows, cols, axis, dom)
        return L.fp4_hadamard32_quantize_nv(X, rows, cols, ld, axis, 0x1234, rnd, 7, 0, dom, CODES, SCALES, TS, WS,
                                            wb, 0, None)

    assert q() in (B.OK, B.ELAUNCH)       # valid (no GPU here: the launch fails)
    assert q(dom=1) in (B.OK, B.ELAUNCH)
    assert q(axis=0) == B.EUNSUPPORTED   # along rows not built
    assert q(rows=48) == B.ESHAPE        # K = rows % 32
    assert q(cols=62, ld=64) == B.ESHAPE
    assert q(rnd=3) == B.EINVAL


def test_gemm_mx_quant_status_codes():
    def g(M=64, N=128, K=128, layout=0, cl=0, codes=CODES2, scales=SCALES2, a=CODES):
        return L.fp4_gemm_mx_quant(a, SCALES, X, C, M, N, K, 1.0, layout, codes, scales, cl, None)

    assert g() in (B.OK, B.ELAUNCH)      # valid (no GPU here: the launch fails)
    assert g(layout=2) == B.EINVAL
    assert g(cl=2) == B.EINVAL
    assert g(K=96) == B.ESHAPE           # K % 128
    assert g(N=48) == B.ESHAPE           # N % 32 (linear output)
    assert g(N=96, cl=1) == B.ESHAPE     # N % 128 (tiled output)
    assert g(M=-1) == B.ESHAPE
    assert g(codes=None) == B.EINVAL
    assert g(a=None) == B.EINVAL
    assert g(codes=CODES2 + 8) == B.EALIGN
    assert g(scales=SCALES2 + 2) == B.EALIGN
    assert g(scales=CODES2 + 16) == B.EINVAL   # output codes and scales overlap
    assert g(codes=CODES + 64) == B.EINVAL     # output overlaps an input
    assert g(M=0) == B.OK


def test_gemm_mx_swiglu_quant_status_codes():
    def g(M=64, N=128, K=128, layout=0, hl=0, codes=CODES2, scales=SCALES2, a=CODES):
        return L.fp4_gemm_mx_swiglu_quant(a, SCALES, X, C, M, N, K, 1.0, layout, codes, scales, hl, None)

    assert g() in (B.OK, B.ELAUNCH)      # valid (no GPU here: the launch fails)
    assert g(N=256, hl=1) in (B.OK, B.ELAUNCH)
    assert g(layout=2) == B.EINVAL
    assert g(hl=2) == B.EINVAL
    assert g(K=96) == B.ESHAPE           # K % 128
    assert g(N=96) == B.ESHAPE           # N % 64: F = N / 2 a multiple of 32 (linear output)
    assert g(N=128, hl=1) == B.ESHAPE    # N % 256: F a multiple of 128 (tiled output)
    assert g(M=-1) == B.ESHAPE
    assert g(codes=None) == B.EINVAL
    assert g(a=None) == B.EINVAL
    assert g(codes=CODES2 + 8) == B.EALIGN
    assert g(scales=SCALES2 + 2) == B.EALIGN
    assert g(scales=CODES2 + 16) == B.EINVAL   # output codes and scales overlap
    assert g(codes=CODES + 64) == B.EINVAL     # output overlaps an input
    assert g(M=0) == B.OK


def test_swiglu_status_codes():
    def s(M=16, F=64, ldc=128, pair=32, h=C, ldh=64, c=X):
        return L.fp4_swiglu_bf16(c, M, F, ldc, pair, h, ldh, None)

    assert s() in (B.OK, B.ELAUNCH)
    assert s(pair=64) in (B.OK, B.ELAUNCH)
    assert s(F=60, ldc=120, ldh=64) == B.ESHAPE   # F % 8
    assert s(pair=12) == B.ESHAPE                 # pair % 8
    assert s(pair=48) == B.ESHAPE                 # pair does not divide F
    assert s(ldc=120) == B.ESHAPE                 # ldc < 2F
    assert s(ldh=56) == B.ESHAPE                  # ldh < F
    assert s(ldc=132) == B.ESHAPE                 # ldc % 8
    assert s(M=-1) == B.ESHAPE
    assert s(c=None) == B.EINVAL
    assert s(h=None) == B.EINVAL
    assert s(c=X + 8) == B.EALIGN
    assert s(h=C + 2) == B.EALIGN
    assert s(h=X + 64) == B.EINVAL                # h overlaps c
    assert s(M=0) == B.OK


def test_size_limits():
    # fake device addresses 16 TiB apart, so that only the size rule decides
    x, codes, scales, c = 0x100000000000, 0x200000000000, 0x300000000000, 0x400000000000
    # MX producer: the 8-element chunk count must stay below 2^32
    assert q_mx(x=x, rows=2 ** 22, cols=2 ** 13, ld=2 ** 13, codes=codes, scales=scales) == B.ESHAPE
    assert q_mx(x=x, rows=2 ** 22 - 32, cols=2 ** 13, ld=2 ** 13, codes=codes, scales=scales) in (B.OK, B.ELAUNCH)
    # tiled: the padded row count counts (2^22 - 31 rows pad to 2^22)
    assert q_mx(x=x, rows=2 ** 22 - 31, cols=2 ** 13, ld=2 ** 13, codes=codes, scales=scales, layout=1) == B.ESHAPE
    # MX GEMM: each operand's code bytes must stay below 2^32
    def g(M, N=256, K=8192, a=codes, sa=scales, b=x, sb=x + (1 << 40)):
        return L.fp4_gemm_mx(a, sa, b, sb, M, N, K, 1.0, 0, c, 0, N, None)

    assert g(M=2 ** 20) == B.ESHAPE                  # 2^20 rows x 4096 bytes = 2^32
    assert g(M=2 ** 20 - 1) in (B.OK, B.ELAUNCH)
    assert g(M=256, N=2 ** 20) == B.ESHAPE
    # dimensions above INT32_MAX are rejected outright
    assert g(M=2 ** 31) == B.ESHAPE


def test_binding_rejects_wrong_output_buffers():
    # the C ABI cannot see buffer sizes: the binding checks every
    # caller-supplied output before calling it (CPU tensors: it raises
    # before any library call)
    x = torch.zeros((64, 128), dtype=torch.bfloat16)
    u8 = torch.uint8
    bad_mx = [
        dict(codes=torch.zeros((63, 64), dtype=u8)),                    # too few rows
        dict(codes=torch.zeros((64, 128), dtype=u8)[:, :64]),           # strided view
        dict(codes=torch.zeros((64, 64), dtype=torch.int16)),           # dtype
        dict(scales=torch.zeros((64, 3), dtype=u8)),                    # shape
    ]
    for kw in bad_mx:
        with pytest.raises(ValueError):
            B.fp4_quantize_mx(x, **kw)
    with pytest.raises(ValueError):
        B.fp4_quantize_mx(x, layout=B.LAYOUT_TILED, codes=torch.zeros((64, 64), dtype=u8),
                          scales=torch.zeros((64, 4), dtype=u8))      # tiled scales are [K/128, Rp, 4]
    for kw in [dict(codes=torch.zeros((64, 32), dtype=u8)), dict(scales=torch.zeros((64, 4), dtype=u8)),
               dict(tensor_scale=torch.zeros((2,), dtype=torch.float32)),
               dict(tensor_scale=torch.zeros((1,), dtype=torch.float64))]:
        with pytest.raises(ValueError):
            B.fp4_quantize_nv(x, B.NV_GLOBAL, **kw)
    a = torch.zeros((64, 64), dtype=u8)
    s = torch.zeros((64, 4), dtype=u8)
    for c in [torch.zeros((63, 64)), torch.zeros((64, 128))[:, ::2], torch.zeros((64, 64), dtype=torch.float16)]:
        with pytest.raises(ValueError):
            B.fp4_gemm_mx(a, s, a, s, c=c)
    with pytest.raises(ValueError):
        B.fp4_swiglu_bf16(torch.zeros((4, 64), dtype=torch.bfloat16), 32, h=torch.zeros((4, 16), dtype=torch.bfloat16))
