"""Operands near the library's size limits: element offsets past 2^32 in the
producers (16 GiB of bf16 input), and a GEMM operand of almost 2^32 code
bytes (the 32-bit DMA offsets' range).  The outputs at sampled rows and
32-row groups (first, middle, last) equal the oracle's."""
import numpy as np
import pytest
import torch

from tests.gpu_common import B, announce, assert_bytes_equal, bf16_bits_of, device, gemm_check, oracle

pytestmark = pytest.mark.gpu


def big_bf16(R, K, dev, seed, scale=0.5):
    """A seeded [R x K] bf16 tensor filled slice by slice (bounded
    temporaries)."""
    g = torch.Generator(device=dev).manual_seed(seed)
    x = torch.empty((R, K), dtype=torch.bfloat16, device=dev)
    step = max(1, (1 << 28) // K)
    for r0 in range(0, R, step):
        r1 = min(R, r0 + step)
        x[r0:r1] = (torch.randn((r1 - r0, K), generator=g, device=dev) * scale).to(torch.bfloat16)
    return x


def test_mx_rows_past_32bit_element_offsets():
    # 262144 x 32768 bf16: element offsets reach 2^33, 2^30 chunks of 8
    dev = device()
    R, K = 262144, 32768
    announce(f"limits: mx rows {R}x{K} linear + tiled")
    x = big_bf16(R, K, dev, seed=501)
    codes, scales = B.fp4_quantize_mx(x, layout=B.LAYOUT_LINEAR)
    for r in (0, 1, R // 2 - 1, R // 2, R - 1):
        wc, ws = oracle.quantize_mx(bf16_bits_of(x[r:r + 1]))
        assert_bytes_equal(codes[r:r + 1].cpu().numpy(), wc, f"codes row {r}")
        assert_bytes_equal(scales[r:r + 1].cpu().numpy(), ws, f"scales row {r}")
    del codes, scales
    codes, scales = B.fp4_quantize_mx(x, layout=B.LAYOUT_TILED)
    for g in (0, R // 64, R // 32 - 1):
        wc, ws = oracle.tile_mx(*oracle.quantize_mx(bf16_bits_of(x[32 * g:32 * g + 32])))
        assert_bytes_equal(codes[32 * g:32 * g + 32].cpu().numpy(), wc, f"tiled codes group {g}")
        assert_bytes_equal(scales[:, 32 * g:32 * g + 32].cpu().numpy(), ws, f"tiled scales group {g}")


def test_mx_columns_past_32bit_element_offsets():
    # x 131072 x 32768 quantized along columns: the logical operand is
    # 32768 x 131072; element offsets of x reach 2^32
    dev = device()
    rows, cols = 131072, 32768
    announce(f"limits: mx columns of {rows}x{cols}, tiled")
    x = big_bf16(rows, cols, dev, seed=502)
    codes, scales = B.fp4_quantize_mx(x, axis=B.ALONG_COLS, layout=B.LAYOUT_TILED)
    for g in (0, cols // 64, cols // 32 - 1):
        xt = bf16_bits_of(x[:, 32 * g:32 * g + 32]).T.copy()  # logical rows 32 g .. 32 g + 31
        wc, ws = oracle.tile_mx(*oracle.quantize_mx(xt))
        assert_bytes_equal(codes[32 * g:32 * g + 32].cpu().numpy(), wc, f"codes group {g}")
        assert_bytes_equal(scales[:, 32 * g:32 * g + 32].cpu().numpy(), ws, f"scales group {g}")


def test_nv_tile_rows_past_32bit_element_offsets():
    dev = device()
    R, K = 262144, 32768
    announce(f"limits: nv tile128 rows {R}x{K}")
    x = big_bf16(R, K, dev, seed=503)
    codes, scales, ts = B.fp4_quantize_nv(x, domain=B.NV_TILE128)
    TK = K // 128
    for tr in (0, R // 256, R // 128 - 1):  # whole 128-row tiles (their scales S)
        rows = slice(128 * tr, 128 * tr + 128)
        wc, ws, wt = oracle.quantize_nv(bf16_bits_of(x[rows]), domain=oracle.NV_TILE128)
        assert_bytes_equal(codes[rows].cpu().numpy(), wc, f"codes tile row {tr}")
        assert_bytes_equal(scales[rows].cpu().numpy(), ws, f"scales tile row {tr}")
        got_ts = ts.reshape(R // 128, TK)[tr].cpu().numpy()
        assert np.array_equal(got_ts.view(np.uint32), np.asarray(wt, dtype=np.float32).reshape(-1).view(np.uint32))


def to_tiled(codes, scales):
    """Linear MX operand -> the tiled layout, on the device (R % 32 == 0)."""
    R, K2 = codes.shape
    K = 2 * K2
    tc = codes.reshape(R // 32, 32, K // 64, 2, 16).permute(0, 2, 3, 1, 4).reshape(R, K2).contiguous()
    ts = scales.reshape(R, K // 128, 4).permute(1, 0, 2).contiguous()
    return tc, ts


@pytest.mark.parametrize("layout", ["linear", "tiled"])
def test_gemm_mx_operand_near_4gib(layout):
    # A has (2^20 - 256) rows x 8192 K: 4 GiB - 1 MiB of codes, the largest
    # the 32-bit DMA offsets allow at this K
    dev = device()
    M, N, K = (1 << 20) - 256, 256, 8192
    announce(f"limits: gemm mx {M}x{N}x{K} {layout}")
    g = torch.Generator(device=dev).manual_seed(504)
    a = torch.randint(0, 256, (M, K // 2), dtype=torch.uint8, device=dev, generator=g)
    sa = torch.randint(120, 135, (M, K // 32), dtype=torch.uint8, device=dev, generator=g)
    b = torch.randint(0, 256, (N, K // 2), dtype=torch.uint8, device=dev, generator=g)
    sb = torch.randint(120, 135, (N, K // 32), dtype=torch.uint8, device=dev, generator=g)
    if layout == "tiled":
        ta, tsa = to_tiled(a, sa)
        tb, tsb = to_tiled(b, sb)
        c = B.fp4_gemm_mx(ta, tsa, tb, tsb, out_dtype=torch.float32, layout=B.LAYOUT_TILED, m=M, n=N)
        del ta, tsa, tb, tsb
    else:
        c = B.fp4_gemm_mx(a, sa, b, sb, out_dtype=torch.float32)
    rows = [0, 1, 255, M // 2, M - 257, M - 1]
    bq = oracle.dequant_mx(b.cpu().numpy(), sb.cpu().numpy())
    aq = oracle.dequant_mx(a[rows].cpu().numpy(), sa[rows].cpu().numpy())
    ref, w = oracle.gemm_ref(aq, bq)
    gemm_check(c[rows].cpu().numpy(), ref, w, f"gemm rows {rows}")
