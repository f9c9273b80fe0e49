"""GPU checks of the MXFP4 GEMM that writes its output as the next GEMM's
MXFP4 operand (fp4_gemm_mx_quant): every output byte (codes, E8M0 scales,
padding rows) equals the MX row producer applied to the bf16 C of the plain
GEMM -- the two library paths that the other tests pin to the oracle -- for
both input and output layouts, ragged M, alpha != 1, K = 0, and the MLP
up-projection size."""
import numpy as np
import pytest
import torch

from tests.gpu_common import B, announce, assert_bytes_equal, device, np_u8, synth

pytestmark = pytest.mark.gpu


def operands(M, N, K, dev, layout, seed=90):
    a = B.fp4_quantize_mx(synth.activation(M, K, seed).to(dev), layout=layout)
    b = B.fp4_quantize_mx(synth.weight(N, K, seed + 1).to(dev), layout=layout)
    return a, b


def unfused(a, b, M, N, alpha, layout, c_layout):
    c16 = B.fp4_gemm_mx(*a, *b, alpha=alpha, out_dtype=torch.bfloat16, layout=layout, m=M, n=N)
    return B.fp4_quantize_mx(c16, layout=c_layout)


CASES = [(1, 128, 128), (33, 256, 384), (300, 384, 256), (512, 640, 1024), (640, 1024, 2048)]


@pytest.mark.parametrize("M,N,K", CASES)
@pytest.mark.parametrize("layout", ["linear", "tiled"])
@pytest.mark.parametrize("c_layout", ["linear", "tiled"])
@pytest.mark.parametrize("alpha", [1.0, -0.375])
def test_gemm_mx_quant_equals_gemm_then_producer(M, N, K, layout, c_layout, alpha):
    dev = device()
    announce(f"gemm mx quant {M}x{N}x{K} in={layout} out={c_layout} alpha={alpha}")
    L = B.LAYOUT_TILED if layout == "tiled" else B.LAYOUT_LINEAR
    CL = B.LAYOUT_TILED if c_layout == "tiled" else B.LAYOUT_LINEAR
    a, b = operands(M, N, K, dev, L)
    # poisoned outputs: every byte (padding rows included) must be written
    cs, ss = B.mx_output_shapes(M, N, CL)
    codes = torch.full(cs, 0xA5, dtype=torch.uint8, device=dev)
    scales = torch.full(ss, 0xA5, dtype=torch.uint8, device=dev)
    B.fp4_gemm_mx_quant(*a, *b, alpha=alpha, layout=L, m=M, n=N, c_layout=CL, codes=codes, scales=scales)
    rc, rs = unfused(a, b, M, N, alpha, L, CL)
    torch.cuda.synchronize()
    assert_bytes_equal(np_u8(scales), np_u8(rs), "scales")
    assert_bytes_equal(np_u8(codes), np_u8(rc), "codes")


def test_gemm_mx_quant_linear_n_not_multiple_of_128():
    # linear output: N % 32 == 0 suffices (a partial last 128-column group)
    dev = device()
    announce("gemm mx quant N = 352, linear output")
    M, N, K = 200, 352, 512
    a, b = operands(M, N, K, dev, B.LAYOUT_LINEAR, seed=92)
    codes, scales = B.fp4_gemm_mx_quant(*a, *b, m=M, n=N)
    rc, rs = unfused(a, b, M, N, 1.0, B.LAYOUT_LINEAR, B.LAYOUT_LINEAR)
    torch.cuda.synchronize()
    assert_bytes_equal(np_u8(scales), np_u8(rs), "scales")
    assert_bytes_equal(np_u8(codes), np_u8(rc), "codes")


def test_gemm_mx_quant_k_zero():
    dev = device()
    announce("gemm mx quant K = 0")
    M, N = 45, 256
    empty = [torch.empty((R, 0), dtype=torch.uint8, device=dev) for R in (M, M, N, N)]
    for CL in (B.LAYOUT_LINEAR, B.LAYOUT_TILED):
        cs, ss = B.mx_output_shapes(M, N, CL)
        codes = torch.full(cs, 0xA5, dtype=torch.uint8, device=dev)
        scales = torch.full(ss, 0xA5, dtype=torch.uint8, device=dev)
        B.fp4_gemm_mx_quant(*empty, m=M, n=N, c_layout=CL, codes=codes, scales=scales)
        torch.cuda.synchronize()
        assert int(codes.max().item()) == 0 and int(scales.max().item()) == 0


def test_gemm_mx_quant_full_size_mlp_up():
    dev = device()
    announce("gemm mx quant full 8192x14336x4096 tiled")
    X = synth.config_tensor("qkv", "X").to(dev)
    W = synth.config_tensor("nvfp4", "W").to(dev)
    M, N, K = X.shape[0], W.shape[0], X.shape[1]
    L = B.LAYOUT_TILED
    a = B.fp4_quantize_mx(X, layout=L)
    b = B.fp4_quantize_mx(W, layout=L)
    codes, scales = B.fp4_gemm_mx_quant(*a, *b, layout=L, m=M, n=N, c_layout=L)
    rc, rs = unfused(a, b, M, N, 1.0, L, L)
    torch.cuda.synchronize()
    assert_bytes_equal(np_u8(scales), np_u8(rs), "scales")
    assert_bytes_equal(np_u8(codes), np_u8(rc), "codes")
