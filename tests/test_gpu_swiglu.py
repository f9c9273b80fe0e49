"""GPU checks of the SwiGLU path: fp4_swiglu_bf16 against the oracle
(interleaved and [gate | up] layouts, padded row pitches, every finite bf16
gate), equal to it except where the oracle's value lies within the
kernel's proven SiLU error of a bf16 midpoint (tests/swiglu_rule.py; those
elements are counted and printed), and fp4_gemm_mx_swiglu_quant -- the gate/up GEMM whose epilogue
writes SwiGLU(C) as an MXFP4 operand -- byte for byte against the chain it
fuses: the bf16 GEMM, fp4_swiglu_bf16 and the MX row producer (each pinned
to the oracle by its own tests), for both input and output layouts, ragged
M, alpha != 1, K = 0 and the full MLP gate/up size."""
import numpy as np
import pytest
import torch

from tests.gpu_common import B, announce, assert_bytes_equal, bf16_bits_of, device, np_u8, oracle, synth
from tests.swiglu_rule import check_h


def up_values(c_bits, F, pair):
    """float64 up value of every hidden column (the layout of C)."""
    j = np.arange(F)
    ucol = (j // pair) * 2 * pair + (j % pair) + pair
    return (c_bits[:, ucol].astype(np.uint32) << 16).view(np.float32).astype(np.float64)

pytestmark = pytest.mark.gpu


def gate_up_c(M, F, pair, ldc, seed):
    """bf16 C [M x ldc] with SwiGLU-like gate (heavy both sides) and up
    columns; columns past 2F are filler."""
    g = torch.Generator().manual_seed(seed)
    c = torch.randn((M, ldc), generator=g) * 4.0
    return c.to(torch.bfloat16)


@pytest.mark.parametrize("M,F,pair,pad", [(1, 32, 32, 0), (37, 320, 32, 8), (129, 1024, 64, 0), (64, 256, 256, 16),
                                          (300, 2048, 32, 0)])
def test_swiglu_matches_oracle(M, F, pair, pad):
    dev = device()
    announce(f"swiglu {M}x{F} pair={pair} pad={pad}")
    ldc = 2 * F + pad
    c = gate_up_c(M, F, pair, ldc, seed=M + F)
    h = torch.full((M, F + pad), float("nan"), dtype=torch.bfloat16, device=dev)
    B.fp4_swiglu_bf16(c.to(dev), F, pair=pair, h=h[:, :F])
    cb = bf16_bits_of(c)
    want, hv = oracle.swiglu_bf16(cb, F, pair, with_f64=True)
    torch.cuda.synchronize()
    got = bf16_bits_of(h)
    nd, na = check_h(got[:, :F], want, hv, up_values(cb, F, pair))
    print(f"swiglu {M}x{F}: {nd} values differ from the oracle, {na} near a bf16 midpoint")
    assert np.all(got[:, F:] == bf16_bits_of(torch.full((1,), float("nan"), dtype=torch.bfloat16))[0])


def test_swiglu_special_values():
    # every bf16 bit pattern that is finite as the gate, against up values
    # of both signs, small and large: covers -0, subnormals, the -80 / 20
    # cut-offs and overflow of the product
    dev = device()
    announce("swiglu all finite bf16 gates")
    allb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = (allb.astype(np.uint32) << 16).view(np.float32)
    gates = allb[np.isfinite(f)]
    F = 1024
    M = (gates.size + F - 1) // F
    gpad = np.zeros(M * F, dtype=np.uint16)
    gpad[:gates.size] = gates
    ups = synth.bf16_bits(torch.tensor(np.random.default_rng(3).choice(
        np.float32([1.0, -1.0, 3.0e38, -2.5, 1e-30, 0.0, 7.0]), M * F), dtype=torch.bfloat16)).reshape(M, F)
    # [gate | up] layout (pair = F)
    c = np.concatenate([gpad.reshape(M, F), ups], axis=1)
    ct = synth.from_bf16_bits(c).to(dev)
    h = B.fp4_swiglu_bf16(ct, F, pair=F)
    want, hv = oracle.swiglu_bf16(c, F, F, with_f64=True)
    torch.cuda.synchronize()
    got = bf16_bits_of(h)
    nd, na = check_h(got, want, hv, up_values(c, F, F))
    print(f"swiglu all gates: {nd} values differ from the oracle, {na} with a neighbour admitted")


def operands(M, N, K, dev, layout, seed=120):
    a = B.fp4_quantize_mx(synth.activation(M, K, seed).to(dev), layout=layout)
    b = B.fp4_quantize_mx(synth.weight(N, K, seed + 1).to(dev), layout=layout)
    return a, b


def unfused(a, b, M, N, alpha, layout, h_layout):
    c16 = B.fp4_gemm_mx(*a, *b, alpha=alpha, out_dtype=torch.bfloat16, layout=layout, m=M, n=N)
    h = B.fp4_swiglu_bf16(c16, N // 2, pair=32)
    return B.fp4_quantize_mx(h, layout=h_layout)


CASES = [(1, 256, 128), (33, 512, 384), (300, 768, 256), (512, 1280, 1024), (640, 2048, 2048)]


@pytest.mark.parametrize("M,N,K", CASES)
@pytest.mark.parametrize("layout", ["linear", "tiled"])
@pytest.mark.parametrize("h_layout", ["linear", "tiled"])
@pytest.mark.parametrize("alpha", [1.0, -0.375])
def test_gemm_swiglu_quant_equals_chain(M, N, K, layout, h_layout, alpha):
    dev = device()
    announce(f"gemm mx swiglu quant {M}x{N}x{K} in={layout} out={h_layout} alpha={alpha}")
    L = B.LAYOUT_TILED if layout == "tiled" else B.LAYOUT_LINEAR
    HL = B.LAYOUT_TILED if h_layout == "tiled" else B.LAYOUT_LINEAR
    a, b = operands(M, N, K, dev, L)
    cs, ss = B.mx_output_shapes(M, N // 2, HL)
    codes = torch.full(cs, 0xA5, dtype=torch.uint8, device=dev)  # poisoned: every byte must be written
    scales = torch.full(ss, 0xA5, dtype=torch.uint8, device=dev)
    B.fp4_gemm_mx_swiglu_quant(*a, *b, alpha=alpha, layout=L, m=M, n=N, h_layout=HL, codes=codes, scales=scales)
    rc, rs = unfused(a, b, M, N, alpha, L, HL)
    torch.cuda.synchronize()
    assert_bytes_equal(np_u8(scales), np_u8(rs), "scales")
    assert_bytes_equal(np_u8(codes), np_u8(rc), "codes")


def test_gemm_swiglu_quant_f_not_multiple_of_64():
    # linear output: F % 32 == 0 suffices (the last wave holds one block)
    dev = device()
    announce("gemm mx swiglu quant N = 320, linear output")
    M, N, K = 200, 320, 512
    a, b = operands(M, N, K, dev, B.LAYOUT_LINEAR, seed=122)
    codes, scales = B.fp4_gemm_mx_swiglu_quant(*a, *b, m=M, n=N)
    rc, rs = unfused(a, b, M, N, 1.0, B.LAYOUT_LINEAR, B.LAYOUT_LINEAR)
    torch.cuda.synchronize()
    assert_bytes_equal(np_u8(scales), np_u8(rs), "scales")
    assert_bytes_equal(np_u8(codes), np_u8(rc), "codes")


def test_gemm_swiglu_quant_k_zero():
    dev = device()
    announce("gemm mx swiglu quant K = 0")
    M, N = 45, 512
    empty = [torch.empty((R, 0), dtype=torch.uint8, device=dev) for R in (M, M, N, N)]
    for HL in (B.LAYOUT_LINEAR, B.LAYOUT_TILED):
        cs, ss = B.mx_output_shapes(M, N // 2, HL)
        codes = torch.full(cs, 0xA5, dtype=torch.uint8, device=dev)
        scales = torch.full(ss, 0xA5, dtype=torch.uint8, device=dev)
        B.fp4_gemm_mx_swiglu_quant(*empty, m=M, n=N, h_layout=HL, codes=codes, scales=scales)
        torch.cuda.synchronize()
        assert int(codes.max().item()) == 0 and int(scales.max().item()) == 0


def test_pair_gate_up_row_order():
    # the weight layout helper: row 64 b + r = gate row 32 b + r (r < 32),
    # row 64 b + 32 + r = up row 32 b + r
    g = torch.arange(96 * 4, dtype=torch.float32).reshape(96, 4)
    u = -g
    p = B.pair_gate_up(g, u)
    for b in range(3):
        assert torch.equal(p[64 * b:64 * b + 32], g[32 * b:32 * b + 32])
        assert torch.equal(p[64 * b + 32:64 * b + 64], u[32 * b:32 * b + 32])


def test_gemm_swiglu_quant_full_size_mlp_gate_up():
    dev = device()
    announce("gemm mx swiglu quant full 8192x28672x4096 tiled")
    X = synth.config_tensor("mlp_gate_up", "X").to(dev)
    W = synth.config_tensor("mlp_gate_up", "W").to(dev)
    M, N, K = X.shape[0], W.shape[0], X.shape[1]
    L = B.LAYOUT_TILED
    a = B.fp4_quantize_mx(X, layout=L)
    b = B.fp4_quantize_mx(W, layout=L)  # its rows taken as paired gate/up rows
    codes, scales = B.fp4_gemm_mx_swiglu_quant(*a, *b, layout=L, m=M, n=N, h_layout=L)
    rc, rs = unfused(a, b, M, N, 1.0, L, L)
    torch.cuda.synchronize()
    assert_bytes_equal(np_u8(scales), np_u8(rs), "scales")
    assert_bytes_equal(np_u8(codes), np_u8(rc), "codes")
