"""The fused GEMM epilogues against the oracle, on every element.

fp4_gemm_mx_quant writes C = A B^T as the next GEMM's MXFP4 operand and
fp4_gemm_mx_swiglu_quant writes H = SwiGLU(C) as one; neither writes C.  To
compare them with the oracle without feeding any GPU value to it, the
operands are built so that the GEMM is exact: random E2M1 codes with E8M0
scale bytes drawn from a narrow range, so that every partial sum of every
output is an integer multiple of the smallest product below 2^24 of it --
exactly representable in binary32 in any summation order.  The oracle's
float64 C is then the kernel's binary32 accumulator bit for bit (asserted),
its bf16 rounding is the kernel's, and the expected outputs are the oracle's
quantize_mx(bf16(C)) and quantize_mx(swiglu_bf16(bf16(C))).  The SwiGLU case
uses the validity rule of tests/swiglu_rule.py: an MX block may differ from
the oracle's only if it holds an H value the rule admits other than the
oracle's, and must then equal the quantization of an admitted choice.
Full Llama-3-8B MLP sizes and small ragged ones, both layouts."""
import numpy as np
import pytest
import torch

from tests.gpu_common import B, announce, assert_bytes_equal, device, np_u8, oracle, untile_mx
from tests.swiglu_rule import check_quantized_h

pytestmark = pytest.mark.gpu


def exact_operand(R, K, seed, e_base, e_span):
    """Random MX operand [R x K] (linear layout): uniform codes, scale bytes
    127 + e_base + {0 .. e_span - 1}."""
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, (R, K // 2), dtype=np.uint8)
    scales = (127 + e_base + rng.integers(0, e_span, (R, K // 32))).astype(np.uint8)
    return codes, scales


def exact_pair(M, N, K, seed):
    """A [M x K], B [N x K] whose GEMM is exact in binary32: products are
    multiples of u0 = 2^-2 2^(ea_min + eb_min), at most 36 2^(ea_max +
    eb_max) = 144 2^(spans - 2) u0 each, so every partial sum of K of them
    stays below 2^24 u0."""
    sa, sb = (3, 2) if K <= 4096 else (2, 2)
    assert K * 144 * 2 ** (sa + sb - 2) < 2 ** 24, "not exact in binary32"
    a = exact_operand(M, K, seed, -4, sa)
    b = exact_operand(N, K, seed + 1, -4, sb)
    return a, b


def upload(op, layout, dev):
    codes, scales = op
    if layout == B.LAYOUT_TILED:
        codes, scales = oracle.tile_mx(codes, scales)
    return torch.from_numpy(np.ascontiguousarray(codes)).to(dev), torch.from_numpy(np.ascontiguousarray(scales)).to(dev)


def exact_c(a, b, alpha):
    """The oracle's C (float64), checked to be a binary32 value everywhere."""
    C, _ = oracle.gemm_ref(oracle.dequant_mx(*a), oracle.dequant_mx(*b), alpha, weights=False)
    assert np.array_equal(C, C.astype(np.float32).astype(np.float64)), "C is not exact in binary32"
    return C


def linear_out(codes, scales, R, K, layout):
    c, s = np_u8(codes), np_u8(scales)
    if layout == B.LAYOUT_TILED:
        c, s, cpad, spad = untile_mx(c, s, R, K)
        assert not cpad.any() and not spad.any(), "tiled padding rows must be zero"
    return c, s


CASES = [(1, 256, 128), (33, 512, 384), (300, 768, 256), (640, 2048, 2048)]


@pytest.mark.parametrize("M,N,K", CASES)
@pytest.mark.parametrize("layout", ["linear", "tiled"])
@pytest.mark.parametrize("c_layout", ["linear", "tiled"])
@pytest.mark.parametrize("alpha", [1.0, -0.5])
def test_gemm_quant_against_oracle(M, N, K, layout, c_layout, alpha):
    dev = device()
    announce(f"gemm mx quant vs oracle {M}x{N}x{K} in={layout} out={c_layout} alpha={alpha}")
    L = B.LAYOUT_TILED if layout == "tiled" else B.LAYOUT_LINEAR
    CL = B.LAYOUT_TILED if c_layout == "tiled" else B.LAYOUT_LINEAR
    a, b = exact_pair(M, N, K, seed=M + N + K)
    codes, scales = B.fp4_gemm_mx_quant(*upload(a, L, dev), *upload(b, L, dev), alpha=alpha, layout=L, m=M, n=N,
                                        c_layout=CL)
    want_c, want_s = oracle.quantize_mx(oracle.double_to_bf16_array(exact_c(a, b, alpha)))
    torch.cuda.synchronize()
    got_c, got_s = linear_out(codes, scales, M, N, CL)
    assert_bytes_equal(got_s, want_s, "scales")
    assert_bytes_equal(got_c, want_c, "codes")


def swiglu_expect(a, b, alpha, F):
    cb = oracle.double_to_bf16_array(exact_c(a, b, alpha))
    h, hv = oracle.swiglu_bf16(cb, F, 32, with_f64=True)
    j = np.arange(F)
    ucol = (j // 32) * 64 + (j % 32) + 32
    u = (cb[:, ucol].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return h, hv, u


@pytest.mark.parametrize("M,N,K", CASES)
@pytest.mark.parametrize("layout", ["linear", "tiled"])
@pytest.mark.parametrize("h_layout", ["linear", "tiled"])
@pytest.mark.parametrize("alpha", [1.0, -0.5])
def test_gemm_swiglu_quant_against_oracle(M, N, K, layout, h_layout, alpha):
    dev = device()
    announce(f"gemm mx swiglu quant vs oracle {M}x{N}x{K} in={layout} out={h_layout} alpha={alpha}")
    L = B.LAYOUT_TILED if layout == "tiled" else B.LAYOUT_LINEAR
    HL = B.LAYOUT_TILED if h_layout == "tiled" else B.LAYOUT_LINEAR
    a, b = exact_pair(M, N, K, seed=7 * M + N + K)
    codes, scales = B.fp4_gemm_mx_swiglu_quant(*upload(a, L, dev), *upload(b, L, dev), alpha=alpha, layout=L, m=M,
                                               n=N, h_layout=HL)
    h, hv, u = swiglu_expect(a, b, alpha, N // 2)
    torch.cuda.synchronize()
    got_c, got_s = linear_out(codes, scales, M, N // 2, HL)
    nb, na = check_quantized_h(got_c, got_s, h, hv, u, oracle.quantize_mx)
    print(f"{M}x{N}x{K}: {nb} MX blocks differ from the oracle's, {na} hold a near-midpoint H value")


def test_gemm_quant_full_size_mlp_up_against_oracle():
    # the MLP up projection's output 8192 x 14336 (K = 4096) quantized in
    # the epilogue, every element against the oracle
    dev = device()
    M, N, K = 8192, 14336, 4096
    announce(f"gemm mx quant vs oracle full {M}x{N}x{K} tiled")
    L = B.LAYOUT_TILED
    a, b = exact_pair(M, N, K, seed=301)
    codes, scales = B.fp4_gemm_mx_quant(*upload(a, L, dev), *upload(b, L, dev), layout=L, m=M, n=N, c_layout=L)
    want_c, want_s = oracle.quantize_mx(oracle.double_to_bf16_array(exact_c(a, b, 1.0)))
    torch.cuda.synchronize()
    got_c, got_s = linear_out(codes, scales, M, N, L)
    assert_bytes_equal(got_s, want_s, "scales")
    assert_bytes_equal(got_c, want_c, "codes")


def test_gemm_swiglu_quant_full_size_mlp_gate_up_against_oracle():
    # the gate/up projection 8192 x 28672 x 4096 with SwiGLU and the MX
    # producer of H (8192 x 14336) in its epilogue, every block against the
    # oracle under the validity rule
    dev = device()
    M, N, K = 8192, 28672, 4096
    announce(f"gemm mx swiglu quant vs oracle full {M}x{N}x{K} tiled")
    L = B.LAYOUT_TILED
    a, b = exact_pair(M, N, K, seed=302)
    codes, scales = B.fp4_gemm_mx_swiglu_quant(*upload(a, L, dev), *upload(b, L, dev), layout=L, m=M, n=N,
                                               h_layout=L)
    h, hv, u = swiglu_expect(a, b, 1.0, N // 2)
    torch.cuda.synchronize()
    got_c, got_s = linear_out(codes, scales, M, N // 2, L)
    nb, na = check_quantized_h(got_c, got_s, h, hv, u, oracle.quantize_mx)
    print(f"full gate/up: {nb} of {M * N // 64} MX blocks differ from the oracle's, {na} hold a near-midpoint H value")
