"""The amax fusion: GEMMs that also report max |C| (fp4_gemm_*_amax) and the
one-pass "global nvfp" producer that takes that amax (fp4_quantize_nv_amax).
The reported amax must be exactly the maximum magnitude of the C the GEMM
stored (checked on the host, every element), folded into the running value
with max; the one-pass producer, given max |x|, must equal the CPU oracle's
two-pass global NVFP4 quantization byte for byte; chained after a GEMM it
must equal the two-pass producer run on the same C."""
import numpy as np
import pytest
import torch

from tests.gpu_common import B, announce, assert_bytes_equal, device, np_u8, oracle, synth

pytestmark = pytest.mark.gpu


def host_amax_bits(c: torch.Tensor) -> int:
    """max |C| of the stored output as binary32 bits."""
    if c.dtype == torch.bfloat16:
        bits = c.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32) & 0x7FFF
        return int(bits.max()) << 16 if bits.size else 0
    bits = c.cpu().numpy().view(np.uint32) & 0x7FFFFFFF
    return int(bits.max()) if bits.size else 0


def amax_bits(t: torch.Tensor) -> int:
    return int(t.cpu().numpy().view(np.uint32)[0])


def mx_pair(M, N, K, dev, layout):
    xa = synth.activation(M, K, 70).to(dev)
    xb = synth.weight(N, K, 71).to(dev)
    a = B.fp4_quantize_mx(xa, layout=layout)
    b = B.fp4_quantize_mx(xb, layout=layout)
    return a, b


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (33, 257, 384), (300, 200, 256), (512, 768, 1024)])
@pytest.mark.parametrize("out", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("layout", ["linear", "tiled"])
def test_gemm_mx_amax(M, N, K, out, layout):
    dev = device()
    announce(f"gemm mx amax {M}x{N}x{K} out={out} {layout}")
    L = B.LAYOUT_TILED if layout == "tiled" else B.LAYOUT_LINEAR
    (a, sa), (b, sb) = mx_pair(M, N, K, dev, L)
    amax = torch.zeros(1, dtype=torch.float32, device=dev)
    c = B.fp4_gemm_mx(a, sa, b, sb, alpha=-0.75, out_dtype=out, layout=L, m=M, n=N, c_amax=amax)
    torch.cuda.synchronize()
    assert amax_bits(amax) == host_amax_bits(c)
    # folded with max: a larger running value stays, a smaller one is raised
    big = torch.full((1,), 1e30, dtype=torch.float32, device=dev)
    small = torch.full((1,), 1e-30, dtype=torch.float32, device=dev)
    B.fp4_gemm_mx(a, sa, b, sb, alpha=-0.75, out_dtype=out, layout=L, m=M, n=N, c=c, c_amax=big)
    B.fp4_gemm_mx(a, sa, b, sb, alpha=-0.75, out_dtype=out, layout=L, m=M, n=N, c=c, c_amax=small)
    torch.cuda.synchronize()
    assert float(big.item()) == np.float32(1e30)
    assert amax_bits(small) == host_amax_bits(c)


def test_gemm_mx_amax_ldc_and_k_zero():
    dev = device()
    announce("gemm mx amax with ldc > N, and K = 0")
    M, N, K = 130, 200, 256
    (a, sa), (b, sb) = mx_pair(M, N, K, dev, B.LAYOUT_LINEAR)
    full = torch.full((M, N + 24), 1e4, dtype=torch.bfloat16, device=dev)
    c = full[:, :N]
    amax = torch.zeros(1, dtype=torch.float32, device=dev)
    B.fp4_gemm_mx(a, sa, b, sb, out_dtype=torch.bfloat16, c=c, c_amax=amax)
    torch.cuda.synchronize()
    assert amax_bits(amax) == host_amax_bits(c.contiguous())  # the padding columns (1e4) are not C
    # K = 0: C = 0 is written and the running amax is left as it was
    z = torch.zeros(1, dtype=torch.float32, device=dev)
    empty = [torch.empty((R, 0), dtype=torch.uint8, device=dev) for R in (M, M, N, N)]
    c0 = B.fp4_gemm_mx(*empty, c_amax=z)
    torch.cuda.synchronize()
    assert float(c0.abs().max().item()) == 0.0 and amax_bits(z) == 0


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (200, 300, 384), (256, 384, 1024)])
@pytest.mark.parametrize("domain", [0, 1])
def test_gemm_nv_amax(M, N, K, domain):
    dev = device()
    announce(f"gemm nv amax {M}x{N}x{K} domain={domain}")
    a = B.fp4_quantize_nv(synth.activation(M, K, 72).to(dev), domain)
    b = B.fp4_quantize_nv(synth.weight(N, K, 73).to(dev), domain)
    amax = torch.zeros(1, dtype=torch.float32, device=dev)
    c = B.fp4_gemm_nv(*a, *b, domain, alpha=1.5, out_dtype=torch.bfloat16, c_amax=amax)
    torch.cuda.synchronize()
    assert amax_bits(amax) == host_amax_bits(c)


NV1_SHAPES = [(1, 16), (37, 96), (256, 256), (129, 4096)]


@pytest.mark.parametrize("rows,cols", NV1_SHAPES)
@pytest.mark.parametrize("sr", [False, True])
def test_quantize_nv_one_pass_matches_oracle(rows, cols, sr):
    dev = device()
    announce(f"nv one pass {rows}x{cols} sr={sr}")
    xb = synth.bf16_bits(synth.activation(rows, cols, 74))
    amax_host = np.float32(np.abs(synth.from_bf16_bits(xb).float().numpy()).max())
    amax = torch.tensor([amax_host], dtype=torch.float32, device=dev)
    codes, scales, ts = B.fp4_quantize_nv(synth.from_bf16_bits(xb).to(dev), B.NV_GLOBAL, round=B.SR if sr else B.RNE,
                                          seed=5, stream_id=2, amax=amax)
    torch.cuda.synchronize()
    oc, os_, ots = oracle.quantize_nv(xb, sr=sr, seed=5, stream=2, domain=oracle.NV_GLOBAL)
    assert_bytes_equal(ts.cpu().numpy().view(np.uint32), ots.view(np.uint32), "tensor scale")
    assert_bytes_equal(np_u8(scales), os_, "block scales")
    assert_bytes_equal(np_u8(codes), oc, "codes")


@pytest.mark.parametrize("role", ["X", "W"])
@pytest.mark.parametrize("sr", [False, True])
def test_quantize_nv_one_pass_full_size(role, sr):
    # the NVFP4 configuration's operands (8192 x 4096 and 14336 x 4096) in one
    # pass from a host-computed amax, against the oracle's two-pass definition
    dev = device()
    announce(f"nv one pass full nvfp4.{role} sr={sr}")
    xt = synth.config_tensor("nvfp4", role)
    xb = synth.bf16_bits(xt)
    amax_host = np.float32(np.abs(xt.float().numpy()).max())
    amax = torch.tensor([amax_host], dtype=torch.float32, device=dev)
    codes, scales, ts = B.fp4_quantize_nv(xt.to(dev), B.NV_GLOBAL, round=B.SR if sr else B.RNE, seed=5,
                                          stream_id=2, amax=amax)
    oc, os_, ots = oracle.quantize_nv(xb, sr=sr, seed=5, stream=2, domain=oracle.NV_GLOBAL)
    torch.cuda.synchronize()
    assert_bytes_equal(ts.cpu().numpy().view(np.uint32), ots.view(np.uint32), "tensor scale")
    assert_bytes_equal(np_u8(scales), os_, "block scales")
    assert_bytes_equal(np_u8(codes), oc, "codes")


def test_quantize_nv_one_pass_zero_amax():
    # an all-zero operand: amax 0 gives S = 1, zero codes, as the two-pass producer
    dev = device()
    announce("nv one pass zero operand")
    x = torch.zeros((64, 128), dtype=torch.bfloat16, device=dev)
    codes, scales, ts = B.fp4_quantize_nv(x, B.NV_GLOBAL, amax=torch.zeros(1, dtype=torch.float32, device=dev))
    torch.cuda.synchronize()
    oc, os_, ots = oracle.quantize_nv(synth.bf16_bits(x.cpu()), domain=oracle.NV_GLOBAL)
    assert_bytes_equal(ts.cpu().numpy().view(np.uint32), ots.view(np.uint32), "tensor scale")
    assert_bytes_equal(np_u8(scales), os_, "block scales")
    assert_bytes_equal(np_u8(codes), oc, "codes")


@pytest.mark.parametrize("sr", [False, True])
def test_chain_gemm_amax_then_one_pass(sr):
    # NV GEMM with its output amax, then the one-pass producer on that output:
    # identical to the two-pass producer on the same output
    dev = device()
    announce(f"chain nv gemm -> one-pass nv quantize sr={sr}")
    M, N, K = 512, 1024, 512
    a = B.fp4_quantize_nv(synth.activation(M, K, 75).to(dev), B.NV_GLOBAL)
    b = B.fp4_quantize_nv(synth.weight(N, K, 76).to(dev), B.NV_GLOBAL)
    amax = torch.zeros(1, dtype=torch.float32, device=dev)
    c = B.fp4_gemm_nv(*a, *b, B.NV_GLOBAL, out_dtype=torch.bfloat16, c_amax=amax)
    one = B.fp4_quantize_nv(c, B.NV_GLOBAL, round=B.SR if sr else B.RNE, seed=3, amax=amax)
    two = B.fp4_quantize_nv(c, B.NV_GLOBAL, round=B.SR if sr else B.RNE, seed=3)
    torch.cuda.synchronize()
    assert amax_bits(amax) == host_amax_bits(c)
    for g, w, name in zip(one, two, ("codes", "block scales", "tensor scale")):
        assert_bytes_equal(np_u8(g.view(torch.uint8)), np_u8(w.view(torch.uint8)), name)
