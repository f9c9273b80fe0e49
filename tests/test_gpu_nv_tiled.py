"""The NVFP4 tiled consumer layout on the GPU: the producers (rows: per-tile
and global domain, RNE and SR; columns with and without the Hadamard;
the allocation-free variant) against oracle.tile_nv of the oracle's linear
outputs, byte for byte with every padding byte checked (outputs poisoned
first); the NVFP4 GEMM on tiled operands against the fp64 oracle and equal,
bit for bit, to the same GEMM on linear operands; and the full Llama-3-8B
NVFP4 size, every element."""
import numpy as np
import pytest
import torch

from tests.gpu_common import B, announce, assert_bytes_equal, device, gemm_check, np_u8, oracle, synth

pytestmark = pytest.mark.gpu

T = B.LAYOUT_TILED


def poisoned(R, K, dev):
    cs, ss = B.nv_output_shapes(R, K, T)
    return (torch.full(cs, 0xA5, dtype=torch.uint8, device=dev), torch.full(ss, 0xA5, dtype=torch.uint8, device=dev))


def check_tiled(codes, scales, ts, oc, os_, ots, what):
    tc, tsc = oracle.tile_nv(oc, os_)
    assert_bytes_equal(np_u8(codes), tc, f"{what} codes")
    assert_bytes_equal(np_u8(scales), tsc, f"{what} scales")
    assert np.array_equal(ts.cpu().numpy().view(np.uint32), ots.view(np.uint32)), f"{what} tensor scales"


@pytest.mark.parametrize("rows,cols", [(1, 128), (37, 256), (200, 384), (256, 1024), (300, 640)])
@pytest.mark.parametrize("domain", [0, 1])
@pytest.mark.parametrize("sr", [False, True])
def test_nv_rows_tiled(rows, cols, domain, sr):
    dev = device()
    announce(f"nv tiled rows {rows}x{cols} domain={domain} sr={sr}")
    xt = synth.activation(rows, cols, rows + cols)
    c, s = poisoned(rows, cols, dev)
    _, _, ts = B.fp4_quantize_nv(xt.to(dev), domain, round=B.SR if sr else B.RNE, seed=7, stream_id=3, codes=c,
                                 scales=s, layout=T)
    oc, os_, ots = oracle.quantize_nv(synth.bf16_bits(xt), sr=sr, seed=7, stream=3, domain=domain)
    torch.cuda.synchronize()
    check_tiled(c, s, ts, oc, os_, ots, "rows")


@pytest.mark.parametrize("rows,cols", [(128, 40), (256, 128), (384, 200), (128, 1000)])
@pytest.mark.parametrize("domain", [0, 1])
@pytest.mark.parametrize("had", [None, 0x6C3A9E15])
def test_nv_cols_tiled(rows, cols, domain, had):
    dev = device()
    announce(f"nv tiled cols {rows}x{cols} domain={domain} hadamard={had is not None}")
    xt = synth.grad_student_t3(rows, cols, rows + 3 * cols)
    c, s = poisoned(cols, rows, dev)
    sr = had is not None
    _, _, ts = B.fp4_quantize_nv(xt.to(dev), domain, axis=B.ALONG_COLS, round=B.SR if sr else B.RNE, seed=7,
                                 stream_id=1, hadamard_mask=had, codes=c, scales=s, layout=T)
    xb = synth.bf16_bits(xt)
    if had is None:
        oc, os_, ots = oracle.quantize_nv(xb, axis=oracle.AXIS_COLS, sr=sr, seed=7, stream=1, domain=domain)
    else:
        oc, os_, ots = oracle.hadamard32_quantize_nv(xb, had, axis=oracle.AXIS_COLS, sr=sr, seed=7, stream=1,
                                                     domain=domain)
    torch.cuda.synchronize()
    check_tiled(c, s, ts, oc, os_, ots, "cols")


def test_nv_noalloc_tiled():
    dev = device()
    announce("nv noalloc tiled")
    xt = synth.activation(96, 512, 71)
    c, s = poisoned(96, 512, dev)
    _, _, ts = B.fp4_quantize_nv_noalloc(xt.to(dev), 0, codes=c, scales=s, layout=T)
    oc, os_, ots = oracle.quantize_nv(synth.bf16_bits(xt), domain=0)
    torch.cuda.synchronize()
    check_tiled(c, s, ts, oc, os_, ots, "noalloc")


def nv_pair(xt, dev, domain, layout):
    return B.fp4_quantize_nv(xt.to(dev), domain, layout=layout)


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (200, 300, 384), (256, 384, 1024), (511, 129, 256)])
@pytest.mark.parametrize("domain", [0, 1])
def test_nv_gemm_tiled(M, N, K, domain):
    dev = device()
    announce(f"nv gemm tiled {M}x{N}x{K} domain={domain}")
    xa, xb = synth.activation(M, K, 80), synth.weight(N, K, 81)
    a_t = nv_pair(xa, dev, domain, T)
    b_t = nv_pair(xb, dev, domain, T)
    a_l = nv_pair(xa, dev, domain, B.LAYOUT_LINEAR)
    b_l = nv_pair(xb, dev, domain, B.LAYOUT_LINEAR)
    c_t = B.fp4_gemm_nv(*a_t, *b_t, domain, alpha=0.5, layout=T, m=M, n=N)
    c_l = B.fp4_gemm_nv(*a_l, *b_l, domain, alpha=0.5)
    c16 = B.fp4_gemm_nv(*a_t, *b_t, domain, alpha=0.5, layout=T, m=M, n=N, out_dtype=torch.bfloat16)
    oa = oracle.quantize_nv(synth.bf16_bits(xa), domain=domain)
    ob = oracle.quantize_nv(synth.bf16_bits(xb), domain=domain)
    cref, w = oracle.gemm_ref(oracle.dequant_nv(*oa, domain), oracle.dequant_nv(*ob, domain), 0.5)
    torch.cuda.synchronize()
    ct = c_t.cpu().numpy()
    gemm_check(ct, cref, w, f"nv tiled {M}x{N}x{K} d{domain}")
    # the same products and the same accumulation order as the linear layout
    assert np.array_equal(ct.view(np.uint32), c_l.cpu().numpy().view(np.uint32))
    from tests import second_formulation as sf
    assert np.array_equal(c16.view(torch.int16).cpu().numpy().view(np.uint16), sf.f32_to_bf16_bits_rne(ct))


@pytest.mark.parametrize("domain", [0, 1])
def test_nv_tiled_full_size(domain):
    # the Llama-3-8B NVFP4 GEMM 8192 x 14336 x 4096 on tiled operands, every
    # element against the fp64 oracle (operands checked against it first)
    dev = device()
    announce(f"nv tiled full domain={domain}")
    xa, xb = synth.config_tensor("nvfp4", "X"), synth.config_tensor("nvfp4", "W")
    M, N, K = xa.shape[0], xb.shape[0], xa.shape[1]
    a = nv_pair(xa, dev, domain, T)
    b = nv_pair(xb, dev, domain, T)
    c = B.fp4_gemm_nv(*a, *b, domain, layout=T, m=M, n=N)
    oa = oracle.quantize_nv(synth.bf16_bits(xa), domain=domain)
    ob = oracle.quantize_nv(synth.bf16_bits(xb), domain=domain)
    torch.cuda.synchronize()
    check_tiled(*a, *oa, "A")
    check_tiled(*b, *ob, "B")
    cref, w = oracle.gemm_ref(oracle.dequant_nv(*oa, domain), oracle.dequant_nv(*ob, domain))
    worst = gemm_check(c.cpu().numpy(), cref, w, f"nv tiled full d{domain}")
    print(f"nv tiled domain {domain}: worst |err| / sum|ab| = {worst:.3e}")


_SR_ORACLE = {}


@pytest.mark.parametrize("domain", [0, 1])
@pytest.mark.parametrize("layout", ["linear", "tiled"])
def test_nv_sr_rows_full_size(domain, layout):
    # the backward workload's dY (8192 x 4096, Student-t with 3 degrees of
    # freedom, scaled 1e-3) along rows with stochastic rounding, in both
    # scale domains and both layouts: every code, block scale and tensor
    # scale against the oracle (the workgroups past the first wave included)
    dev = device()
    announce(f"nv SR rows full backward.dY domain={domain} {layout}")
    xt = synth.config_tensor("backward", "dY")
    codes, scales, ts = B.fp4_quantize_nv(xt.to(dev), domain, round=B.SR, seed=7, stream_id=3,
                                          layout=T if layout == "tiled" else B.LAYOUT_LINEAR)
    if domain not in _SR_ORACLE:
        _SR_ORACLE[domain] = oracle.quantize_nv(synth.bf16_bits(xt), sr=True, seed=7, stream=3, domain=domain)
    oc, os_, ots = _SR_ORACLE[domain]
    torch.cuda.synchronize()
    if layout == "tiled":
        check_tiled(codes, scales, ts, oc, os_, ots, "dY")
    else:
        assert np.array_equal(ts.cpu().numpy().view(np.uint32), ots.view(np.uint32)), "tensor scales"
        assert_bytes_equal(np_u8(scales), os_, "block scales")
        assert_bytes_equal(np_u8(codes), oc, "codes")

