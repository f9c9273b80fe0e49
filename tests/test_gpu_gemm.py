"""GPU parity of the block-scaled FP4 GEMMs: every fp32 output element within
1e-5 * |alpha| * sum_k |dq(a) dq(b)| of the fp64 reference on the oracle's
dequantized operands; bf16 outputs equal to round-to-nearest-even of the same
kernel's fp32 output.  Operands come from the GPU producers, which the
quantizer tests pin byte for byte to the oracle; here they are compared to the
oracle's bytes again before the GEMM is checked."""
import numpy as np
import pytest
import torch

from tests.gpu_common import (B, announce, assert_bytes_equal, device, gemm_check, np_u8, oracle, synth)
from tests import second_formulation as sf

pytestmark = pytest.mark.gpu


def mx_operand(xt, dev, axis=B.ALONG_ROWS, sr=False, had=False, mask=0, stream=0):
    xb = synth.bf16_bits(xt)
    x = xt.to(dev)
    if had:
        c, s = B.fp4_hadamard32_quantize(x, mask, axis=axis, round=B.SR if sr else B.RNE, seed=synth.SR_SEED,
                                         stream_id=stream)
        oc, os_ = oracle.hadamard32_quantize(xb, mask, axis=axis, sr=sr, seed=synth.SR_SEED, stream=stream)
    else:
        c, s = B.fp4_quantize_mx(x, axis=axis, round=B.SR if sr else B.RNE, seed=synth.SR_SEED, stream_id=stream)
        oc, os_ = oracle.quantize_mx(xb, axis=axis, sr=sr, seed=synth.SR_SEED, stream=stream)
    torch.cuda.synchronize()
    assert_bytes_equal(np_u8(c), oc, "operand codes")
    assert_bytes_equal(np_u8(s), os_, "operand scales")
    return c, s, oc, os_


def test_tiny_config_bruteforce():
    dev = device()
    announce("gemm mx tiny 256^3")
    a, sa, oa, osa = mx_operand(synth.config_tensor("tiny", "A"), dev)
    b, sb, ob, osb = mx_operand(synth.config_tensor("tiny", "B"), dev)
    c = B.fp4_gemm_mx(a, sa, b, sb)
    c16 = B.fp4_gemm_mx(a, sa, b, sb, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    cref, w = oracle.gemm_bruteforce(oracle.dequant_mx(oa, osa), oracle.dequant_mx(ob, osb))
    gemm_check(c.cpu().numpy(), cref, w, "tiny fp32")
    want16 = sf.f32_to_bf16_bits_rne(c.cpu().numpy())
    got16 = c16.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got16, want16), "bf16 output != RNE of the fp32 output"


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (33, 257, 384), (300, 200, 256), (256, 512, 1024),
                                   (511, 129, 128), (640, 384, 2048)])
@pytest.mark.parametrize("alpha", [1.0, -0.375])
def test_mx_ragged(M, N, K, alpha):
    dev = device()
    announce(f"gemm mx ragged {M}x{N}x{K} alpha={alpha}")
    a, sa, oa, osa = mx_operand(synth.activation(M, K, 20), dev)
    b, sb, ob, osb = mx_operand(synth.weight(N, K, 21), dev)
    c = B.fp4_gemm_mx(a, sa, b, sb, alpha=alpha)
    torch.cuda.synchronize()
    cref, w = oracle.gemm_ref(oracle.dequant_mx(oa, osa), oracle.dequant_mx(ob, osb), alpha)
    gemm_check(c.cpu().numpy(), cref, w, f"{M}x{N}x{K}")


def test_mx_ldc_and_k_zero():
    dev = device()
    announce("gemm mx ldc > N, K = 0")
    M, N, K = 64, 96, 256
    a, sa, oa, osa = mx_operand(synth.activation(M, K, 22), dev)
    b, sb, ob, osb = mx_operand(synth.weight(N, K, 23), dev)
    big = torch.full((M, 128), 7.0, dtype=torch.float32, device=dev)
    B.fp4_gemm_mx(a, sa, b, sb, c=big[:, :N])
    torch.cuda.synchronize()
    cref, w = oracle.gemm_ref(oracle.dequant_mx(oa, osa), oracle.dequant_mx(ob, osb))
    gemm_check(big[:, :N].cpu().numpy(), cref, w, "ldc")
    assert torch.all(big[:, N:] == 7.0)
    z = torch.empty((0,), dtype=torch.uint8, device=dev)
    c0 = torch.full((5, 6), 3.0, device=dev)
    B.lib().fp4_gemm_mx(z.data_ptr(), z.data_ptr(), z.data_ptr(), z.data_ptr(), 5, 6, 0, 1.0, 0, c0.data_ptr(), 0,
                        6, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.all(c0 == 0)


def test_mx_one_hot_layout_pins():
    # single nonzero elements with distinct scales per K block pin the nibble
    # order, the lane -> (row, K) mapping and the scale-byte selection
    dev = device()
    announce("gemm mx one-hot pins")
    M, N, K = 64, 64, 256
    rng = np.random.default_rng(30)
    for trial in range(6):
        A = np.zeros((M, K), np.float32)
        Bm = np.zeros((N, K), np.float32)
        for _ in range(6):
            A[rng.integers(M), rng.integers(K)] = rng.choice([0.5, 1.0, -3.0, 6.0]) * 2.0 ** rng.integers(-8, 8)
            Bm[rng.integers(N), rng.integers(K)] = rng.choice([1.5, -2.0, 4.0]) * 2.0 ** rng.integers(-8, 8)
        k = int(rng.integers(K))
        A[int(rng.integers(M)), k] = 1.0
        Bm[int(rng.integers(N)), k] = -1.5
        a, sa, oa, osa = mx_operand(synth.from_bf16_bits(sf.f32_to_bf16_bits_rne(A)), dev)
        b, sb, ob, osb = mx_operand(synth.from_bf16_bits(sf.f32_to_bf16_bits_rne(Bm)), dev)
        c = B.fp4_gemm_mx(a, sa, b, sb)
        torch.cuda.synchronize()
        cref, _ = oracle.gemm_bruteforce(oracle.dequant_mx(oa, osa), oracle.dequant_mx(ob, osb))
        assert np.array_equal(c.cpu().numpy().astype(np.float64), cref), f"trial {trial}"


def test_hadamard_wgrad_identity_on_gpu():
    dev = device()
    announce("gemm mx hadamard identity")
    mask = synth.sign_mask(7)
    x = np.zeros((128, 128), np.uint16)
    for i in range(128):
        x[i, i] = 0x3F80
    xt = synth.from_bf16_bits(x)
    a, sa, _, _ = mx_operand(xt, dev, axis=B.ALONG_COLS, had=True, mask=mask)
    c = B.fp4_gemm_mx(a, sa, a, sa, alpha=1.0 / 32)
    torch.cuda.synchronize()
    # tokens i and j live in the same 32-block iff i // 32 == j // 32
    want = np.eye(128)
    assert np.array_equal(c.cpu().numpy().astype(np.float64), want)


FULL_GEMMS = [
    # (name, A spec, B spec, alpha)
    ("qkv", ("qkv", "X", "rows", False, False, 0), ("qkv", "W", "rows", False, False, 0), 1.0),
    ("mlp_gate_up", ("mlp_gate_up", "X", "rows", False, False, 0), ("mlp_gate_up", "W", "rows", False, False, 0), 1.0),
    ("mlp_down", ("mlp_down", "H", "rows", False, False, 0), ("mlp_down", "W", "rows", False, False, 0), 1.0),
    ("dgrad", ("backward", "dY", "rows", True, False, 0), ("backward", "W", "cols", False, False, 1), 1.0),
    ("wgrad", ("backward", "dY", "cols", True, True, 1), ("backward", "X", "cols", False, True, 1), 1.0 / 32),
]


# every element of every configuration's GEMM is checked against the fp64
# oracle (0.3 - 1.9 TFLOP of fp64 library matmul on the host, seconds each)
ALL_ELEMENTS = {g[0] for g in FULL_GEMMS}


@pytest.mark.parametrize("name,aspec,bspec,alpha", FULL_GEMMS, ids=[g[0] for g in FULL_GEMMS])
def test_mx_full_size(name, aspec, bspec, alpha):
    dev = device()
    announce(f"gemm mx full {name}")
    mask = synth.sign_mask(synth.HADAMARD_MASK_SEED)

    def operand(spec):
        cfg, role, axis, sr, had, stream = spec
        return mx_operand(synth.config_tensor(cfg, role), dev, axis=B.ALONG_ROWS if axis == "rows" else B.ALONG_COLS,
                          sr=sr, had=had, mask=mask, stream=stream)

    a, sa, oa, osa = operand(aspec)
    b, sb, ob, osb = operand(bspec)
    c = B.fp4_gemm_mx(a, sa, b, sb, alpha=alpha)
    c16 = B.fp4_gemm_mx(a, sa, b, sb, alpha=alpha, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    M = oa.shape[0]
    if name in ALL_ELEMENTS:
        rows = np.arange(M)
    else:
        rows = np.unique(np.concatenate([np.arange(0, M, max(1, M // 96)), [M - 1]]))[:128]
    A = oracle.dequant_mx(oa[rows], osa[rows])
    Bd = oracle.dequant_mx(ob, osb)
    cref, w = oracle.gemm_ref(A, Bd, alpha)
    cg = c[torch.as_tensor(rows, device=dev)].cpu().numpy()
    worst = gemm_check(cg, cref, w, name)
    got16 = c16[torch.as_tensor(rows, device=dev)].view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got16, sf.f32_to_bf16_bits_rne(cg)), "bf16 output != RNE of fp32 output"
    print(f"{name}: worst |err| / sum|ab| = {worst:.3e}")


# ------------------------------------------------------------------ NVFP4


def nv_operand(xt, dev, domain):
    xb = synth.bf16_bits(xt)
    c, s, ts = B.fp4_quantize_nv(xt.to(dev), domain)
    torch.cuda.synchronize()
    oc, os_, ots = oracle.quantize_nv(xb, domain=domain)
    assert_bytes_equal(np_u8(c), oc, "nv codes")
    assert_bytes_equal(np_u8(s), os_, "nv scales")
    assert_bytes_equal(ts.cpu().numpy().view(np.uint32), ots.view(np.uint32), "nv tensor scales")
    return c, s, ts, oc, os_, ots


@pytest.mark.parametrize("M,N,K", [(128, 128, 128), (1, 1, 128), (200, 300, 384), (256, 384, 1024)])
@pytest.mark.parametrize("domain", [0, 1])
def test_nv_small(M, N, K, domain):
    dev = device()
    announce(f"gemm nv {M}x{N}x{K} domain={domain}")
    a, sa, ta, oa, osa, ota = nv_operand(synth.activation(M, K, 40), dev, domain)
    b, sb, tb, ob, osb, otb = nv_operand(synth.weight(N, K, 41), dev, domain)
    c = B.fp4_gemm_nv(a, sa, ta, b, sb, tb, domain, alpha=0.5)
    c16 = B.fp4_gemm_nv(a, sa, ta, b, sb, tb, domain, alpha=0.5, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    cref, w = oracle.gemm_ref(oracle.dequant_nv(oa, osa, ota, domain), oracle.dequant_nv(ob, osb, otb, domain), 0.5)
    gemm_check(c.cpu().numpy(), cref, w, f"nv {M}x{N}x{K} d{domain}")
    got16 = c16.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got16, sf.f32_to_bf16_bits_rne(c.cpu().numpy()))


@pytest.mark.parametrize("domain", [0, 1])
def test_nv_full_size(domain):
    # every element of the 8192 x 14336 x 4096 NVFP4 GEMM against the fp64 oracle
    dev = device()
    announce(f"gemm nv full domain={domain}")
    a, sa, ta, oa, osa, ota = nv_operand(synth.config_tensor("nvfp4", "X"), dev, domain)
    b, sb, tb, ob, osb, otb = nv_operand(synth.config_tensor("nvfp4", "W"), dev, domain)
    c = B.fp4_gemm_nv(a, sa, ta, b, sb, tb, domain)
    torch.cuda.synchronize()
    cref, w = oracle.gemm_ref(oracle.dequant_nv(oa, osa, ota, domain), oracle.dequant_nv(ob, osb, otb, domain))
    worst = gemm_check(c.cpu().numpy(), cref, w, f"nv full d{domain}")
    print(f"nv domain {domain}: worst |err| / sum|ab| = {worst:.3e}")


# ------------------------------------------------------------------ tiled layout


def mx_operand_tiled(xt, dev, axis=B.ALONG_ROWS, sr=False, had=False, mask=0, stream=0):
    """Tiled operand from the GPU producer (checked against the oracle's tiled
    bytes) plus the oracle's linear codes for the reference."""
    xb = synth.bf16_bits(xt)
    x = xt.to(dev)
    if had:
        c, s = B.fp4_hadamard32_quantize(x, mask, axis=axis, round=B.SR if sr else B.RNE, seed=synth.SR_SEED,
                                         stream_id=stream, layout=B.LAYOUT_TILED)
        oc, os_ = oracle.hadamard32_quantize(xb, mask, axis=axis, sr=sr, seed=synth.SR_SEED, stream=stream)
    else:
        c, s = B.fp4_quantize_mx(x, axis=axis, round=B.SR if sr else B.RNE, seed=synth.SR_SEED, stream_id=stream,
                                 layout=B.LAYOUT_TILED)
        oc, os_ = oracle.quantize_mx(xb, axis=axis, sr=sr, seed=synth.SR_SEED, stream=stream)
    torch.cuda.synchronize()
    tc, ts = oracle.tile_mx(oc, os_)
    assert_bytes_equal(np_u8(c), tc, "tiled operand codes")
    assert_bytes_equal(np_u8(s), ts, "tiled operand scales")
    return c, s, oc, os_


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (33, 257, 384), (300, 200, 256), (256, 512, 1024),
                                   (511, 129, 128), (640, 384, 2048), (4096, 256, 512)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_mx_tiled_ragged(M, N, K, out):
    dev = device()
    announce(f"gemm mx tiled {M}x{N}x{K} {out}")
    a, sa, oa, osa = mx_operand_tiled(synth.activation(M, K, 60), dev)
    b, sb, ob, osb = mx_operand_tiled(synth.weight(N, K, 61), dev)
    c = B.fp4_gemm_mx(a, sa, b, sb, alpha=0.75, layout=B.LAYOUT_TILED, m=M, n=N)
    torch.cuda.synchronize()
    cref, w = oracle.gemm_ref(oracle.dequant_mx(oa, osa), oracle.dequant_mx(ob, osb), 0.75)
    gemm_check(c.cpu().numpy(), cref, w, f"tiled {M}x{N}x{K}")
    if out == "bf16":
        c16 = B.fp4_gemm_mx(a, sa, b, sb, alpha=0.75, layout=B.LAYOUT_TILED, m=M, n=N, out_dtype=torch.bfloat16)
        # odd ldc: the epilogue's element path
        big = torch.zeros((M, N + 3), dtype=torch.bfloat16, device=dev)
        B.fp4_gemm_mx(a, sa, b, sb, alpha=0.75, layout=B.LAYOUT_TILED, m=M, n=N, c=big[:, :N])
        torch.cuda.synchronize()
        want16 = sf.f32_to_bf16_bits_rne(c.cpu().numpy())
        assert np.array_equal(c16.view(torch.int16).cpu().numpy().view(np.uint16), want16)
        assert np.array_equal(big[:, :N].contiguous().view(torch.int16).cpu().numpy().view(np.uint16), want16)
        assert torch.all(big[:, N:] == 0)


TILED_FULL_GEMMS = [
    ("qkv", ("qkv", "X", "rows", False, False, 0), ("qkv", "W", "rows", False, False, 0), 1.0),
    ("mlp_gate_up", ("mlp_gate_up", "X", "rows", False, False, 0), ("mlp_gate_up", "W", "rows", False, False, 0), 1.0),
    ("mlp_down", ("mlp_down", "H", "rows", False, False, 0), ("mlp_down", "W", "rows", False, False, 0), 1.0),
    ("dgrad", ("backward", "dY", "rows", True, False, 0), ("backward", "W", "cols", False, False, 1), 1.0),
    ("wgrad", ("backward", "dY", "cols", True, True, 1), ("backward", "X", "cols", False, True, 1), 1.0 / 32),
]


@pytest.mark.parametrize("name,aspec,bspec,alpha", TILED_FULL_GEMMS, ids=[g[0] for g in TILED_FULL_GEMMS])
def test_mx_tiled_full_size(name, aspec, bspec, alpha):
    # the tiled instantiation the benchmark runs, every output element of
    # every configuration's GEMM against the fp64 oracle (fp32 output; the
    # bf16 output equals its round to nearest even)
    dev = device()
    announce(f"gemm mx tiled full {name}")
    mask = synth.sign_mask(synth.HADAMARD_MASK_SEED)

    def operand(spec):
        cfg, role, axis, sr, had, stream = spec
        return mx_operand_tiled(synth.config_tensor(cfg, role), dev,
                                axis=B.ALONG_ROWS if axis == "rows" else B.ALONG_COLS, sr=sr, had=had, mask=mask,
                                stream=stream)

    a, sa, oa, osa = operand(aspec)
    b, sb, ob, osb = operand(bspec)
    M, N = oa.shape[0], ob.shape[0]
    c = B.fp4_gemm_mx(a, sa, b, sb, alpha=alpha, layout=B.LAYOUT_TILED, m=M, n=N)
    c16 = B.fp4_gemm_mx(a, sa, b, sb, alpha=alpha, layout=B.LAYOUT_TILED, m=M, n=N, out_dtype=torch.bfloat16)
    cref, w = oracle.gemm_ref(oracle.dequant_mx(oa, osa), oracle.dequant_mx(ob, osb), alpha)
    torch.cuda.synchronize()
    cg = c.cpu().numpy()
    worst = gemm_check(cg, cref, w, name)
    assert np.array_equal(c16.view(torch.int16).cpu().numpy().view(np.uint16), sf.f32_to_bf16_bits_rne(cg)), \
        "bf16 output != RNE of fp32 output"
    print(f"tiled {name}: worst |err| / sum|ab| = {worst:.3e}")
