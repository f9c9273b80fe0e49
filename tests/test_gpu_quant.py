"""GPU parity of the quantization producers against the CPU oracle: codes,
scale bytes and FP32 tensor scales must be identical byte for byte, for RNE
and for stochastic rounding at a fixed seed, on small ragged shapes and on the
full Llama-3-8B operand sizes the benchmark uses."""
import numpy as np
import pytest
import torch

from tests.gpu_common import B, announce, assert_bytes_equal, device, np_u8, oracle, synth, to_dev

pytestmark = pytest.mark.gpu


def special_values(rows, cols, seed):
    """bf16 with zeros blocks, subnormals, exact ties after scaling, huge values."""
    rng = np.random.default_rng(seed)
    x = synth.bf16_bits(synth.activation(rows, cols, seed)).copy()
    flat = x.reshape(-1)
    n = flat.size
    picks = rng.integers(0, n, n // 4)
    specials = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x3E80, 0x3F40, 0x3FA0, 0x3FE0, 0x4020, 0x4060,
                         0x40A0, 0x40C0, 0x40E0, 0x7F7F, 0xFF7F, 0x0080, 0xBE80], dtype=np.uint16)
    flat[picks] = specials[rng.integers(0, specials.size, picks.size)]
    if cols >= 64 and rows >= 2:
        x[1, :32] = 0          # an all-zero block
        x[0, 32:64] = 0x0001   # a subnormal-only block
    return x


MX_SHAPES = [(1, 32, None), (3, 64, None), (37, 96, None), (256, 256, None), (50, 96, 136), (129, 4096, None)]


@pytest.mark.parametrize("rows,cols,ld", MX_SHAPES)
@pytest.mark.parametrize("sr", [False, True])
@pytest.mark.parametrize("dist", ["act", "special"])
def test_mx_rows_small(rows, cols, ld, sr, dist):
    dev = device()
    announce(f"mx rows {rows}x{cols} ld={ld} sr={sr} {dist}")
    xb = synth.bf16_bits(synth.activation(rows, cols, 3)) if dist == "act" else special_values(rows, cols, 4)
    x = to_dev(synth.from_bf16_bits(xb), dev, ld)
    codes, scales = B.fp4_quantize_mx(x, round=B.SR if sr else B.RNE, seed=7, stream_id=3)
    torch.cuda.synchronize()
    oc, os_ = oracle.quantize_mx(xb, sr=sr, seed=7, stream=3)
    assert_bytes_equal(np_u8(scales), os_, "scales")
    assert_bytes_equal(np_u8(codes), oc, "codes")


COL_SHAPES = [(32, 4, 8), (64, 40, None), (96, 260, 264), (256, 256, 264), (128, 1028, 1032)]


@pytest.mark.parametrize("rows,cols,ld", COL_SHAPES)
@pytest.mark.parametrize("sr", [False, True])
@pytest.mark.parametrize("had", [False, True])
def test_mx_cols_small(rows, cols, ld, sr, had):
    dev = device()
    announce(f"mx cols {rows}x{cols} ld={ld} sr={sr} hadamard={had}")
    xb = special_values(rows, cols, 5) if not had else synth.bf16_bits(synth.grad_student_t3(rows, cols, 6))
    x = to_dev(synth.from_bf16_bits(xb), dev, ld)
    mask = synth.sign_mask(7)
    rnd = B.SR if sr else B.RNE
    if had:
        codes, scales = B.fp4_hadamard32_quantize(x, mask, axis=B.ALONG_COLS, round=rnd, seed=7, stream_id=1)
        oc, os_ = oracle.hadamard32_quantize(xb, mask, axis=oracle.AXIS_COLS, sr=sr, seed=7, stream=1)
    else:
        codes, scales = B.fp4_quantize_mx(x, axis=B.ALONG_COLS, round=rnd, seed=7, stream_id=1)
        oc, os_ = oracle.quantize_mx(xb, axis=oracle.AXIS_COLS, sr=sr, seed=7, stream=1)
    torch.cuda.synchronize()
    assert_bytes_equal(np_u8(scales), os_, "scales")
    assert_bytes_equal(np_u8(codes), oc, "codes")


@pytest.mark.parametrize("rows,cols", [(1, 32), (5, 64), (64, 512)])
@pytest.mark.parametrize("sr", [False, True])
def test_hadamard_rows_small(rows, cols, sr):
    dev = device()
    announce(f"hadamard rows {rows}x{cols} sr={sr}")
    xb = synth.bf16_bits(synth.grad_student_t3(rows, cols, 8))
    for mask in (0, 0xFFFFFFFF, synth.sign_mask(7)):
        codes, scales = B.fp4_hadamard32_quantize(synth.from_bf16_bits(xb).to(dev), mask, axis=B.ALONG_ROWS,
                                                  round=B.SR if sr else B.RNE, seed=9, stream_id=0)
        torch.cuda.synchronize()
        oc, os_ = oracle.hadamard32_quantize(xb, mask, axis=oracle.AXIS_ROWS, sr=sr, seed=9, stream=0)
        assert_bytes_equal(np_u8(scales), os_, f"scales mask={mask:#x}")
        assert_bytes_equal(np_u8(codes), oc, f"codes mask={mask:#x}")


# cols: one tile; two, the second partial; three (an odd tile count); K % 64
# == 0 with a partial last tile (word-sized scale stores)
NV_SHAPES = [(1, 16, None), (3, 48, None), (130, 144, None), (300, 400, 416), (256, 256, None), (70, 384, None),
             (129, 192, None)]


@pytest.mark.parametrize("rows,cols,ld", NV_SHAPES)
@pytest.mark.parametrize("domain", [0, 1])
@pytest.mark.parametrize("sr", [False, True])
def test_nv_small(rows, cols, ld, domain, sr):
    dev = device()
    announce(f"nv {rows}x{cols} ld={ld} domain={domain} sr={sr}")
    xb = synth.bf16_bits(synth.activation(rows, cols, 10))
    x = to_dev(synth.from_bf16_bits(xb), dev, ld)
    codes, scales, ts = B.fp4_quantize_nv(x, domain, round=B.SR if sr else B.RNE, seed=7, stream_id=2)
    torch.cuda.synchronize()
    oc, os_, ots = oracle.quantize_nv(xb, sr=sr, seed=7, stream=2, domain=domain)
    assert_bytes_equal(ts.cpu().numpy().view(np.uint32), ots.view(np.uint32), "tensor scales")
    assert_bytes_equal(np_u8(scales), os_, "block scales")
    assert_bytes_equal(np_u8(codes), oc, "codes")


@pytest.mark.parametrize("domain", [0, 1])
def test_nv_scales_not_word_aligned(domain):
    # scale bytes at an odd address: written byte by byte, same bytes
    dev = device()
    announce(f"nv scales at an odd address, domain={domain}")
    rows, cols = 200, 512
    xb = synth.bf16_bits(synth.activation(rows, cols, 13))
    big = torch.full((rows * cols // 16 + 2,), 0xA5, dtype=torch.uint8, device=dev)
    sc = big[1:1 + rows * cols // 16].view(rows, cols // 16)
    codes, scales, ts = B.fp4_quantize_nv(synth.from_bf16_bits(xb).to(dev), domain, scales=sc)
    torch.cuda.synchronize()
    oc, os_, ots = oracle.quantize_nv(xb, domain=domain)
    assert_bytes_equal(np_u8(sc), os_, "block scales")
    assert_bytes_equal(np_u8(codes), oc, "codes")
    assert int(big[0].item()) == 0xA5 and int(big[-1].item()) == 0xA5


def test_nv_zero_tile_and_empty():
    dev = device()
    announce("nv zero tile / empty operand")
    xb = synth.bf16_bits(synth.activation(256, 256, 11)).copy()
    xb[:128, 128:] = 0
    for domain in (0, 1):
        codes, scales, ts = B.fp4_quantize_nv(synth.from_bf16_bits(xb).to(dev), domain)
        torch.cuda.synchronize()
        oc, os_, ots = oracle.quantize_nv(xb, domain=domain)
        assert_bytes_equal(ts.cpu().numpy().view(np.uint32), ots.view(np.uint32), "tensor scales")
        assert_bytes_equal(np_u8(scales), os_, "block scales")
        assert_bytes_equal(np_u8(codes), oc, "codes")
    # an empty operand still gets its global tensor scale (1.0)
    empty = torch.zeros((0, 64), dtype=torch.bfloat16, device=dev)
    _, _, ts = B.fp4_quantize_nv(empty, B.NV_GLOBAL)
    torch.cuda.synchronize()
    assert ts.item() == 1.0


def test_outputs_written_exactly_guard_bytes():
    # poison the outputs and a 4 KiB tail: every logical byte is overwritten, the tail is untouched
    dev = device()
    announce("guard bytes")
    rows, cols = 40, 96
    xb = synth.bf16_bits(synth.activation(rows, cols, 12))
    x = synth.from_bf16_bits(xb).to(dev)
    nbytes_c, nbytes_s = rows * cols // 2, rows * cols // 32
    cbuf = torch.full((nbytes_c + 4096,), 0xA5, dtype=torch.uint8, device=dev)
    sbuf = torch.full((nbytes_s + 4096,), 0xA5, dtype=torch.uint8, device=dev)
    codes = cbuf[:nbytes_c].view(rows, cols // 2)
    scales = sbuf[:nbytes_s].view(rows, cols // 32)
    B.fp4_quantize_mx(x, codes=codes, scales=scales)
    torch.cuda.synchronize()
    oc, os_ = oracle.quantize_mx(xb)
    assert_bytes_equal(np_u8(codes), oc, "codes")
    assert_bytes_equal(np_u8(scales), os_, "scales")
    assert np.all(np_u8(cbuf[nbytes_c:]) == 0xA5) and np.all(np_u8(sbuf[nbytes_s:]) == 0xA5)


def tiny_and_wide_blocks(rows, cols, seed):
    """bf16 [rows x cols]: every 32-element block holds one value of magnitude
    2^e (e in -100, 0, 60, 126; random sign) and 31 random bf16 patterns no
    larger than it, so that after the block scale y spans zero, subnormal and
    tiny binary32, full mantissas and exact grid points."""
    rng = np.random.default_rng(seed)
    nb = rows * cols // 32
    e = rng.choice(np.array([-100, 0, 60, 126]), nb)
    top = ((e + 127) << 7).astype(np.uint16)
    body = rng.integers(0, 0x8000, (nb, 31)).astype(np.uint32)
    body = np.minimum(body, top[:, None].astype(np.uint32)).astype(np.uint16)
    blk = np.concatenate([top[:, None], body], axis=1)
    blk |= (rng.integers(0, 2, blk.shape) << 15).astype(np.uint16)
    rot = rng.integers(0, 32, nb)  # the large value anywhere in the block
    idx = (np.arange(32)[None, :] + rot[:, None]) % 32
    blk = np.take_along_axis(blk, idx, axis=1)
    return blk.reshape(rows, cols)


@pytest.mark.parametrize("axis", ["rows", "cols"])
def test_sr_tiny_and_wide_blocks(axis):
    # stochastic rounding where r16 = 0 meets tiny nonzero y (it must round
    # up) and y from zero to the saturation range: byte for byte
    dev = device()
    announce(f"SR tiny and wide blocks along {axis}")
    xb = tiny_and_wide_blocks(2048, 4096, 5)
    x = synth.from_bf16_bits(xb).to(dev)
    if axis == "rows":
        codes, scales = B.fp4_quantize_mx(x, round=B.SR, seed=11, stream_id=4)
        oc, os_ = oracle.quantize_mx(xb, sr=True, seed=11, stream=4)
    else:
        xt = x.t().contiguous()
        codes, scales = B.fp4_quantize_mx(xt, axis=B.ALONG_COLS, round=B.SR, seed=11, stream_id=4)
        oc, os_ = oracle.quantize_mx(xb, sr=True, seed=11, stream=4)
    torch.cuda.synchronize()
    assert_bytes_equal(np_u8(scales), os_, "scales")
    assert_bytes_equal(np_u8(codes), oc, "codes")


def test_repeat_is_deterministic():
    dev = device()
    announce("determinism")
    x = synth.grad_student_t3(512, 1024, 13).to(dev)
    a = B.fp4_quantize_mx(x, round=B.SR, seed=7)
    b = B.fp4_quantize_mx(x, round=B.SR, seed=7)
    c = B.fp4_hadamard32_quantize(x, 0x1234, round=B.SR, seed=7)
    d = B.fp4_hadamard32_quantize(x, 0x1234, round=B.SR, seed=7)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert torch.equal(c[0], d[0]) and torch.equal(c[1], d[1])


# ------------------------------------------------------------------ full sizes

FULL = [
    ("qkv", "X", "rows", False, False),
    ("qkv", "W", "rows", False, False),
    ("mlp_gate_up", "W", "rows", False, False),
    ("mlp_down", "H", "rows", False, False),
    ("mlp_down", "W", "rows", False, False),
    ("backward", "dY", "rows", True, False),      # dgrad A: SR along rows
    ("backward", "W", "cols", False, False),      # dgrad B: W^T, transpose-quantize
    ("backward", "dY", "cols", True, True),       # wgrad A: Hadamard + SR along tokens
    ("backward", "X", "cols", False, True),       # wgrad B: Hadamard along tokens
]


@pytest.mark.parametrize("cfg,role,axis,sr,had", FULL)
def test_mx_full_size(cfg, role, axis, sr, had):
    dev = device()
    announce(f"full {cfg}.{role} axis={axis} sr={sr} hadamard={had}")
    xt = synth.config_tensor(cfg, role)
    xb = synth.bf16_bits(xt)
    x = xt.to(dev)
    ax = B.ALONG_ROWS if axis == "rows" else B.ALONG_COLS
    stream = 0 if axis == "rows" else 1
    mask = synth.sign_mask(synth.HADAMARD_MASK_SEED)
    if had:
        codes, scales = B.fp4_hadamard32_quantize(x, mask, axis=ax, round=B.SR if sr else B.RNE,
                                                  seed=synth.SR_SEED, stream_id=stream)
        oc, os_ = oracle.hadamard32_quantize(xb, mask, axis=ax, sr=sr, seed=synth.SR_SEED, stream=stream)
    else:
        codes, scales = B.fp4_quantize_mx(x, axis=ax, round=B.SR if sr else B.RNE, seed=synth.SR_SEED,
                                          stream_id=stream)
        oc, os_ = oracle.quantize_mx(xb, axis=ax, sr=sr, seed=synth.SR_SEED, stream=stream)
    torch.cuda.synchronize()
    assert_bytes_equal(np_u8(scales), os_, "scales")
    assert_bytes_equal(np_u8(codes), oc, "codes")


@pytest.mark.parametrize("role", ["X", "W"])
@pytest.mark.parametrize("domain", [0, 1])
def test_nv_full_size(role, domain):
    dev = device()
    announce(f"full nvfp4.{role} domain={domain}")
    xt = synth.config_tensor("nvfp4", role)
    xb = synth.bf16_bits(xt)
    codes, scales, ts = B.fp4_quantize_nv(xt.to(dev), domain)
    torch.cuda.synchronize()
    oc, os_, ots = oracle.quantize_nv(xb, domain=domain)
    assert_bytes_equal(ts.cpu().numpy().view(np.uint32), ots.view(np.uint32), "tensor scales")
    assert_bytes_equal(np_u8(scales), os_, "block scales")
    assert_bytes_equal(np_u8(codes), oc, "codes")


# ------------------------------------------------------------------ tiled (consumer) layout

TILED_CASES = [
    # rows, cols, axis, sr, had
    (1, 128, "rows", False, False), (33, 384, "rows", False, False), (70, 640, "rows", True, False),
    (64, 1024, "rows", False, True), (96, 512, "rows", True, True), (300, 1152, "rows", False, False),
    (128, 36, "cols", False, False), (256, 100, "cols", True, False), (384, 64, "cols", False, True),
    (128, 260, "cols", True, True),
]


@pytest.mark.parametrize("rows,cols,axis,sr,had", TILED_CASES)
def test_mx_tiled_small(rows, cols, axis, sr, had):
    dev = device()
    announce(f"tiled {axis} {rows}x{cols} sr={sr} hadamard={had}")
    ld = (cols + 7) // 8 * 8
    xb = synth.bf16_bits(synth.grad_student_t3(rows, cols, 50) if had else synth.activation(rows, cols, 51))
    x = to_dev(synth.from_bf16_bits(xb), dev, ld)
    ax = B.ALONG_ROWS if axis == "rows" else B.ALONG_COLS
    mask = synth.sign_mask(7)
    rnd = B.SR if sr else B.RNE
    if had:
        codes, scales = B.fp4_hadamard32_quantize(x, mask, axis=ax, round=rnd, seed=7, stream_id=1, layout=B.LAYOUT_TILED)
        oc, os_ = oracle.hadamard32_quantize(xb, mask, axis=ax, sr=sr, seed=7, stream=1)
    else:
        codes, scales = B.fp4_quantize_mx(x, axis=ax, round=rnd, seed=7, stream_id=1, layout=B.LAYOUT_TILED)
        oc, os_ = oracle.quantize_mx(xb, axis=ax, sr=sr, seed=7, stream=1)
    torch.cuda.synchronize()
    tc, ts = oracle.tile_mx(oc, os_)
    assert_bytes_equal(np_u8(scales), ts, "tiled scales")
    assert_bytes_equal(np_u8(codes), tc, "tiled codes")


def test_tiled_padding_overwritten():
    # poisoned outputs: the producer writes every byte of the tiled buffers, padding rows included
    dev = device()
    announce("tiled padding poison")
    rows, cols = 45, 256
    xb = synth.bf16_bits(synth.activation(rows, cols, 52))
    (cs, ss) = B.mx_output_shapes(rows, cols, B.LAYOUT_TILED)
    codes = torch.full(cs, 0xA5, dtype=torch.uint8, device=dev)
    scales = torch.full(ss, 0xA5, dtype=torch.uint8, device=dev)
    B.fp4_quantize_mx(synth.from_bf16_bits(xb).to(dev), layout=B.LAYOUT_TILED, codes=codes, scales=scales)
    torch.cuda.synchronize()
    oc, os_ = oracle.quantize_mx(xb)
    tc, ts = oracle.tile_mx(oc, os_)
    assert_bytes_equal(np_u8(codes), tc, "codes")
    assert_bytes_equal(np_u8(scales), ts, "scales")


TILED_FULL = [
    ("qkv", "X", "rows", False, False),
    ("qkv", "W", "rows", False, False),
    ("mlp_down", "H", "rows", False, False),
    ("backward", "dY", "rows", True, False),
    ("backward", "W", "cols", False, False),
    ("backward", "dY", "cols", True, True),
    ("backward", "X", "cols", False, True),
]


@pytest.mark.parametrize("cfg,role,axis,sr,had", TILED_FULL)
def test_mx_tiled_full_size(cfg, role, axis, sr, had):
    dev = device()
    announce(f"tiled full {cfg}.{role} axis={axis} sr={sr} hadamard={had}")
    xt = synth.config_tensor(cfg, role)
    xb = synth.bf16_bits(xt)
    ax = B.ALONG_ROWS if axis == "rows" else B.ALONG_COLS
    stream = 0 if axis == "rows" else 1
    mask = synth.sign_mask(synth.HADAMARD_MASK_SEED)
    rnd = B.SR if sr else B.RNE
    if had:
        codes, scales = B.fp4_hadamard32_quantize(xt.to(dev), mask, axis=ax, round=rnd, seed=synth.SR_SEED,
                                                  stream_id=stream, layout=B.LAYOUT_TILED)
        oc, os_ = oracle.hadamard32_quantize(xb, mask, axis=ax, sr=sr, seed=synth.SR_SEED, stream=stream)
    else:
        codes, scales = B.fp4_quantize_mx(xt.to(dev), axis=ax, round=rnd, seed=synth.SR_SEED, stream_id=stream,
                                          layout=B.LAYOUT_TILED)
        oc, os_ = oracle.quantize_mx(xb, axis=ax, sr=sr, seed=synth.SR_SEED, stream=stream)
    torch.cuda.synchronize()
    tc, ts = oracle.tile_mx(oc, os_)
    assert_bytes_equal(np_u8(scales), ts, "tiled scales")
    assert_bytes_equal(np_u8(codes), tc, "tiled codes")
