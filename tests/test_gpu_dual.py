"""GPU parity of the dual-output MX producer (fp4_quantize_mx_dual): from one
read of x it writes x along rows and x^T along columns (optionally with the
fixed-sign Hadamard); each output must equal the CPU oracle's separate
producer output byte for byte, in both layouts, for every rounding
combination, on ragged shapes and at the backward-pass operand size."""
import numpy as np
import pytest
import torch

from tests.gpu_common import B, announce, assert_bytes_equal, device, np_u8, oracle, synth, to_dev

pytestmark = pytest.mark.gpu


def expected(xb, round_rows, had, round_cols, mask, seed, s_rows, s_cols):
    rc, rs = oracle.quantize_mx(xb, sr=round_rows, seed=seed, stream=s_rows)
    if had:
        cc, cs = oracle.hadamard32_quantize(xb, mask, axis=oracle.AXIS_COLS, sr=round_cols, seed=seed, stream=s_cols)
    else:
        cc, cs = oracle.quantize_mx(xb, axis=oracle.AXIS_COLS, sr=round_cols, seed=seed, stream=s_cols)
    return rc, rs, cc, cs


def run_dual(x, round_rows, had, round_cols, mask, seed, s_rows, s_cols, layout):
    out = B.fp4_quantize_mx_dual(x, round_rows=B.SR if round_rows else B.RNE, stream_id_rows=s_rows,
                                 hadamard_cols=had, sign_mask=mask, round_cols=B.SR if round_cols else B.RNE,
                                 stream_id_cols=s_cols, seed=seed, layout=layout)
    torch.cuda.synchronize()
    return [np_u8(t) for t in out]


DUAL_LINEAR = [(32, 32, None), (64, 96, 104), (96, 160, None), (160, 288, 296), (256, 256, None)]
ROUNDS = [(False, False, False), (False, True, False), (True, False, True), (True, True, True), (False, False, True)]


@pytest.mark.parametrize("rows,cols,ld", DUAL_LINEAR)
@pytest.mark.parametrize("round_rows,round_cols,had", ROUNDS)
def test_dual_linear_small(rows, cols, ld, round_rows, round_cols, had):
    dev = device()
    announce(f"dual linear {rows}x{cols} ld={ld} sr_rows={round_rows} sr_cols={round_cols} hadamard={had}")
    xb = synth.bf16_bits(synth.grad_student_t3(rows, cols, 60))
    x = to_dev(synth.from_bf16_bits(xb), dev, ld)
    mask = synth.sign_mask(7)
    got = run_dual(x, round_rows, had, round_cols, mask, 11, 2, 5, B.LAYOUT_LINEAR)
    want = expected(xb, round_rows, had, round_cols, mask, 11, 2, 5)
    for g, w, name in zip(got, want, ("row codes", "row scales", "column codes", "column scales")):
        assert_bytes_equal(g, w, name)


DUAL_TILED = [(128, 128), (256, 384), (384, 256)]


@pytest.mark.parametrize("rows,cols", DUAL_TILED)
@pytest.mark.parametrize("round_rows,round_cols,had", ROUNDS[:4])
def test_dual_tiled_small(rows, cols, round_rows, round_cols, had):
    dev = device()
    announce(f"dual tiled {rows}x{cols} sr_rows={round_rows} sr_cols={round_cols} hadamard={had}")
    xb = synth.bf16_bits(synth.activation(rows, cols, 61))
    x = synth.from_bf16_bits(xb).to(dev)
    mask = synth.sign_mask(7)
    got = run_dual(x, round_rows, had, round_cols, mask, 13, 0, 1, B.LAYOUT_TILED)
    rc, rs, cc, cs = expected(xb, round_rows, had, round_cols, mask, 13, 0, 1)
    trc, trs = oracle.tile_mx(rc, rs)
    tcc, tcs = oracle.tile_mx(cc, cs)
    for g, w, name in zip(got, (trc, trs, tcc, tcs), ("row codes", "row scales", "column codes", "column scales")):
        assert_bytes_equal(g, w, name)


def test_dual_equals_separate_calls_and_writes_every_byte():
    # poisoned outputs, then byte equality with the two single-output producers on the GPU
    dev = device()
    announce("dual vs separate producers, poisoned outputs")
    rows, cols = 640, 384
    xb = synth.bf16_bits(synth.grad_student_t3(rows, cols, 62))
    x = synth.from_bf16_bits(xb).to(dev)
    mask = synth.sign_mask(9)
    for layout in (B.LAYOUT_LINEAR, B.LAYOUT_TILED):
        (rcs, rss) = B.mx_output_shapes(rows, cols, layout)
        (ccs, css) = B.mx_output_shapes(cols, rows, layout)
        bufs = [torch.full(s, 0xA5, dtype=torch.uint8, device=dev) for s in (rcs, rss, ccs, css)]
        B.fp4_quantize_mx_dual(x, round_rows=B.SR, stream_id_rows=4, hadamard_cols=True, sign_mask=mask,
                               round_cols=B.SR, stream_id_cols=6, seed=21, layout=layout, codes_rows=bufs[0],
                               scales_rows=bufs[1], codes_cols=bufs[2], scales_cols=bufs[3])
        r = B.fp4_quantize_mx(x, round=B.SR, seed=21, stream_id=4, layout=layout)
        c = B.fp4_hadamard32_quantize(x, mask, axis=B.ALONG_COLS, round=B.SR, seed=21, stream_id=6, layout=layout)
        torch.cuda.synchronize()
        for g, w, name in zip(bufs, (*r, *c), ("row codes", "row scales", "column codes", "column scales")):
            assert_bytes_equal(np_u8(g), np_u8(w), f"layout {layout} {name}")


# the backward pass's dY (SR along rows for dgrad; Hadamard + SR along tokens
# for wgrad) and the forward X (RNE rows; Hadamard RNE columns kept for wgrad)
DUAL_FULL = [("backward", "dY", True, True), ("qkv", "X", False, False)]


@pytest.mark.parametrize("cfg,role,round_rows,round_cols", DUAL_FULL)
def test_dual_full_size(cfg, role, round_rows, round_cols):
    dev = device()
    announce(f"dual full {cfg}.{role} sr_rows={round_rows} sr_cols={round_cols} tiled")
    xt = synth.config_tensor(cfg, role)
    xb = synth.bf16_bits(xt)
    mask = synth.sign_mask(synth.HADAMARD_MASK_SEED)
    got = run_dual(xt.to(dev), round_rows, True, round_cols, mask, synth.SR_SEED, 0, 1, B.LAYOUT_TILED)
    rc, rs, cc, cs = expected(xb, round_rows, True, round_cols, mask, synth.SR_SEED, 0, 1)
    trc, trs = oracle.tile_mx(rc, rs)
    tcc, tcs = oracle.tile_mx(cc, cs)
    for g, w, name in zip(got, (trc, trs, tcc, tcs), ("row codes", "row scales", "column codes", "column scales")):
        assert_bytes_equal(g, w, name)
