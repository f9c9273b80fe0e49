"""GPU parity of NVFP4 along columns (the transpose a wgrad operand needs)
and of the fixed-sign Hadamard-32 ahead of NVFP4: codes, E4M3 block scales
and FP32 tensor scales identical to the CPU oracle byte for byte, both scale
domains, RNE and SR, on ragged shapes (K a multiple of 16 but not of 32,
column counts that are not multiples of the 128-wide tile) and at the
backward-pass operand sizes."""
import numpy as np
import pytest
import torch

from tests.gpu_common import B, announce, assert_bytes_equal, device, np_u8, oracle, synth, to_dev

pytestmark = pytest.mark.gpu


def check(got, want):
    (c, s, t), (oc, os_, ot) = got, want
    assert_bytes_equal(t.cpu().numpy().view(np.uint32), ot.view(np.uint32), "tensor scales")
    assert_bytes_equal(np_u8(s), os_, "block scales")
    assert_bytes_equal(np_u8(c), oc, "codes")


NV_COL_SHAPES = [(16, 4, 8), (48, 36, 40), (160, 260, 264), (256, 128, None), (400, 100, 104)]


@pytest.mark.parametrize("rows,cols,ld", NV_COL_SHAPES)
@pytest.mark.parametrize("domain", [0, 1])
@pytest.mark.parametrize("sr", [False, True])
def test_nv_cols_small(rows, cols, ld, domain, sr):
    dev = device()
    announce(f"nv cols {rows}x{cols} ld={ld} domain={domain} sr={sr}")
    xb = synth.bf16_bits(synth.grad_student_t3(rows, cols, 80))
    x = to_dev(synth.from_bf16_bits(xb), dev, ld)
    got = B.fp4_quantize_nv(x, domain, axis=B.ALONG_COLS, round=B.SR if sr else B.RNE, seed=9, stream_id=4)
    torch.cuda.synchronize()
    check(got, oracle.quantize_nv(xb, axis=oracle.AXIS_COLS, sr=sr, seed=9, stream=4, domain=domain))


HAD_COL_SHAPES = [(32, 4, 8), (64, 40, None), (160, 260, 264), (384, 128, None)]


@pytest.mark.parametrize("rows,cols,ld", HAD_COL_SHAPES)
@pytest.mark.parametrize("domain", [0, 1])
@pytest.mark.parametrize("sr", [False, True])
def test_hadamard_nv_cols_small(rows, cols, ld, domain, sr):
    dev = device()
    announce(f"hadamard nv cols {rows}x{cols} ld={ld} domain={domain} sr={sr}")
    xb = synth.bf16_bits(synth.grad_student_t3(rows, cols, 81))
    x = to_dev(synth.from_bf16_bits(xb), dev, ld)
    for mask in (0, synth.sign_mask(13)):
        got = B.fp4_quantize_nv(x, domain, axis=B.ALONG_COLS, round=B.SR if sr else B.RNE, seed=9, stream_id=4,
                                hadamard_mask=mask)
        torch.cuda.synchronize()
        check(got, oracle.hadamard32_quantize_nv(xb, mask, axis=oracle.AXIS_COLS, sr=sr, seed=9, stream=4,
                                                 domain=domain))


def test_nv_cols_empty_and_zero():
    dev = device()
    announce("nv cols empty / zero operands")
    for had in (None, 0x5A5A5A5A):
        ts = torch.full((1,), 7.0, dtype=torch.float32, device=dev)
        B.fp4_quantize_nv(torch.empty((0, 64), dtype=torch.bfloat16, device=dev), B.NV_GLOBAL, axis=B.ALONG_COLS,
                          tensor_scale=ts, hadamard_mask=had)
        torch.cuda.synchronize()
        assert float(ts.item()) == 1.0  # an empty global domain has S = 1
        x = torch.zeros((64, 128), dtype=torch.bfloat16, device=dev)
        for domain in (0, 1):
            got = B.fp4_quantize_nv(x, domain, axis=B.ALONG_COLS, hadamard_mask=had)
            torch.cuda.synchronize()
            xb = synth.bf16_bits(x.cpu())
            want = (oracle.quantize_nv(xb, axis=oracle.AXIS_COLS, domain=domain) if had is None else
                    oracle.hadamard32_quantize_nv(xb, had, axis=oracle.AXIS_COLS, domain=domain))
            check(got, want)


# the backward pass's wgrad operands in NVFP4: dY^T and X^T along tokens
# (Hadamard + SR and Hadamard + RNE), and W^T for dgrad (plain)
NV_COL_FULL = [("backward", "dY", True, True), ("backward", "X", True, False), ("backward", "W", False, False)]


@pytest.mark.parametrize("cfg,role,had,sr", NV_COL_FULL)
@pytest.mark.parametrize("domain", [0, 1])
def test_nv_cols_full_size(cfg, role, had, sr, domain):
    dev = device()
    announce(f"nv cols full {cfg}.{role} hadamard={had} sr={sr} domain={domain}")
    xt = synth.config_tensor(cfg, role)
    xb = synth.bf16_bits(xt)
    mask = synth.sign_mask(synth.HADAMARD_MASK_SEED)
    got = B.fp4_quantize_nv(xt.to(dev), domain, axis=B.ALONG_COLS, round=B.SR if sr else B.RNE, seed=synth.SR_SEED,
                            stream_id=1, hadamard_mask=mask if had else None)
    torch.cuda.synchronize()
    if had:
        want = oracle.hadamard32_quantize_nv(xb, mask, axis=oracle.AXIS_COLS, sr=sr, seed=synth.SR_SEED, stream=1,
                                             domain=domain)
    else:
        want = oracle.quantize_nv(xb, axis=oracle.AXIS_COLS, sr=sr, seed=synth.SR_SEED, stream=1, domain=domain)
    check(got, want)
