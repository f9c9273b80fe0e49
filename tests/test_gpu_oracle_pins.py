"""Exhaustive and hand-derived checks of the GPU producers against the oracle.

1. The RNE producers round with gfx950's scaled FP4 convert.  That it
   equals the oracle's E2M1 rule is checked here for every finite bf16 bit
   pattern at every shared exponent E it can meet: for each E in
   [-127, 125] (125: the largest finite bf16 has floor(log2) = 127), every
   pattern x with |x| < 2^(E+3) is placed in 32-element blocks whose first
   element 2^(E+2) fixes the block's shared exponent at E (|x| < 2^(E+3)
   keeps floor(log2 amax) = E + 2); E = -127 also takes every pattern below
   2^-124 (the clamp).  8.4 M elements, through the row producer (bf16
   convert), the column producer on the transposed input (binary32 convert)
   and the tiled row producer.
2. The NVFP4 op-order golden cases (tests/golden/nv_op_order.txt), whose
   bytes change under another order of the binary32 operations, on both
   domains along rows.
"""
import numpy as np
import pytest
import torch

from tests import golden_io
from tests.gpu_common import B, announce, assert_bytes_equal, device, np_u8, oracle, synth, untile_mx

pytestmark = pytest.mark.gpu

ROW = 4096  # elements per row of the sweep matrix: 128 blocks


def sweep_matrix():
    """bf16 bits [rows x 4096]: blocks of (anchor 2^(E+2), 31 patterns)."""
    blocks = []
    pos = np.arange(0x7F80, dtype=np.uint32)  # every finite non-negative bf16
    for E in range(-127, 126):
        lim = (E + 3 + 127) << 7  # bit pattern of 2^(E+3)
        below = pos[pos < lim] if E > -127 else pos[pos < ((-124 + 127) << 7)]
        pats = np.concatenate([below, below | 0x8000]).astype(np.uint16)
        anchor = np.uint16((E + 2 + 127) << 7)
        n = (pats.size + 30) // 31
        body = np.zeros(n * 31, dtype=np.uint16)
        body[:pats.size] = pats
        blk = np.empty((n, 32), dtype=np.uint16)
        blk[:, 0] = anchor
        blk[:, 1:] = body.reshape(n, 31)
        blocks.append(blk)
    allb = np.concatenate(blocks)
    per_row = ROW // 32
    rows = (allb.shape[0] + per_row - 1) // per_row
    rows = (rows + 127) // 128 * 128  # whole 128-row tiles (the transposed input's cols % 4 == 0)
    out = np.zeros((rows * per_row, 32), dtype=np.uint16)
    out[:allb.shape[0]] = allb
    return out.reshape(rows, ROW), allb.shape[0]


def test_rne_convert_every_bf16_at_every_exponent():
    dev = device()
    announce("RNE sweep: every bf16 x every shared exponent")
    xb, nblocks = sweep_matrix()
    want_c, want_s = oracle.quantize_mx(xb)
    # the block layout is what the sweep claims: one scale byte E + 127 per E
    assert set(np.unique(want_s.ravel()[:nblocks]).tolist()) == set(range(0, 253))
    x = synth.from_bf16_bits(xb).to(dev)
    rows, K = xb.shape
    c_rows, s_rows = B.fp4_quantize_mx(x)
    c_cols, s_cols = B.fp4_quantize_mx(x.t().contiguous(), axis=B.ALONG_COLS)
    c_t, s_t = B.fp4_quantize_mx(x, layout=B.LAYOUT_TILED)
    torch.cuda.synchronize()
    assert_bytes_equal(np_u8(s_rows), want_s, "scales (rows)")
    assert_bytes_equal(np_u8(c_rows), want_c, "codes (rows, bf16 convert)")
    assert_bytes_equal(np_u8(s_cols), want_s, "scales (cols)")
    assert_bytes_equal(np_u8(c_cols), want_c, "codes (cols, binary32 convert)")
    lc, ls, _, _ = untile_mx(np_u8(c_t), np_u8(s_t), rows, K)
    assert_bytes_equal(ls, want_s, "scales (tiled)")
    assert_bytes_equal(lc, want_c, "codes (tiled)")


@pytest.mark.parametrize("case", ["order1", "order2"])
@pytest.mark.parametrize("domain", [0, 1])
def test_nv_operation_order_golden(case, domain):
    dev = device()
    announce(f"nv op-order golden {case} domain={domain}")
    g = golden_io.load("nv_op_order.txt")
    x = synth.from_bf16_bits(golden_io.bf16_row(g[f"{case}_x"])).to(dev)
    c, s, ts = B.fp4_quantize_nv(x, domain)
    torch.cuda.synchronize()
    assert ts.cpu().numpy().ravel().view(np.uint32).tolist() == g[f"{case}_tensor_scale_f32"]
    assert np_u8(s).ravel().tolist() == g[f"{case}_scales"]
    assert np_u8(c).ravel().tolist() == g[f"{case}_codes"]
