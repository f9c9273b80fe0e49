"""Pins of the oracle's NVFP4 quantizer: global and per-128x128-tile tensor
scales, E4M3 block scales with the clamp, RNE and SR.  CPU only."""
import numpy as np
import pytest

import oracle
from fp4_block_scaled_quantizer_amd import synth
from tests import golden_io
from tests import second_formulation as sf


def test_nv_worked_example_global_and_tile():
    g = golden_io.load("nv_worked_examples.txt")
    x = golden_io.bf16_row(g["nv_x"])
    for dom in (oracle.NV_GLOBAL, oracle.NV_TILE128):
        codes, scales, ts = oracle.quantize_nv(x, domain=dom)
        assert ts.ravel().view(np.uint32).tolist() == g["nv_tensor_scale_f32"]
        assert scales.ravel().tolist() == g["nv_scales"]
        assert codes.ravel().tolist() == g["nv_codes"]


@pytest.mark.parametrize("case", ["order1", "order2"])
def test_nv_operation_order_golden(case):
    # hand-derived cases whose bytes depend on the order of the binary32
    # operations: (b / 6) / S for the block scale (case 1) and x * (1 / d)
    # for the elements (case 2)
    g = golden_io.load("nv_op_order.txt")
    x = golden_io.bf16_row(g[f"{case}_x"])
    for dom in (oracle.NV_GLOBAL, oracle.NV_TILE128):
        codes, scales, ts = oracle.quantize_nv(x, domain=dom)
        assert ts.ravel().view(np.uint32).tolist() == g[f"{case}_tensor_scale_f32"]
        assert scales.ravel().tolist() == g[f"{case}_scales"]
        assert codes.ravel().tolist() == g[f"{case}_codes"]


def test_nv_operation_order_cases_discriminate():
    # the other orders, in binary32, change a byte of the golden cases: so
    # an oracle (or kernel) using them fails the test above
    f32 = np.float32
    S = f32(976) / f32(2688)
    assert oracle.e4m3_rne_satfinite(float((f32(22.875) / f32(6)) / S)) == 0x52
    assert oracle.e4m3_rne_satfinite(float(f32(22.875) / (f32(6) * S))) == 0x53
    d = f32(1.875)
    assert oracle.e2m1_rne(float(f32(2.34375) * (f32(1) / d))) == 3
    assert oracle.e2m1_rne(float(f32(2.34375) / d)) == 2


def test_nv_tensor_scale_and_block_scale_closed_forms():
    assert oracle.nv_tensor_scale(0.0) == 1.0
    assert oracle.nv_tensor_scale(2688.0) == 1.0
    assert oracle.nv_tensor_scale(5376.0) == 2.0
    # the block holding the domain amax gets the largest E4M3 scale
    for A in (1e-3, 0.37, 6.0, 97.0, 3e4):
        S = oracle.nv_tensor_scale(A)
        assert oracle.nv_block_scale(float(np.float32(A)), S) == 0x7E
    # clamp: a zero block (or one far below the domain amax) gets 0x01, never 0
    assert oracle.nv_block_scale(0.0, 1.0) == 0x01
    assert oracle.nv_block_scale(1e-6, 1.0) == 0x01


def test_nv_dequant_error_bound_and_max_block():
    x = synth.bf16_bits(synth.activation(130, 160, 21))
    xf = sf.bf16_to_f32(x).astype(np.float64)
    for dom in (oracle.NV_GLOBAL, oracle.NV_TILE128):
        codes, scales, ts = oracle.quantize_nv(x, domain=dom)
        dq = oracle.dequant_nv(codes, scales, ts, dom)
        R, K = x.shape
        TK = (K + 127) // 128
        for r in range(R):
            for j in range(K // 16):
                S = ts.ravel()[0] if dom == 0 else ts[r // 128, (16 * j) // 128]
                d = float(np.float32(oracle.e4m3_value(int(scales[r, j]))) * np.float32(S))
                blk = xf[r, 16 * j:16 * j + 16]
                e = np.abs(dq[r, 16 * j:16 * j + 16] - blk)
                # half the local E2M1 gap (at most 1 below 4, 2 in [4, 6]) times d,
                # plus a relative hair for the binary32 reciprocal; saturated elements excluded
                y = np.abs(blk) / d
                ok = y <= 6.0
                gap = np.where(y < 2, 0.5, np.where(y < 4, 1.0, 2.0))
                assert np.all(e[ok] <= (gap[ok] / 2) * d * (1 + 1e-6) + 1e-30)
        # per domain, the block holding the amax gets 0x7E
        if dom == oracle.NV_GLOBAL:
            r, k = np.unravel_index(np.argmax(np.abs(xf)), xf.shape)
            assert scales[r, k // 16] == 0x7E
        del TK


def test_nv_tile_shape_zero_tile_and_isolation():
    x = synth.bf16_bits(synth.activation(256, 384, 22))
    x[:128, 128:256] = 0  # an all-zero tile
    codes, scales, ts = oracle.quantize_nv(x, domain=oracle.NV_TILE128)
    assert ts.shape == (2, 3)
    assert ts[0, 1] == 1.0
    assert np.all(scales[:128, 8:16] == 0x01)
    assert np.all((codes[:128, 64:128] & 0x77) == 0)
    # an x50 outlier in one tile does not change its neighbours' tensor scales
    y = x.copy()
    y[200, 300] = 0x4800  # 131072.0
    _, _, ts2 = oracle.quantize_nv(y, domain=oracle.NV_TILE128)
    changed = ts2 != ts
    assert changed[1, 2] and changed.sum() == 1


def test_nv_power_of_two_invariance():
    x = synth.bf16_bits(synth.activation(128, 128, 23))
    for dom in (oracle.NV_GLOBAL, oracle.NV_TILE128):
        c, s, ts = oracle.quantize_nv(x, domain=dom)
        for t in (-7, 3):
            xt = sf.f32_to_bf16_bits_rne(sf.bf16_to_f32(x) * np.float32(2.0 ** t)).reshape(x.shape)
            ct, st, tst = oracle.quantize_nv(xt, domain=dom)
            assert np.array_equal(ct, c) and np.array_equal(st, s)
            assert np.array_equal(tst, (ts * np.float32(2.0 ** t)).astype(np.float32))


def test_nv_edge_tiles_are_their_own_domains():
    x = synth.bf16_bits(synth.activation(130, 144, 24))
    codes, scales, ts = oracle.quantize_nv(x, domain=oracle.NV_TILE128)
    assert ts.shape == (2, 2)
    xf = np.abs(sf.bf16_to_f32(x))
    assert ts[1, 1] == oracle.nv_tensor_scale(float(xf[128:, 128:].max()))
    assert ts[0, 1] == oracle.nv_tensor_scale(float(xf[:128, 128:].max()))


def test_nv_sr_and_axis():
    x = synth.bf16_bits(synth.grad_student_t3(64, 32, 25))
    c_cols, s_cols, t_cols = oracle.quantize_nv(x, axis=oracle.AXIS_COLS, sr=True, seed=7, stream=2,
                                                domain=oracle.NV_TILE128)
    c_rows, s_rows, t_rows = oracle.quantize_nv(np.ascontiguousarray(x.T), sr=True, seed=7, stream=2,
                                                domain=oracle.NV_TILE128)
    assert np.array_equal(c_cols, c_rows) and np.array_equal(s_cols, s_rows) and np.array_equal(t_cols, t_rows)
    c_rne, s_rne, _ = oracle.quantize_nv(x, axis=oracle.AXIS_COLS, domain=oracle.NV_TILE128)
    assert np.array_equal(s_rne, s_cols)  # SR changes codes only
    assert not np.array_equal(c_rne, c_cols)


def test_nv_rejects_out_of_contract():
    x = np.zeros((1, 16), dtype=np.uint16)
    x[0, 0] = 0x0001  # domain amax 2^-133 < 2^-100
    with pytest.raises(oracle.OracleInputError):
        oracle.quantize_nv(x)
    with pytest.raises(oracle.OracleInputError):
        oracle.quantize_nv(np.zeros((1, 24), dtype=np.uint16))


def _small_int_bf16(rows, cols, seed):
    """bf16 bits of integers in [-3, 3]: every Hadamard-32 output is an
    integer of magnitude <= 96, exact in bf16."""
    rng = np.random.default_rng(seed)
    v = rng.integers(-3, 4, size=(rows, cols)).astype(np.float32)
    return sf.f32_to_bf16_bits_rne(v)


@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("domain", [0, 1])
@pytest.mark.parametrize("sr", [False, True])
def test_hadamard_nv_equals_explicit_transform_then_nv(axis, domain, sr):
    # the transform through the explicit Sylvester matrix (float64, exact on
    # these inputs), the result as bf16 rows of the logical operand, then the
    # plain NVFP4 oracle: same codes, block scales and tensor scales
    rows, cols = (160, 96) if axis == 0 else (96, 160)
    x = _small_int_bf16(rows, cols, 30 + axis)
    mask = synth.sign_mask(11)
    codes, scales, ts = oracle.hadamard32_quantize_nv(x, mask, axis=axis, sr=sr, seed=5, stream=3, domain=domain)
    logical = sf.bf16_to_f32(x if axis == 0 else np.ascontiguousarray(x.T)).astype(np.float64)
    H = sf.sylvester_hadamard(32).astype(np.float64)
    d = np.array([-1.0 if (mask >> i) & 1 else 1.0 for i in range(32)])
    R, K = logical.shape
    blocks = logical.reshape(R, K // 32, 32) * d
    t = np.einsum("ij,rbj->rbi", H, blocks).reshape(R, K)
    assert np.array_equal(t, np.round(t)) and np.abs(t).max() <= 256
    tb = sf.f32_to_bf16_bits_rne(t.astype(np.float32))
    c2, s2, t2 = oracle.quantize_nv(tb, sr=sr, seed=5, stream=3, domain=domain)
    assert np.array_equal(codes, c2) and np.array_equal(scales, s2)
    assert np.array_equal(ts.view(np.uint32), t2.view(np.uint32))


def test_hadamard_nv_mask_flip_negates_and_needs_k32():
    x = synth.bf16_bits(synth.grad_student_t3(64, 96, 33))
    for domain in (0, 1):
        c0, s0, t0 = oracle.hadamard32_quantize_nv(x, 0, axis=oracle.AXIS_COLS, domain=domain)
        c1, s1, t1 = oracle.hadamard32_quantize_nv(x, 0xFFFFFFFF, axis=oracle.AXIS_COLS, domain=domain)
        assert np.array_equal(s0, s1) and np.array_equal(t0, t1)
        d0 = oracle.dequant_nv(c0, s0, t0, domain)
        d1 = oracle.dequant_nv(c1, s1, t1, domain)
        assert np.array_equal(d1, -d0)
    with pytest.raises(oracle.OracleInputError):
        oracle.hadamard32_quantize_nv(np.zeros((16, 48), dtype=np.uint16), 0, axis=oracle.AXIS_ROWS)
