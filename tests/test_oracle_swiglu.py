"""Pins of the oracle's SwiGLU, the activation whose bf16 output H the fused
GEMM epilogue quantizes: the binary32 exponential and SiLU against float64
mathematics, exact special cases and an identity, the interleaved gate/up
column layout against a direct construction, and the bf16 rounding against
torch's conversion.  CPU only."""
import math

import numpy as np
import pytest
import torch

import oracle

U24 = 2.0 ** -24  # half the binary32 spacing at 1


def test_exp_sequence_within_two_half_ulps():
    # dense grid over the whole domain [-20, 80] plus the reduced-argument
    # range: a wrong polynomial coefficient, ln2 part or reduction sign is
    # off by far more than 2^-23 relative
    ts = np.concatenate([np.linspace(-20, 80, 20001, dtype=np.float32),
                         np.random.default_rng(0).uniform(-0.5, 0.5, 4000).astype(np.float32),
                         np.float32([0.0, 1e-30, -1e-30, 0.3465736, -0.3465736, 80.0, -20.0])])
    worst = 0.0
    for t in ts:
        ref = math.exp(float(t))
        worst = max(worst, abs(oracle.exp_f32_seq(float(t)) - ref) / ref)
    assert worst <= 2 * U24, worst / U24


def test_exp_sequence_exact_points():
    assert oracle.exp_f32_seq(0.0) == 1.0
    # k = 1, r = ln2 - ln2_hi - ln2_lo ~ 1e-14: p = 1 + r rounds to 1, e = 2
    assert oracle.exp_f32_seq(float(np.float32(math.log(2.0)))) == 2.0


def silu64(x):
    return x / (1.0 + math.exp(-x))


def test_silu_within_three_half_ulps():
    # a wrong Newton step or seed, or a dropped clamp, is off by far more
    xs = np.concatenate([np.linspace(-80, 80, 20001, dtype=np.float32),
                         np.random.default_rng(1).uniform(-4, 4, 4000).astype(np.float32),
                         np.float32([1e-20, -1e-20, 1e-38, -1e-38, 0.5, -0.5, 19.99, -19.99])])
    worst = 0.0
    for x in xs:
        r = silu64(float(x))
        if r != 0.0:
            worst = max(worst, abs(oracle.silu_f32(float(x)) - r) / abs(r))
    assert worst <= 3 * U24, worst / U24


def test_silu_special_cases():
    assert oracle.silu_f32(0.0) == 0.0
    assert math.copysign(1.0, oracle.silu_f32(-0.0)) == -1.0       # -0 * y
    assert oracle.silu_f32(math.inf) == math.inf
    assert math.isnan(oracle.silu_f32(math.nan))
    # above 20, 1 + e^-x rounds to 1 and the reciprocal converges to 1:
    # SiLU is the identity, exactly
    for x in np.float32([20.0001, 21.5, 100.0, 3.0e38]):
        assert oracle.silu_f32(float(x)) == float(x)
    # below -80 the argument is clamped: x / (1 + e^80), within 1e-33 of the
    # true value (which is nearer 0 still)
    for x in (-80.01, -100.0, -1000.0):
        r = oracle.silu_f32(x)
        assert r < 0.0 and abs(r - x / (1.0 + math.exp(80.0))) <= 4 * U24 * abs(r)
    # SiLU(1) = 1 / (1 + 1/e) = 0.7310585786...
    assert abs(oracle.silu_f32(1.0) - 0.7310585786300049) <= 3 * U24


def test_silu_odd_part_identity():
    # sigma(x) + sigma(-x) = 1, so SiLU(x) - SiLU(-x) = x
    for x in np.random.default_rng(2).uniform(-30, 30, 3000).astype(np.float32):
        x = float(x)
        d = oracle.silu_f32(x) - oracle.silu_f32(-x)
        assert abs(d - x) <= 8 * U24 * max(abs(x), 1e-30), x


def test_float_to_bf16_matches_torch():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2 ** 32, 20000, dtype=np.uint64).astype(np.uint32)
    # ties to even both ways, and values that round up into the next binade
    ties = (rng.integers(0, 2 ** 16, 2000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    bits = np.concatenate([bits, ties, np.uint32([0x3F7FFFFF, 0x7F7FFFFF, 0x00008000, 0x80018000])])
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.float_to_bf16(float(v)) for v in f], dtype=np.uint16)
    assert np.array_equal(got, want)
    assert oracle.float_to_bf16(math.inf) == 0x7F80 and oracle.float_to_bf16(-math.inf) == 0xFF80


def bf16_bits(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bits_to_f64(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("pair", [32, 64, 96])
def test_swiglu_layout_against_direct_construction(pair):
    # C built from separate gate and up matrices by interleaving groups of
    # `pair` columns; H must be SiLU(gate) * up (a swapped or misaligned
    # gate/up is off by far more than the bf16 rounding)
    M, F = 7, 192
    rng = np.random.default_rng(4 + pair)
    g = bf16_bits(rng.normal(0, 3, (M, F)))
    u = bf16_bits(rng.normal(0, 1, (M, F)))
    c = np.zeros((M, 2 * F + 16), dtype=np.uint16)  # ldc > 2F
    view = c[:, :2 * F].reshape(M, F // pair, 2, pair)
    view[:, :, 0, :] = g.reshape(M, F // pair, pair)
    view[:, :, 1, :] = u.reshape(M, F // pair, pair)
    h = bits_to_f64(oracle.swiglu_bf16(c, F, pair))
    gf, uf = bits_to_f64(g), bits_to_f64(u)
    ref = gf / (1.0 + np.exp(-gf)) * uf
    assert np.all(np.abs(h - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30)


def test_swiglu_stacked_halves():
    # pair = F is the plain [gate | up] layout
    M, F = 5, 64
    rng = np.random.default_rng(9)
    g = bf16_bits(rng.normal(0, 2, (M, F)))
    u = bf16_bits(rng.normal(0, 2, (M, F)))
    h = bits_to_f64(oracle.swiglu_bf16(np.concatenate([g, u], axis=1), F, F))
    gf, uf = bits_to_f64(g), bits_to_f64(u)
    assert np.all(np.abs(h - gf / (1.0 + np.exp(-gf)) * uf) <= 2.0 ** -8 * np.abs(gf * uf) + 1e-30)


def test_swiglu_rejects_pair_not_dividing_f():
    with pytest.raises(ValueError):
        oracle.swiglu_bf16(np.zeros((2, 128), dtype=np.uint16), 64, 48)
