"""Pins of the oracle's scalar format steps: E2M1 (RNE and stochastic), E4M3
and the MX shared exponent.  CPU only."""
import math

import numpy as np
import pytest

import oracle
from tests import second_formulation as sf

ALL_BF16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def finite_bf16():
    f = sf.bf16_to_f32(ALL_BF16)
    return ALL_BF16[np.isfinite(f)], f[np.isfinite(f)]


# ------------------------------------------------------------------ E2M1


def test_e2m1_table_from_bit_fields():
    # the oracle's magnitude table equals the value decoded from sign/exp/mant fields
    for c in range(16):
        assert oracle.e2m1_value(c) == sf.e2m1_decode_bits(c)
    assert sorted({abs(sf.e2m1_decode_bits(c)) for c in range(16)}) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def test_e2m1_all_codes_round_trip():
    # decode -> encode returns the same code for all 16 codes (incl. -0 -> 0x8)
    for c in range(16):
        v = oracle.e2m1_value(c)
        y = np.float32(-0.0) if c == 8 else np.float32(v)
        assert oracle.e2m1_rne(float(y)) == c, c
        for r in (0, 1, 12345, 65535):
            assert oracle.e2m1_sr(float(y), r) == c, (c, r)


@pytest.mark.parametrize("y,code", [
    (0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6),
    (0.2500001, 1), (0.7499999, 1), (5.0000005, 7), (6.0, 7), (7.99, 7), (1e30, 7),
    (-0.1, 8), (-0.0, 8), (0.0, 0), (-6.5, 15), (-1.3, 11),
])
def test_e2m1_rne_ties_and_saturation(y, code):
    assert oracle.e2m1_rne(float(np.float32(y))) == code


@pytest.mark.parametrize("E", [-127, -20, -6, 0, 6, 20, 125])
def test_e2m1_rne_exhaustive_vs_nearest_search(E):
    # every finite bf16 pattern, scaled by 2^-E in binary32, against the
    # second formulation's exhaustive nearest-value search
    bits, f = finite_bf16()
    with np.errstate(over="ignore"):
        y = (f * np.float32(2.0 ** -E)).astype(np.float32)
    y = y[np.isfinite(y)]
    lib = oracle._load()
    got = np.fromiter((lib.oc_e2m1_rne(float(v)) for v in y), dtype=np.uint8, count=y.size)
    want = sf.e2m1_rne_vec(y)
    assert np.array_equal(got, want)


def test_e2m1_sign_symmetry():
    rng = np.random.default_rng(1)
    ys = rng.standard_normal(2000).astype(np.float32) * 3
    for y in ys:
        assert oracle.e2m1_rne(float(-y)) == oracle.e2m1_rne(float(y)) ^ 8
        r = int(rng.integers(0, 65536))
        assert oracle.e2m1_sr(float(-y), r) == oracle.e2m1_sr(float(y), r) ^ 8


@pytest.mark.parametrize("y", [0.1, 0.3, 0.5, 0.6, 1.25, 1.3, 2.2, 2.75, 3.1, 4.5, 5.9, 0.0, 4.0])
def test_e2m1_sr_exact_unbiased_over_all_r16(y):
    # enumerate all 65536 random words: the mean of the dequantized value is y
    # exactly whenever f * 2^16 is an integer, else within 2^-16 of a step
    y = np.float32(y)
    vals = np.array([oracle.e2m1_value(oracle.e2m1_sr(float(y), r)) for r in range(65536)])
    mags = sf.MAGS
    lo = mags[mags <= y].max()
    hi = mags[mags > y].min() if y < 6 else lo
    f = (float(y) - lo) / (hi - lo) if hi > lo else 0.0
    ups = int(np.sum(vals > lo))
    assert ups == math.ceil(f * 65536)
    assert set(np.unique(vals)) <= {lo, hi}
    step = hi - lo
    assert abs(vals.mean() - float(y)) <= step * 2.0 ** -16 + 1e-15
    if float(f * 65536).is_integer():
        assert vals.mean() == pytest.approx(float(y), abs=0, rel=1e-15)


def test_e2m1_sr_representable_never_moves_and_saturates():
    for c in range(8):
        y = oracle.e2m1_value(c)
        for r in range(0, 65536, 977):
            assert oracle.e2m1_sr(y, r) == c
    for r in (0, 65535):
        assert oracle.e2m1_sr(7.5, r) == 7
        assert oracle.e2m1_sr(-100.0, r) == 15


def test_e2m1_sr_unbiased_over_seeds_statistical():
    # mean over Philox-driven draws stays within 4 sigma of y
    rng = np.random.default_rng(2)
    for y in (0.3, 1.1, 2.4, 4.7):
        n = 20000
        vals = np.array([oracle.e2m1_value(oracle.e2m1_sr(y, oracle.r16(s, 0, 0, 0))) for s in range(n)])
        sd = vals.std()
        assert abs(vals.mean() - y) <= 4 * sd / math.sqrt(n) + 1e-12, y
    del rng


# ------------------------------------------------------------------ E4M3


def e4m3_table():
    return np.array([oracle.e4m3_value(c) for c in range(0x7F)])


def test_e4m3_values_closed_form():
    t = e4m3_table()
    assert t[0] == 0 and t[1] == 2.0 ** -9 and t[7] == 7 * 2.0 ** -9
    assert t[8] == 2.0 ** -6 and t[0x38] == 1.0 and t[0x7E] == 448.0
    assert np.all(np.diff(t) > 0)  # strictly increasing over 0x00..0x7E
    assert oracle.e4m3_value(0x80 | 0x38) == -1.0


def test_e4m3_round_trip_and_ties():
    t = e4m3_table()
    for c in range(0x7F):
        assert oracle.e4m3_rne_satfinite(float(t[c])) == c
    for c in range(0x7E):
        mid = (t[c] + t[c + 1]) / 2
        assert np.float32(mid) == mid  # midpoints are exact binary32
        want = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_rne_satfinite(float(mid)) == want, hex(c)
        # just off the midpoint goes to the nearer side
        below = np.nextafter(np.float32(mid), np.float32(0))
        above = np.nextafter(np.float32(mid), np.float32(1e9))
        assert oracle.e4m3_rne_satfinite(float(below)) == c
        assert oracle.e4m3_rne_satfinite(float(above)) == c + 1


def test_e4m3_saturation_and_zero():
    assert oracle.e4m3_rne_satfinite(448.0) == 0x7E
    assert oracle.e4m3_rne_satfinite(463.9) == 0x7E
    assert oracle.e4m3_rne_satfinite(1e30) == 0x7E
    assert oracle.e4m3_rne_satfinite(0.0) == 0x00
    assert oracle.e4m3_rne_satfinite(7.5 * 2.0 ** -9) == 0x08
    assert oracle.e4m3_rne_satfinite(2.0 ** -10) == 0x00  # tie 0x00 / 0x01 -> even
    assert oracle.e4m3_rne_satfinite(float(np.float32(2.0 ** -10 * 1.0001))) == 0x01


# ------------------------------------------------------------------ MX exponent


def test_mx_exponent_closed_forms():
    for k in range(-120, 120, 7):
        assert oracle.mx_shared_exponent(2.0 ** k) == k - 2
        assert oracle.mx_shared_exponent(6 * 2.0 ** k) == k
        assert oracle.mx_shared_exponent(7 * 2.0 ** k) == k
        # largest bf16 below 2^(k+1) has the same exponent as 2^k
        below = float((2 - 2 ** -7) * 2.0 ** k)
        assert oracle.mx_shared_exponent(below) == k - 2
    assert oracle.mx_shared_exponent(0.0) == -127
    assert oracle.mx_shared_exponent(2.0 ** -130) == -127  # subnormal amax clamps
    assert oracle.mx_shared_exponent(2.0 ** -125) == -127
    assert oracle.mx_shared_exponent(2.0 ** -124) == -126
    big = float(np.float32(3.0e38))
    assert oracle.mx_shared_exponent(big) == 127 - 2


def test_mx_exponent_matches_log2_formulation():
    bits, f = finite_bf16()
    a = np.abs(f)
    got = np.fromiter((oracle.mx_shared_exponent(float(v)) for v in a), dtype=np.int64, count=a.size)
    assert np.array_equal(got, sf.mx_exponent_vec(a))
