"""Pins of the oracle's SwiGLU, the activation whose bf16 output H the fused
GEMM epilogue quantizes: H = bf16(SiLU(g) * u), evaluated in binary64 and
rounded once.  Pinned against a second formulation of the bf16 rounding (an exact search
over every bf16 value), a 40-digit decimal evaluation of SiLU over every
finite bf16 gate, hand-derived values, an identity, and the interleaved
gate/up column layout against a direct construction.  CPU only."""
import decimal
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

ALL = np.arange(65536, dtype=np.uint32)


def bits_to_f64(b):
    return (np.asarray(b).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_bits(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


# every finite non-negative bf16 value in increasing order (bit patterns
# 0x0000 .. 0x7F7F are increasing), with 2^128 appended as the rounding
# target past the largest (it stands for infinity)
POS_BITS = np.arange(0x7F80, dtype=np.uint32)
POS_VALS = np.concatenate([bits_to_f64(POS_BITS), [2.0 ** 128]])


def bf16_nearest_by_search(v: float) -> int:
    """Second formulation: bracket |v| between consecutive bf16 values by a
    search over the table, compare with their midpoint exactly (rationals),
    ties to the even bit pattern; sign copied."""
    if v == 0.0:
        return 0x8000 if math.copysign(1.0, v) < 0 else 0
    s = 0x8000 if v < 0 else 0
    a = Fraction(abs(v))
    i = int(np.searchsorted(POS_VALS, abs(v), side="right")) - 1
    if i >= len(POS_VALS) - 1:
        return s | 0x7F80
    lo, hi = Fraction(POS_VALS[i]), Fraction(POS_VALS[i + 1])
    mid = (lo + hi) / 2
    if a < mid:
        k = i
    elif a > mid:
        k = i + 1
    else:
        k = i if i % 2 == 0 else i + 1
    return s | (0x7F80 if k == len(POS_VALS) - 1 else k)


def test_double_to_bf16_against_exact_search():
    rng = np.random.default_rng(11)
    vals = list(rng.standard_normal(3000) * 10.0 ** rng.integers(-45, 39, 3000))
    # every midpoint of a sample of adjacent pairs, exactly and one binary64
    # step either side; the subnormal range; the overflow boundary
    idx = rng.integers(0, 0x7F7F, 3000)
    mids = (POS_VALS[idx] + POS_VALS[idx + 1]) / 2
    vals += list(mids) + list(np.nextafter(mids, 0)) + list(np.nextafter(mids, np.inf))
    vals += [2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135, 2.0 ** -126 * (1 - 2.0 ** -9), 2.0 ** -140,
             2.0 ** 128 * (1 - 2.0 ** -9), np.nextafter(2.0 ** 128 * (1 - 2.0 ** -9), 0), 3.0e38, 1e300, 0.0]
    vals += [-v for v in vals[::7]]
    for v in vals:
        assert oracle.double_to_bf16(float(v)) == bf16_nearest_by_search(float(v)), v
    assert oracle.double_to_bf16(math.inf) == 0x7F80 and oracle.double_to_bf16(-0.0) == 0x8000
    # the array form is the scalar one element by element
    arr = np.array(vals[:500])
    assert np.array_equal(oracle.double_to_bf16_array(arr),
                          np.array([oracle.double_to_bf16(float(v)) for v in arr], dtype=np.uint16))


def h_exact_bits(g: float, u: float, ctx):
    """bf16 of SiLU(g) u from 40-digit decimal arithmetic: P = g u (exact)
    times sigma(g), written without cancellation on either side (1 / (1 +
    e^-g) for g >= 0, e^g / (1 + e^g) below); compared exactly with the
    midpoint that brackets it.  Returns (bits, near): near is True when the
    value lies within 2^-50 (relative) of that midpoint, closer than a
    binary64 evaluation resolves.  |g| > 1000 is not passed here (the
    closed forms below cover it)."""
    P = Fraction(g) * Fraction(u)
    if P == 0:
        return (0x8000 if math.copysign(1.0, g) * math.copysign(1.0, u) < 0 else 0), False
    with decimal.localcontext(ctx):
        Pd = decimal.Decimal(P.numerator) / decimal.Decimal(P.denominator)
        G = decimal.Decimal(g)
        D = Pd / (1 + (-G).exp()) if g >= 0 else Pd * G.exp() / (1 + G.exp())
    a = abs(float(D))
    sign = 0x8000 if P < 0 else 0
    i = int(np.searchsorted(POS_VALS, a, side="right")) - 1
    i = min(max(i, 0), len(POS_VALS) - 2)
    # float(D) may sit one table entry off: step to the bracket of the exact D
    Dabs = abs(D)
    while i > 0 and decimal.Decimal(POS_VALS[i]) > Dabs:
        i -= 1
    while i < len(POS_VALS) - 2 and decimal.Decimal(POS_VALS[i + 1]) <= Dabs:
        i += 1
    with decimal.localcontext(ctx):
        mid = (decimal.Decimal(POS_VALS[i]) + decimal.Decimal(POS_VALS[i + 1])) / 2
        near = abs(Dabs - mid) <= decimal.Decimal(2) ** -50 * Dabs
    k = i if Dabs < mid else i + 1
    return sign | (0x7F80 if k == len(POS_VALS) - 1 else k), near


@pytest.mark.timeout(600)
def test_swiglu_against_decimal_every_bf16_gate():
    ctx = decimal.Context(prec=40, Emax=10 ** 6, Emin=-10 ** 6)
    g = bits_to_f64(ALL)
    ok = np.isfinite(g) & (np.abs(g) <= 1000)
    gates = ALL[ok]
    # up values (bf16): plain, ones whose products land on bf16 midpoints
    # for many gates (1 + 2^-7, 1 + 3 2^-7), tiny, and product-overflowing
    ub = bf16_bits(np.float32([1.0, -1.0078125, 1.0234375, 3.0e-30, -2.5e36]))
    for u, bits in zip(bits_to_f64(ub), ub):
        c = np.stack([gates.astype(np.uint16), np.full(gates.size, bits, dtype=np.uint16)], axis=1)
        got, hv = oracle.swiglu_bf16(c, 1, 1, with_f64=True)
        got, hv = got[:, 0], hv[:, 0]
        res = [h_exact_bits(float(gv), float(u), ctx) for gv in bits_to_f64(gates)]
        want = np.array([r[0] for r in res], dtype=np.uint16)
        near = np.array([r[1] for r in res])
        # the binary64 evaluation rounds like the real value everywhere except
        # within 2^-50 of a midpoint, where it still rounds its own value
        bad = np.flatnonzero((got != want) & ~near)
        assert bad.size == 0, (float(u), [(hex(gates[i]), hex(got[i]), hex(want[i])) for i in bad[:5]])
        assert np.array_equal(got, oracle.double_to_bf16_array(hv))
        assert near.sum() <= 0.02 * near.size, int(near.sum())


def test_swiglu_large_gates_closed_form():
    # |g| > 1000: SiLU(g) u = P (1 - s) with 0 < s < e^-1000 for g > 0: in
    # binary64 1 + e^-g is 1, so H is P (exact) rounded to nearest even; for
    # g < -1000, |SiLU(g) u| < |P| e^-1000 is far below the smallest bf16
    # and rounds to a zero of P's sign
    g = bits_to_f64(ALL)
    big = ALL[np.isfinite(g) & (np.abs(g) > 1000)]
    for ubits in bf16_bits(np.float32([1.0, -1.0078125, 1.0234375, 3e-30])):
        u = bits_to_f64(ubits)
        c = np.stack([big.astype(np.uint16), np.full(big.size, ubits, dtype=np.uint16)], axis=1)
        got = oracle.swiglu_bf16(c, 1, 1)[:, 0]
        for gb, h in zip(big, got):
            gv = float(bits_to_f64(gb))
            P = gv * float(u)  # exact in binary64
            if gv < 0:
                want = 0x8000 if P < 0 else 0
            else:
                want = bf16_nearest_by_search(P)
            assert h == want, (gv, float(u), hex(h), hex(want))


def one(g, u):
    gb = int(np.float32(g).view(np.uint32) >> 16)
    ub = int(np.float32(u).view(np.uint32) >> 16)
    assert bits_to_f64(gb) == g and bits_to_f64(ub) == u, "inputs must be bf16 values"
    return int(oracle.swiglu_bf16(np.array([[gb, ub]], dtype=np.uint16), 1, 1)[0, 0])


def test_swiglu_hand_derived_values():
    # SiLU(1) = 1 / (1 + 1/e) = 0.73105857...; in [0.5, 1) the bf16 step is
    # 2^-8: 0.73105857 * 256 = 187.15 -> 187 / 256 = 0.73046875 = 1.4609375
    # * 2^-1: exponent field 126, fraction 59 -> 0x3F3B
    assert one(1.0, 1.0) == 0x3F3B
    # g = 96, u = 1 + 2^-7: P = 96.75, the midpoint of 96.5 (fraction 65,
    # 0x42C1) and 97 (fraction 66, 0x42C2; the bf16 step in [64, 128) is
    # 0.5).  In binary64 1 + e^-96 = 1 + 2e-42 rounds to 1, so the evaluated
    # value is P itself and the tie goes to even: 97 (the real value, 2e-42
    # relative below the midpoint, would give 96.5 -- one of the
    # near-midpoint cases the definition leaves to binary64)
    assert one(96.0, 1.0078125) == 0x42C2
    assert one(96.0, -1.0078125) == 0xC2C2
    # u = 1 + 3 2^-7: P = 98.25, midpoint of 98 (fraction 68, even, 0x42C4)
    # and 98.5 -> 98
    assert one(96.0, 1.0234375) == 0x42C4
    # g = 8: 1 + e^-8 = 1.000335...; 8 u / 1.000335 for u = 1.0078125:
    # 8.0625 / 1.00033546 = 8.05979...; the bf16 step in [8, 16) is 2^-4:
    # 8.05979 * 16 = 128.957 -> 129 / 16 = 8.0625 = 1.0078125 * 2^3:
    # exponent field 130, fraction 1 -> 0x4101
    assert one(8.0, 1.0078125) == 0x4101
    # zero gate: SiLU(0) u = 0 with the sign of 0 * u
    assert one(0.0, 3.0) == 0x0000 and one(-0.0, 3.0) == 0x8000 and one(0.0, -3.0) == 0x8000
    # the product overflows bf16: 2^127 * 2 = 2^128 -> infinity
    assert one(2.0 ** 127, 2.0) == 0x7F80 and one(2.0 ** 127, -2.0) == 0xFF80


def test_swiglu_value_odd_part_identity():
    # sigma(x) + sigma(-x) = 1, so SiLU(x) - SiLU(-x) = x (binary64 value)
    for x in np.random.default_rng(2).uniform(-30, 30, 3000):
        x = float(np.float32(x))
        d = oracle.swiglu_f64(x, 1.0) - oracle.swiglu_f64(-x, 1.0)
        assert abs(d - x) <= 1e-15 * max(abs(x), 1.0), x


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


@pytest.mark.parametrize("pair", [32, 64, 96])
def test_swiglu_layout_against_direct_construction(pair):
    # C built from separate gate and up matrices by interleaving groups of
    # `pair` columns; H must be SiLU(gate) * up rounded once (a swapped or
    # misaligned gate/up is off by far more)
    M, F = 7, 192
    rng = np.random.default_rng(4 + pair)
    g = bf16_bits(rng.normal(0, 3, (M, F)))
    u = bf16_bits(rng.normal(0, 1, (M, F)))
    c = np.zeros((M, 2 * F + 16), dtype=np.uint16)  # ldc > 2F
    view = c[:, :2 * F].reshape(M, F // pair, 2, pair)
    view[:, :, 0, :] = g.reshape(M, F // pair, pair)
    view[:, :, 1, :] = u.reshape(M, F // pair, pair)
    h = oracle.swiglu_bf16(c, F, pair)
    gf, uf = bits_to_f64(g), bits_to_f64(u)
    want = np.array([[bf16_nearest_by_search(float(a / (1.0 + math.exp(-a)) * b)) for a, b in zip(ra, rb)]
                     for ra, rb in zip(gf, uf)], dtype=np.uint16)
    assert np.array_equal(h, want)


def test_swiglu_stacked_halves_and_values():
    # pair = F is the plain [gate | up] layout; with_f64 returns the values
    # H was rounded from
    M, F = 5, 64
    rng = np.random.default_rng(9)
    g = bf16_bits(rng.normal(0, 2, (M, F)))
    u = bf16_bits(rng.normal(0, 2, (M, F)))
    h, hv = oracle.swiglu_bf16(np.concatenate([g, u], axis=1), F, F, with_f64=True)
    gf, uf = bits_to_f64(g), bits_to_f64(u)
    ref = gf / (1.0 + np.exp(-gf)) * uf
    assert np.all(np.abs(hv - ref) <= 1e-15 * np.abs(ref))
    assert np.array_equal(h, oracle.double_to_bf16_array(hv))


def test_swiglu_rejects_pair_not_dividing_f():
    with pytest.raises(ValueError):
        oracle.swiglu_bf16(np.zeros((2, 128), dtype=np.uint16), 64, 48)
