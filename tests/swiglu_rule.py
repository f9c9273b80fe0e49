"""When a kernel's H = bf16(SiLU(g) * u) may differ from the oracle's (test code).

The oracle rounds SiLU(g) u, evaluated in binary64, once to bf16.  The
kernels evaluate SiLU(g) in binary32 by a fixed sequence whose error over
every finite bf16 g is bounded on the host (test_device_helpers:
SILU_REL_BOUND relative for normal results, SILU_ABS_BOUND absolute in the
subnormal range), multiply by u in binary32 (one more rounding: 2^-24
relative, 2^-150 absolute) and round that to bf16.  So the kernel's binary32
value lies within

    W = (SILU_REL_BOUND + 2^-24 + SILU_REL_BOUND 2^-24 + 2^-50) |h|
        + SILU_ABS_BOUND |u|   (only where |SiLU(g)| < 2^-126)
        + 2^-150

of the oracle's binary64 value h (2^-50 covers h's own error), and its bf16
must be one of the bf16 values whose rounding interval meets [h - W, h + W]:
the oracle's own, or (where a bf16 midpoint lies within W of h) a
neighbour.  Far from the subnormal range W is below a bf16 step, so at most
one neighbour qualifies; a subnormal binary32 SiLU (gates below about -87)
times a large up value can admit several.  `allowed_range` gives, per
element, the admitted magnitudes as a range of bit patterns.
"""
from __future__ import annotations

import itertools

import numpy as np

import oracle

SILU_REL_BOUND = 4 * 2.0 ** -24
SILU_ABS_BOUND = 2.0 ** -149


def _mag_value(mag):
    """bf16 magnitude bit patterns (0 .. 0x7F80) -> float64, 0x7F80 -> 2^128
    (the rounding target past the largest finite value)."""
    mag = np.asarray(mag, dtype=np.uint32)
    v = (np.minimum(mag, 0x7F7F) << 16).view(np.float32).astype(np.float64)
    return np.where(mag >= 0x7F80, 2.0 ** 128, v)


def window(hv, u):
    hv = np.abs(np.asarray(hv, dtype=np.float64))
    u = np.abs(np.asarray(u, dtype=np.float64))
    rel = SILU_REL_BOUND + 2.0 ** -24 + SILU_REL_BOUND * 2.0 ** -24 + 2.0 ** -50
    with np.errstate(divide="ignore", invalid="ignore"):
        silu_sub = np.where(u > 0, hv / u, 0.0) < 2.0 ** -126 * (1 + 2.0 ** -20)
    return rel * hv + np.where(silu_sub, SILU_ABS_BOUND * u, 0.0) + 2.0 ** -150


def allowed_range(want, hv, u):
    """Per element: the bf16 magnitude bit patterns [lo, hi] a kernel may
    return (with the oracle's sign): the round-to-nearest images of
    |h| - W and |h| + W, and everything between (rounding is monotonic)."""
    a = np.abs(np.asarray(hv, dtype=np.float64))
    W = window(hv, u)
    lo = oracle.double_to_bf16_array(np.maximum(a - W, 0.0)).astype(np.int64) & 0x7FFF
    hi = oracle.double_to_bf16_array(a + W).astype(np.int64) & 0x7FFF
    return lo, hi


def check_h(got, want, hv, u, what="h"):
    """Every kernel value equals the oracle's or lies in its admitted range.
    NaN patterns (0x7F81..0x7FFF, either sign) compare by NaN-ness.  Returns
    (elements differing, elements where a difference was allowed)."""
    got = np.asarray(got, dtype=np.uint16)
    want = np.asarray(want, dtype=np.uint16)
    gnan = (got & 0x7FFF) > 0x7F80
    wnan = (want & 0x7FFF) > 0x7F80
    assert np.array_equal(gnan, wnan), f"{what}: NaN positions differ"
    lo, hi = allowed_range(want, hv, u)
    g = got.astype(np.int64)
    diff = (got != want) & ~wnan
    ok = ((g & 0x8000) == (want.astype(np.int64) & 0x8000)) & ((g & 0x7FFF) >= lo) & ((g & 0x7FFF) <= hi)
    bad = diff & ~ok
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} of {got.size} values outside the rule; first {i}: "
                             f"gpu {int(got[i]):#06x} oracle {int(want[i]):#06x} h {float(hv[i])!r}")
    return int(diff.sum()), int((hi > lo).sum())


def check_quantized_h(codes, scales, want_h, hv, u, quantize):
    """The MX operand of H written by a fused kernel (linear layout: codes
    [R, F/2], scales [R, F/32]) against quantize(H) of the oracle's H, block
    by block: a block may differ only if it holds elements whose admitted
    range has more than one value, and then must equal the quantization of
    H with some admitted choice for those elements.  quantize(h_bits
    [n, 32]) -> (codes, scales).  Returns (blocks differing, blocks holding
    such an element)."""
    want_h = np.asarray(want_h, dtype=np.uint16)
    R, F = want_h.shape
    wc, ws = quantize(want_h)
    codes = np.asarray(codes)
    scales = np.asarray(scales)
    blk_code_bad = (codes.reshape(R, F // 32, 16) != wc.reshape(R, F // 32, 16)).any(axis=2)
    blk_bad = blk_code_bad | (scales != ws)
    lo, hi = allowed_range(want_h, hv, u)
    has_alt = (hi > lo).reshape(R, F // 32, 32).any(axis=2)
    unexplained = blk_bad & ~has_alt
    if unexplained.any():
        r, j = np.argwhere(unexplained)[0]
        raise AssertionError(f"{int(unexplained.sum())} MX blocks differ with no element near a bf16 midpoint; "
                             f"first row {r} block {j}")
    cand_rows, cand_meta = [], []
    for r, j in np.argwhere(blk_bad):
        blk = want_h[r, 32 * j:32 * j + 32]
        sign = blk.astype(np.int64) & 0x8000
        choices = [[int(blk[e])] if hi[r, 32 * j + e] == lo[r, 32 * j + e] else
                   [int(sign[e] | k) for k in range(lo[r, 32 * j + e], hi[r, 32 * j + e] + 1)] for e in range(32)]
        n = int(np.prod([len(c) for c in choices]))
        assert n <= 4096, "too many admitted H values in one block"
        for combo in itertools.product(*choices):
            cand_rows.append(np.array(combo, dtype=np.uint16))
            cand_meta.append((r, j))
    if cand_rows:
        cc, cs = quantize(np.stack(cand_rows))
        matched = set()
        for (r, j), c16, s1 in zip(cand_meta, cc, cs):
            if np.array_equal(c16, codes[r, 16 * j:16 * j + 16]) and s1[0] == scales[r, j]:
                matched.add((int(r), int(j)))
        missing = [(int(r), int(j)) for r, j in np.argwhere(blk_bad) if (int(r), int(j)) not in matched]
        assert not missing, f"{len(missing)} MX blocks match no allowed choice of H; first {missing[0]}"
    return int(blk_bad.sum()), int(has_alt.sum())
