"""The arithmetic behind the NVFP4 GEMM's choice of fp16 matrix cores.

An NVFP4 operand value is an E2M1 payload times an E4M3 block scale (per 16
elements) times an FP32 tensor scale ("FP4 Is No Longer Just a Hardware
Feature -- The NVFP4 Software Stack Is Taking Shape", section "NVFP4 is more
than a 4-bit value").  The payload-times-block-scale part is what a matrix
core would multiply.  Facts checked here, on every (E2M1, E4M3) pair:
- it has at most 6 significant bits, and 6 occur: one E4M3 value (4
  significant bits) cannot hold it, fp16 (11) and bf16 (8) can;
- two E4M3-precision parts always hold it exactly (hi = the value rounded to
  4 significant bits, lo = the rest, at most 2 significant bits);
- its range 2^-10 .. 2688 exceeds E4M3's 2^-9 .. 448, so the parts need a
  power-of-two shift, and gfx950's scaled fp8 instruction has one per 32
  elements = two NV blocks: a group whose two block scales lie far apart has
  no shift that keeps every part representable (constructed case).
On the NVFP4 configuration's operands (1024-row samples of X and W, both
scale domains) every 32-element group does have such a shift; the fraction
is printed.  The cost of the split on the matrix cores is measured in
tests/test_gpu_mfma_rates.py."""
import numpy as np

import oracle
from fp4_block_scaled_quantizer_amd import synth

E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)
E4M3 = np.array([oracle.e4m3_value(c) for c in range(0x7F)], dtype=np.float64)  # 0x7F is NaN


def sig_bits(v):
    """Significant bits of positive binary64 values (exact)."""
    m, _ = np.frexp(v)
    mi = (m * 2.0 ** 53).astype(np.int64)
    tz = np.zeros(mi.shape, dtype=np.int64)
    t = mi.copy()
    for b in (32, 16, 8, 4, 2, 1):
        z = (t & ((1 << b) - 1)) == 0
        tz += np.where(z, b, 0)
        t = np.where(z, t >> b, t)
    return 53 - tz


def lsb_exponent(v):
    _, e = np.frexp(v)
    return e - sig_bits(v)  # v is an odd integer times 2^this


def round_sig(v, bits):
    """v rounded to nearest even at `bits` significant bits (binary64 exact)."""
    m, e = np.frexp(v)
    return np.ldexp(np.round(np.ldexp(m, bits)), e - bits)


def test_products_need_two_e4m3_parts():
    v = np.unique(np.outer(E2M1[1:], E4M3[1:]).ravel())
    nb = sig_bits(v)
    assert nb.max() == 6 and (nb > 4).any() and (nb <= 11).all()  # not E4M3, always fp16
    hi = round_sig(v, 4)
    lo = v - hi
    nz = lo != 0
    assert (sig_bits(np.abs(lo[nz])) <= 2).all()  # the rest fits a second 4-bit part
    assert v.min() == 2.0 ** -10 and v.max() == 2688.0  # wider than E4M3's 2^-9 .. 448


def group_has_shift(vals):
    """One power-of-two shift s (the 32-element E8M0 scale) under which the
    hi and lo parts of every value are E4M3 values: |v| 2^-s <= 448 and
    every part's lowest bit >= 2^-9 (E4M3's subnormal step)."""
    v = np.abs(vals[vals != 0])
    if v.size == 0:
        return True
    need = int(np.ceil(np.log2(v.max() / 448.0)))
    return need <= int(lsb_exponent(v).min()) + 9


def fraction_with_shift(codes, scales):
    c = np.empty((codes.shape[0], codes.shape[1] * 2), dtype=np.uint8)
    c[:, 0::2] = codes & 15
    c[:, 1::2] = codes >> 4
    v = E2M1[c & 7] * np.repeat(E4M3[scales & 0x7F], 16, axis=1)
    R, K = v.shape
    g = v.reshape(R * K // 32, 32)
    nz = g > 0
    lsb = np.where(nz, lsb_exponent(np.where(nz, g, 1.0)), 1 << 20).min(axis=1)
    mx = g.max(axis=1)
    need = np.ceil(np.log2(np.maximum(mx, 1e-300) / 448.0))
    ok = ~nz.any(axis=1) | (need <= lsb + 9)
    return float(ok.mean())


def test_a_group_without_a_shift_exists():
    # two NV blocks of one 32-element group: block scales 2^-9 (with the
    # payload 1.5: lowest bit 2^-10) and 448 (payload 6: 2688)
    vals = np.concatenate([np.full(16, 1.5 * 2.0 ** -9), np.full(16, 6 * 448.0)])
    assert not group_has_shift(vals)
    assert group_has_shift(vals[:16]) and group_has_shift(vals[16:])


def test_config_operands_fraction():
    for role in ("X", "W"):
        xb = synth.bf16_bits(synth.config_tensor("nvfp4", role)[:1024])
        for domain in (0, 1):
            codes, scales, _ = oracle.quantize_nv(xb, domain=domain)
            f = fraction_with_shift(codes, scales)
            print(f"NVFP4 {role} (1024 rows), domain {domain}: {f:.6f} of 32-element groups split exactly")
            assert 0.0 <= f <= 1.0
