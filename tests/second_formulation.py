"""A second, deliberately different formulation of the quantizer steps, used
only to pin the oracle.  Where the oracle walks a magnitude table element by
element, this module decodes the E2M1 bit fields, does a vectorized
nearest-value search over all codes, takes the MX exponent from log2 instead
of frexp, and builds the Hadamard matrix explicitly by Kronecker products.
It is test code, small and slow, and is never used to produce expected values
for the GPU path.
"""
from __future__ import annotations

import numpy as np


def e2m1_decode_bits(code: int) -> float:
    """Value of a 4-bit E2M1 code from its fields: sign | exp(2) | mant(1),
    exponent bias 1, exponent field 0 is subnormal (0.5 * mantissa)."""
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    mag = 0.5 * m if e == 0 else (1.0 + 0.5 * m) * 2.0 ** (e - 1)
    return -mag if s else mag


MAGS = np.array([e2m1_decode_bits(c) for c in range(8)], dtype=np.float64)


def e2m1_rne_vec(y: np.ndarray) -> np.ndarray:
    """Nearest E2M1 magnitude by exhaustive distance search; ties to the even
    code; sign bit copied from y."""
    y = np.asarray(y, dtype=np.float32)
    # beyond 8 the nearest magnitude is 6 whatever m is; clipping keeps the
    # fp64 distances below from all rounding to the same huge value
    m = np.minimum(np.abs(y.astype(np.float64)), 8.0)
    d = np.abs(m[..., None] - MAGS)  # [..., 8]
    dmin = d.min(axis=-1, keepdims=True)
    cand = d == dmin
    # prefer an even candidate when two tie
    even = cand & (np.arange(8) % 2 == 0)
    pick = np.where(even.any(axis=-1), even.argmax(axis=-1), cand.argmax(axis=-1))
    sign = np.signbit(y).astype(np.uint8)
    return (sign << 3 | pick.astype(np.uint8)).astype(np.uint8)


def mx_exponent_vec(amax: np.ndarray) -> np.ndarray:
    a = np.asarray(amax, dtype=np.float64)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0))) - 2
    e = np.where(a > 0, e, -127)
    return np.clip(e, -127, 127).astype(np.int64)


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    c = codes.astype(np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def mx_quantize_rne_vec(v: np.ndarray):
    """MXFP4 RNE of an fp32 matrix [R, K] along K; returns (codes [R, K/2], scales [R, K/32])."""
    v = np.asarray(v, dtype=np.float32)
    R, K = v.shape
    blocks = v.reshape(R, K // 32, 32)
    amax = np.abs(blocks).max(axis=-1)
    E = mx_exponent_vec(amax)
    inv = np.ldexp(np.float32(1.0), (-E).astype(np.int32)).astype(np.float32)
    y = (blocks * inv[..., None]).astype(np.float32)  # one binary32 multiply
    codes = e2m1_rne_vec(y).reshape(R, K)
    return pack_nibbles(codes), (E + 127).astype(np.uint8)


def sylvester_hadamard(n: int = 32) -> np.ndarray:
    H = np.array([[1.0]])
    while H.shape[0] < n:
        H = np.kron(np.array([[1.0, 1.0], [1.0, -1.0]]), H)
    return H


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits_rne(x: np.ndarray) -> np.ndarray:
    """binary32 -> bf16 bits, round-to-nearest-even (finite inputs)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)
