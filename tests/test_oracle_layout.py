"""Pin of the oracle's tiled-layout index map against a per-element
brute-force reading of its definition (CPU only)."""
import numpy as np
import pytest

import oracle


def brute_tile(codes, scales):
    R, K2 = codes.shape
    K = 2 * K2
    Rp = (R + 31) // 32 * 32
    out = np.zeros(Rp * K2, dtype=np.uint8)
    for r in range(R):
        for k in range(K):
            nib = (codes[r, k // 2] >> (4 * (k & 1))) & 0xF
            g, kb = r // 32, k // 64
            lane = (r % 32) + 32 * ((k % 64) // 32)
            byte = ((g * (K // 64) + kb) * 64 + lane) * 16 + (k % 32) // 2
            out[byte] |= nib << (4 * (k & 1))
    sc = np.zeros(Rp * K // 32, dtype=np.uint8)
    for r in range(R):
        for j in range(K // 32):
            sc[((j // 4) * Rp + r) * 4 + j % 4] = scales[r, j]
    return out.reshape(Rp, K2), sc.reshape(K // 128, Rp, 4)


@pytest.mark.parametrize("R,K", [(1, 128), (32, 128), (33, 256), (70, 384)])
def test_tile_mx_matches_definition(R, K):
    rng = np.random.default_rng(R * 1000 + K)
    codes = rng.integers(0, 256, (R, K // 2)).astype(np.uint8)
    scales = rng.integers(0, 256, (R, K // 32)).astype(np.uint8)
    t, s = oracle.tile_mx(codes, scales)
    bt, bs = brute_tile(codes, scales)
    assert np.array_equal(t, bt) and np.array_equal(s, bs)


def test_tile_mx_block_is_one_mfma_operand():
    # block (0, 0) lane l holds row l % 32, K elements 32 (l / 32) .. +31
    R, K = 32, 128
    codes = np.zeros((R, K // 2), dtype=np.uint8)
    for r in range(R):
        codes[r, :] = r  # every byte of row r = r
    t, _ = oracle.tile_mx(codes, np.zeros((R, K // 32), np.uint8))
    flat = t.reshape(-1)
    for l in range(64):
        assert np.all(flat[l * 16:(l + 1) * 16] == l % 32)


@pytest.mark.parametrize("R,K", [(1, 128), (33, 256), (64, 512), (95, 384)])
def test_untile_inverts_tile(R, K):
    # the tests' inverse of the tiled layout (used to read fused kernels'
    # tiled outputs) undoes oracle.tile_mx and exposes zero padding rows
    from tests.gpu_common import untile_mx

    rng = np.random.default_rng(R * K)
    codes = rng.integers(0, 256, (R, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, (R, K // 32), dtype=np.uint8)
    tc, ts = oracle.tile_mx(codes, scales)
    c, s, cpad, spad = untile_mx(tc, ts, R, K)
    assert np.array_equal(c, codes) and np.array_equal(s, scales)
    assert not cpad.any() and not spad.any()


def brute_tile_nv(codes, scales):
    # element by element from the definition: code nibble of (r, k) goes to
    # block (g = r / 32, step s = k / 128), row f = r mod 32, byte (k mod 128) / 2
    R, K2 = codes.shape
    K = 2 * K2
    Rp = (R + 31) // 32 * 32
    S = K // 128
    out = np.zeros(Rp * K2, dtype=np.uint8)
    sout = np.zeros(Rp * K // 16, dtype=np.uint8)
    for r in range(R):
        g, f = r // 32, r % 32
        for k in range(K):
            nib = (codes[r, k // 2] >> (4 * (k & 1))) & 0xF
            byte = ((g * S + k // 128) * 32 + f) * 64 + (k % 128) // 2
            out[byte] |= nib << (4 * (k & 1))
        for j in range(K // 16):
            sout[((g * S + j // 8) * 32 + f) * 8 + j % 8] = scales[r, j]
    return out.reshape(Rp, K2), sout.reshape(Rp, K // 16)


@pytest.mark.parametrize("R,K", [(1, 128), (33, 256), (64, 384), (70, 512)])
def test_tile_nv_against_bruteforce(R, K):
    rng = np.random.default_rng(R + K)
    codes = rng.integers(0, 256, (R, K // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, (R, K // 16), dtype=np.uint8)
    tc, ts = oracle.tile_nv(codes, scales)
    bc, bs = brute_tile_nv(codes, scales)
    assert np.array_equal(tc, bc) and np.array_equal(ts, bs)
