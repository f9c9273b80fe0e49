"""Shared helpers of the GPU parity tests (test code)."""
import sys

import numpy as np
import pytest
import torch

import oracle
from fp4_block_scaled_quantizer_amd import binding as B
from fp4_block_scaled_quantizer_amd import synth


def device():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    return torch.device("cuda:0")


def announce(msg):
    # name the case before any GPU work, so a failing run says which one
    print(f"[gpu case] {msg}", file=sys.stderr, flush=True)


def to_dev(x_cpu, dev, ld=None):
    """bf16 CPU tensor -> device tensor, optionally inside a wider row pitch."""
    rows, cols = x_cpu.shape
    if ld is None or ld == cols:
        return x_cpu.to(dev)
    big = torch.zeros((rows, ld), dtype=torch.bfloat16)
    big[:, :cols] = x_cpu
    return big.to(dev)[:, :cols]


def ld_of(rows, cols, ld):
    return cols if ld is None else ld


def np_u8(t):
    return t.cpu().numpy()


def assert_bytes_equal(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.argwhere(got != want)
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} of {got.size} bytes differ; first at {i}: "
                             f"gpu {got[i]:#04x} oracle {want[i]:#04x}")


def gemm_check(c_gpu, c_ref, w, what, tol=1e-5):
    c = np.asarray(c_gpu, dtype=np.float64)
    err = np.abs(c - c_ref)
    bound = tol * w
    bad = err > bound
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(f"{what}: {int(bad.sum())} elements out of tolerance; first {i}: gpu {c[i]!r} "
                             f"ref {c_ref[i]!r} err {err[i]:.3e} bound {bound[i]:.3e}")
    return float((err / np.maximum(w, 1e-300)).max())


def untile_mx(codes_t, scales_t, R, K):
    """Inverse of the tiled consumer layout (oracle.tile_mx): returns the
    linear codes [R, K/2] and scales [R, K/32] plus the padding rows'
    codes and scales (which a producer must write as zeros)."""
    codes_t = np.asarray(codes_t, dtype=np.uint8)
    scales_t = np.asarray(scales_t, dtype=np.uint8)
    Rp = (R + 31) // 32 * 32
    c = codes_t.reshape(Rp // 32, K // 64, 2, 32, 16).transpose(0, 3, 1, 2, 4).reshape(Rp, K // 2)
    s = scales_t.reshape(K // 128, Rp, 4).transpose(1, 0, 2).reshape(Rp, K // 32)
    return c[:R], s[:R], c[R:], s[R:]


def bf16_bits_of(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


__all__ = ["device", "announce", "to_dev", "np_u8", "assert_bytes_equal", "gemm_check", "B", "synth", "oracle",
           "bf16_bits_of", "untile_mx"]
