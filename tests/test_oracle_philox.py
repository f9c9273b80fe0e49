"""Pins of the oracle's Philox4x32-10 and of the stochastic-rounding bit stream.

The reference is rocRAND's Philox4x32-10 engine, compiled here for the host
from its header (a library routine the oracle does not use)."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand_ref(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"):
        pytest.skip("hipcc / rocRAND headers not available")
    exe = str(tmp_path_factory.mktemp("philox") / "philox_rocrand")
    subprocess.run([hipcc, "--offload-arch=gfx950", "-O1", os.path.join(HERE, "helpers", "philox_rocrand.cpp"),
                    "-o", exe], check=True, capture_output=True)

    def run(tuples):
        inp = "".join(f"{s} {st} {r} {c}\n" for s, st, r, c in tuples)
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
        return [list(map(int, line.split())) for line in out.strip().splitlines()]

    return run


def test_philox_matches_rocrand(rocrand_ref):
    rng = np.random.default_rng(5)
    tuples = [(0, 0, 0, 0), (7, 0, 0, 0), (7, 1, 8191, 511), (2**64 - 1, 2**32 - 1, 2**30 - 1, 2**32 - 1),
              (0x243F6A8885A308D3, 3, 12, 34)]
    for _ in range(300):
        # the rocRAND offset 4 * (row * 2^32 + col8) must fit 64 bits: row < 2^30
        tuples.append((int(rng.integers(0, 2**63)), int(rng.integers(0, 2**32)), int(rng.integers(0, 2**30)),
                       int(rng.integers(0, 2**32))))
    ref = rocrand_ref(tuples)
    for (seed, stream, row, col8), want in zip(tuples, ref):
        got = oracle.philox4x32_10([col8, row, stream, 0], [seed & 0xFFFFFFFF, seed >> 32])
        assert got == want, (seed, stream, row, col8)


def test_r16_word_and_half_selection(rocrand_ref):
    # element col uses word (col/2) mod 4 of the call for col/8, low half for even col
    seed, stream, row = 7, 1, 4095
    for col in range(0, 64):
        w = rocrand_ref([(seed, stream, row, col >> 3)])[0]
        word = w[(col >> 1) & 3]
        want = (word >> 16) if col & 1 else (word & 0xFFFF)
        assert oracle.r16(seed, stream, row, col) == want


def test_r16_uniformity_chi2():
    # 2^16 draws into 256 bins of the top byte: chi-square with 255 dof
    vals = np.array([oracle.r16(7, 0, r, c) for r in range(64) for c in range(1024)], dtype=np.int64)
    assert vals.min() >= 0 and vals.max() < 65536
    counts = np.bincount(vals >> 8, minlength=256)
    exp = vals.size / 256
    chi2 = float(((counts - exp) ** 2 / exp).sum())
    assert 180 < chi2 < 340  # ~ +-4.5 sigma around 255
    # low byte too
    counts = np.bincount(vals & 0xFF, minlength=256)
    chi2 = float(((counts - exp) ** 2 / exp).sum())
    assert 180 < chi2 < 340
