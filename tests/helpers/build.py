"""Build the GPU test helper libraries in-tree (tests/helpers/lib*.so) with
hipcc for gfx950.  Test infrastructure: nothing in the package loads them."""
from __future__ import annotations

import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))

HELPERS = {"libmfma_rates.so": "mfma_rates.hip"}

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def path(lib: str) -> str:
    return os.path.join(HERE, lib)


def build(verbose: bool = False) -> None:
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    for lib, src in HELPERS.items():
        tmp = path(lib) + ".tmp"
        cmd = [hipcc, *FLAGS, os.path.join(HERE, src), "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
        os.replace(tmp, path(lib))
