"""bench.py's contract, checked without a GPU: one JSON line on one GPU only,
the algorithmic bytes per element it prices the producers with, and that the
committed rocprofv3 counter summaries it reads `traffic` from still match the
GEMM kernels' sources."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def run_bench(*args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300, env=env, cwd=ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
    r = run_bench(env_extra={"WORLD_SIZE": "4"})
    assert r.returncode == 2 and "WORLD_SIZE 4" in r.stderr


def test_no_gpu_no_line():
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is present: the bench would run")
    r = run_bench("--steps", "1", "--warmup", "0")
    assert r.returncode == 1 and "needs a GPU" in r.stderr and r.stdout == ""


def test_algorithmic_bytes_per_element():
    # bf16 in (2 B), E2M1 codes (1/2 B), one scale byte per block, tensor
    # scales per 128 x 128 tile (per-tile NVFP4); the global NVFP4 figure adds
    # the amax pass's second read of the input
    assert bench.MX_BYTES_PER_ELEM == 2.53125
    assert bench.MX_DUAL_BYTES_PER_ELEM == 2 + 2 * 0.53125
    assert bench.NV_TILE_BYTES_PER_ELEM == pytest.approx(2.5627441406, abs=1e-10)
    assert bench.NV_GLOBAL_BYTES_PER_ELEM == 4.5625


@pytest.mark.parametrize("kernel,workload", [("gemm_mx_kernel", "mlp"), ("gemm_mx_kernel", "qkv"),
                                             ("gemm_nv_fp16_kernel", "nvfp4_global"),
                                             ("gemm_nv_fp16_kernel", "nvfp4_tile")])
def test_counter_summaries_match_the_kernel_sources(kernel, workload):
    # a kernel changed since its counters were taken reports traffic null; the
    # committed summaries must be re-taken with the kernel they describe
    t = bench.read_traffic(kernel, workload)
    assert t is not None and t > 0
