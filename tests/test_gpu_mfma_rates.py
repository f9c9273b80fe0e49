"""Would an NVFP4 GEMM on gfx950's 8-bit matrix cores beat the fp16 path?

An E2M1 value times its E4M3 block scale has up to 6 significant bits
(tests/test_nv_fp8_split.py); E4M3 holds 4, so an exact product on fp8
matrix cores takes each operand in two E4M3 parts: four fp8 products for
every fp16 one.  libfp4q's NV GEMM runs v_mfma_f32_32x32x16_f16 on the
exact fp16 dequantization instead.  This measures, on the GPU, the cycles
per instruction of the fp16, bf16, fp8 and fp4 32x32 instructions (8
independent accumulators per wave, one wave per SIMD on every CU, cycles by
s_memtime) and checks the cost of one 128-wide K step of a 32x32 output
block both ways: fp16 = 8 instructions of K 16; two-part fp8 = 4 x 2
instructions of K 64.  A second test holds the FP4 instruction on changing
operands for a few seconds and reports the sustained rate: the practical
ceiling of the MXFP4 GEMM on this chip."""
import ctypes

import numpy as np
import pytest
import torch

from tests.gpu_common import announce, device
from tests.helpers import build as helpers

pytestmark = pytest.mark.gpu

KINDS = {"fp16": (0, 16), "bf16": (1, 16), "fp8": (2, 64), "fp4": (3, 64)}  # kind id, K per instruction


def cycles_per_instruction(kind, blocks=256, iters=2000):
    lib = ctypes.CDLL(helpers.path("libmfma_rates.so"))
    lib.mfma_rate_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p]
    dev = device()
    cyc = torch.zeros(blocks * 4, dtype=torch.int64, device=dev)
    sink = torch.zeros(blocks * 256, dtype=torch.float32, device=dev)
    st = torch.cuda.current_stream(dev).cuda_stream
    for _ in range(2):  # the second launch is the one read
        assert lib.mfma_rate_launch(kind, blocks, iters, cyc.data_ptr(), sink.data_ptr(), st) == 0
    torch.cuda.synchronize()
    return float(cyc.cpu().numpy().astype(np.float64).mean()) / (iters * 8)


def test_fp8_split_does_not_beat_fp16():
    announce("matrix-core instruction rates")
    c = {name: cycles_per_instruction(kid) for name, (kid, _) in KINDS.items()}
    for name, (_, k) in KINDS.items():
        print(f"{name}: {c[name]:.1f} cycles per 32x32x{k} instruction, {k / c[name]:.3f} K per cycle")
    step_fp16 = (128 // 16) * c["fp16"]
    step_fp8_split = 4 * (128 // 64) * c["fp8"]
    step_fp8_one_side = 2 * (128 // 64) * c["fp8"]
    print(f"one 128-wide K step of a 32x32 block: fp16 {step_fp16:.0f} cycles, two-part fp8 "
          f"{step_fp8_split:.0f} ({step_fp8_split / step_fp16:.2f}x), one operand split {step_fp8_one_side:.0f}")
    assert step_fp8_split >= step_fp16, "fp8 matrix cores would win: revisit the NVFP4 GEMM"
    assert c["fp4"] <= c["fp8"]


def test_fp4_sustained_rate_on_changing_operands():
    # The FP4 instruction at full issue (one wave per SIMD, eight independent
    # accumulators) on random operands that change every instruction, held
    # for about 2.7 s: after the first second the chip runs at its sustained,
    # power-limited clock.  The rate over the last 1.5 s is the practical
    # ceiling a GEMM's matrix cores could reach on this chip (no memory
    # traffic at all), next to the 10.1 PFLOP/s nominal dense peak.
    import time
    announce("sustained FP4 matrix-core rate")
    lib = ctypes.CDLL(helpers.path("libmfma_rates.so"))
    lib.mfma_rate_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p]
    dev = device()
    blocks, iters = 256, 20000
    cyc = torch.zeros(blocks * 4, dtype=torch.int64, device=dev)
    sink = torch.zeros(blocks * 256, dtype=torch.float32, device=dev)
    st = torch.cuda.current_stream(dev).cuda_stream
    launch = lambda: lib.mfma_rate_launch(4, blocks, iters, cyc.data_ptr(), sink.data_ptr(), st)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 1.2:
        for _ in range(16):
            assert launch() == 0
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n = 0
    e0.record()
    t1 = time.perf_counter()
    while time.perf_counter() - t1 < 1.5:
        for _ in range(16):
            assert launch() == 0
        n += 16
        e1.record()
        e1.synchronize()
    ms = e0.elapsed_time(e1)
    flops = n * blocks * 4 * iters * 8 * (32 * 32 * 64 * 2)
    cycles_per_instr = float(cyc.cpu().numpy().astype(np.float64).mean()) / (iters * 8)
    rate = flops / (ms * 1e-3) / 1e12
    ghz = cycles_per_instr * iters * 8 / (ms * 1e-3 / n) / 1e9  # s_memtime counts core clock cycles
    print(f"FP4 32x32x64 on changing operands: {rate:.0f} TFLOP/s sustained over {ms / 1e3:.2f} s "
          f"({rate / 10100:.3f} of the 10.1 PFLOP/s nominal peak), {cycles_per_instr:.1f} cycles per instruction, "
          f"{ghz:.2f} GHz implied")
    assert 0 < rate <= 10200 and np.isfinite(sink.cpu().numpy()).all()

