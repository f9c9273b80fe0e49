#!/usr/bin/env python3
"""Benchmark of the FP4 hot path on one MI355X.

A step is one pass of the path over one batch of synthetic Llama-3-8B-shaped
operands.  The default workload is the MLP forward (MXFP4, RNE), the largest
one-GPU configuration: quantize X (8192x4096) and W_gate/up (28672x4096),
the gate/up GEMM (8192x28672x4096, bf16 out), quantize H (8192x14336, a
SiLU-product-like bf16 input) and W_down (4096x14336), the down GEMM
(8192x4096x14336, bf16 out).  Weights are re-quantized every step, as in
training where they change.

Prints one JSON line.  `value` is quantize+GEMM TFLOP/s = GEMM flops per step
/ time per step, with inputs resident in HBM (several input copies are
rotated so the producers read from HBM, not from the 256 MB Infinity Cache).
The timed region is K steps launched back to back with no event markers
between kernels.  `roofline` describes the dominant kernel (by name: for the
MLP, gemm_mx_kernel, both GEMMs): its algorithmic flops (or bytes) per
launch over its average launch duration, from HIP events on the launch
stream around each of its launches in a second pass of K steps (a marker
costs the GPU a few microseconds, so the `value` pass has none);
`kernels` lists every op of the step; `cpu_baseline` times the CPU oracle
on a bounded slice of the same step, single-threaded and on every host core.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

WARM_S = 0.5                 # minimum warmup time (seconds)
HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
FP4_PEAK_TFLOPS = 10100.0    # dense MFMA, fp4/fp6
BF16_PEAK_TFLOPS = 2500.0    # dense MFMA, bf16

# algorithmic bytes per element (payload + block scales + tensor scales, logical rows)
MX_BYTES_PER_ELEM = 2 + 0.5 + 1 / 32
MX_DUAL_BYTES_PER_ELEM = 2 + 2 * (0.5 + 1 / 32)  # one read, two operands written
NV_TILE_BYTES_PER_ELEM = 2 + 0.5 + 1 / 16 + 4 / (128 * 128)
NV_GLOBAL_BYTES_PER_ELEM = 2 + 2 + 0.5 + 1 / 16   # includes the amax pre-pass read


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mlp",
                    choices=["qkv", "mlp", "backward", "backward_dual", "dual_x", "nvfp4_global", "nvfp4_tile",
                             "nvfp4_chain", "nvfp4_chain_2pass", "nvfp4_wgrad", "mlp_chain", "mlp_chain_fused",
                             "mlp_swiglu", "mlp_swiglu_fused", "copy"],
                    help="copy = a plain 1 GiB device copy: the HBM reference for counter scaling")
    ap.add_argument("--copies", type=int, default=4, help="input copies rotated across steps (cold producers)")
    ap.add_argument("--layout", default="tiled", choices=["tiled", "linear"],
                    help="MX operand layout between producer and GEMM (tiled = the GEMM's consumer layout)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


def build_workload(name, dev, copies, layout_name="tiled"):
    """Returns (config dict, list of ops, flops per step).  An op is
    (label, kernel, launch(step), amount, unit, peak, bound)."""
    import torch

    from fp4_block_scaled_quantizer_amd import binding as B
    from fp4_block_scaled_quantizer_amd import synth

    def gen(cfg, role, extra_copies):
        base = synth.config_tensor(cfg, role).to(dev)
        out = [base]
        for i in range(1, extra_copies):
            # distinct buffers with the same distribution: a cheap bit-level
            # perturbation (sign flip of alternate copies) keeps amax patterns
            out.append(base.neg() if i % 2 else base.clone())
        return out

    L = B.LAYOUT_TILED if layout_name == "tiled" else B.LAYOUT_LINEAR

    def mx_bufs(R, K):
        cs, ss = B.mx_output_shapes(R, K, L)
        return (torch.empty(cs, dtype=torch.uint8, device=dev), torch.empty(ss, dtype=torch.uint8, device=dev))

    # the kernel each MX row producer launches in this layout
    qk = "quant_mx_rows_tiled_kernel" if L == B.LAYOUT_TILED else "quant_mx_rows_kernel"
    ops = []
    if name == "copy":
        # a plain copy kernel of known size: 1 GiB read + 1 GiB written per launch
        n = 1 << 29
        src = [torch.empty(n, dtype=torch.bfloat16, device=dev).fill_(1.0) for _ in range(2)]
        dst = torch.empty(n, dtype=torch.bfloat16, device=dev)
        ops = [("device copy 1 GiB", "elementwise copy", lambda s: dst.copy_(src[s % 2]), 2.0 * 2 * n, "GB/s",
                HBM_PEAK_GBS, "hbm")]
        return {"workload": "plain device copy, 1 GiB in + 1 GiB out"}, ops, 0.0
    if name == "qkv":
        X = gen("qkv", "X", copies)
        W = gen("qkv", "W", copies)
        M, K = X[0].shape
        N = W[0].shape[0]
        cx, sx = mx_bufs(M, K)
        cw, sw = mx_bufs(N, K)
        C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        ops = [
            ("quantize X (MXFP4, RNE)", qk,
             lambda s: B.fp4_quantize_mx(X[s % copies], codes=cx, scales=sx, layout=L),
             M * K * MX_BYTES_PER_ELEM, "GB/s", HBM_PEAK_GBS, "hbm"),
            ("quantize W (MXFP4, RNE)", qk,
             lambda s: B.fp4_quantize_mx(W[s % copies], codes=cw, scales=sw, layout=L),
             N * K * MX_BYTES_PER_ELEM, "GB/s", HBM_PEAK_GBS, "hbm"),
            ("GEMM MXFP4 X W^T -> bf16", "gemm_mx_kernel",
             lambda s: B.fp4_gemm_mx(cx, sx, cw, sw, c=C, layout=L, m=M, n=N),
             2.0 * M * N * K, "TFLOP/s", FP4_PEAK_TFLOPS, "mfma"),
        ]
        cfg = {"workload": "Llama-3-8B QKV forward, MXFP4 RNE", "X": [M, K], "W": [N, K], "gemm_mnk": [M, N, K],
               "out": "bf16", "layout": layout_name, "global_batch_tokens": M, "input_copies": copies}
        return cfg, ops, 2.0 * M * N * K
    if name == "mlp":
        X = gen("mlp_gate_up", "X", copies)
        Wg = gen("mlp_gate_up", "W", copies)
        H = gen("mlp_down", "H", copies)
        Wd = gen("mlp_down", "W", copies)
        M, K1 = X[0].shape
        N1 = Wg[0].shape[0]
        K2 = H[0].shape[1]
        N2 = Wd[0].shape[0]
        bufs = {}

        def q(tag, src, R, K):
            bufs[tag] = mx_bufs(R, K)
            return lambda s: B.fp4_quantize_mx(src[s % copies], codes=bufs[tag][0], scales=bufs[tag][1], layout=L)

        C1 = torch.empty((M, N1), dtype=torch.bfloat16, device=dev)
        C2 = torch.empty((M, N2), dtype=torch.bfloat16, device=dev)
        ops = [
            ("quantize X", qk, q("x", X, M, K1), M * K1 * MX_BYTES_PER_ELEM, "GB/s",
             HBM_PEAK_GBS, "hbm"),
            ("quantize W_gate_up", qk, q("wg", Wg, N1, K1), N1 * K1 * MX_BYTES_PER_ELEM, "GB/s",
             HBM_PEAK_GBS, "hbm"),
            ("GEMM gate/up", "gemm_mx_kernel",
             lambda s: B.fp4_gemm_mx(*bufs["x"], *bufs["wg"], c=C1, layout=L, m=M, n=N1),
             2.0 * M * N1 * K1, "TFLOP/s", FP4_PEAK_TFLOPS, "mfma"),
            ("quantize H", qk, q("h", H, M, K2), M * K2 * MX_BYTES_PER_ELEM, "GB/s",
             HBM_PEAK_GBS, "hbm"),
            ("quantize W_down", qk, q("wd", Wd, N2, K2), N2 * K2 * MX_BYTES_PER_ELEM, "GB/s",
             HBM_PEAK_GBS, "hbm"),
            ("GEMM down", "gemm_mx_kernel", lambda s: B.fp4_gemm_mx(*bufs["h"], *bufs["wd"], c=C2, layout=L, m=M, n=N2),
             2.0 * M * N2 * K2, "TFLOP/s", FP4_PEAK_TFLOPS, "mfma"),
        ]
        cfg = {"workload": "Llama-3-8B MLP forward (gate/up + down), MXFP4 RNE",
               "gemms_mnk": [[M, N1, K1], [M, N2, K2]], "out": "bf16", "layout": layout_name, "input_copies": copies}
        return cfg, ops, 2.0 * M * N1 * K1 + 2.0 * M * N2 * K2
    if name == "dual_x":
        # the forward activation's two operands from one read: X along rows (RNE,
        # for fprop) and the Hadamard X^T along tokens (RNE, kept for wgrad)
        X = gen("qkv", "X", copies)
        T, I = X[0].shape
        mask = synth.sign_mask(synth.HADAMARD_MASK_SEED)
        xr, xc = mx_bufs(T, I), mx_bufs(I, T)
        ops = [("dual-quantize X: rows + Hadamard X^T (RNE)", "quant_mx_cols_kernel",
                lambda s: B.fp4_quantize_mx_dual(X[s % copies], hadamard_cols=True, sign_mask=mask, layout=L,
                                                 codes_rows=xr[0], scales_rows=xr[1], codes_cols=xc[0],
                                                 scales_cols=xc[1]),
                T * I * MX_DUAL_BYTES_PER_ELEM, "GB/s", HBM_PEAK_GBS, "hbm")]
        cfg = {"workload": "Llama-3-8B activation X 8192x4096, MXFP4 rows + Hadamard columns from one read",
               "shape": [T, I], "layout": layout_name, "input_copies": copies}
        return cfg, ops, 0.0
    if name in ("backward", "backward_dual"):
        dual = name == "backward_dual"
        dY = gen("backward", "dY", copies)
        W = gen("backward", "W", copies)
        X = gen("backward", "X", copies)
        T, O = dY[0].shape
        I = W[0].shape[1]
        mask = synth.sign_mask(synth.HADAMARD_MASK_SEED)
        bufs = {}

        def alloc(tag, R, K):
            bufs[tag] = mx_bufs(R, K)

        alloc("dy_r", T, O)
        alloc("wt", I, O)
        alloc("dy_c", O, T)
        alloc("x_c", I, T)
        dX = torch.empty((T, I), dtype=torch.bfloat16, device=dev)
        dW = torch.empty((O, I), dtype=torch.float32, device=dev)
        seed = synth.SR_SEED
        ops = [
            ("quantize dY rows (SR)", qk,
             lambda s: B.fp4_quantize_mx(dY[s % copies], round=B.SR, seed=seed, stream_id=0, codes=bufs["dy_r"][0],
                                         scales=bufs["dy_r"][1], layout=L), T * O * MX_BYTES_PER_ELEM, "GB/s",
             HBM_PEAK_GBS,
             "hbm"),
            ("quantize W^T (cols)", "quant_mx_cols_kernel",
             lambda s: B.fp4_quantize_mx(W[s % copies], axis=B.ALONG_COLS, codes=bufs["wt"][0],
                                         scales=bufs["wt"][1], layout=L), O * I * MX_BYTES_PER_ELEM, "GB/s",
             HBM_PEAK_GBS,
             "hbm"),
            ("GEMM dgrad dY W", "gemm_mx_kernel",
             lambda s: B.fp4_gemm_mx(*bufs["dy_r"], *bufs["wt"], c=dX, layout=L, m=T, n=I),
             2.0 * T * I * O, "TFLOP/s", FP4_PEAK_TFLOPS, "mfma"),
            ("Hadamard-quantize dY^T (SR)", "quant_mx_cols_kernel",
             lambda s: B.fp4_hadamard32_quantize(dY[s % copies], mask, axis=B.ALONG_COLS, round=B.SR, seed=seed,
                                                 stream_id=1, codes=bufs["dy_c"][0], scales=bufs["dy_c"][1],
                                                 layout=L),
             T * O * MX_BYTES_PER_ELEM, "GB/s", HBM_PEAK_GBS, "hbm"),
            ("Hadamard-quantize X^T", "quant_mx_cols_kernel",
             lambda s: B.fp4_hadamard32_quantize(X[s % copies], mask, axis=B.ALONG_COLS, codes=bufs["x_c"][0],
                                                 scales=bufs["x_c"][1], layout=L), T * I * MX_BYTES_PER_ELEM, "GB/s",
             HBM_PEAK_GBS, "hbm"),
            ("GEMM wgrad dY^T X (alpha 1/32)", "gemm_mx_kernel",
             lambda s: B.fp4_gemm_mx(*bufs["dy_c"], *bufs["x_c"], alpha=1.0 / 32, c=dW, layout=L, m=O, n=I),
             2.0 * O * I * T, "TFLOP/s", FP4_PEAK_TFLOPS, "mfma"),
        ]
        if dual:
            # one read of dY for both of its operands (dgrad rows, wgrad Hadamard columns)
            ops = [("dual-quantize dY: rows (SR) + Hadamard dY^T (SR)", "quant_mx_cols_kernel",
                    lambda s: B.fp4_quantize_mx_dual(dY[s % copies], round_rows=B.SR, stream_id_rows=0,
                                                     hadamard_cols=True, sign_mask=mask, round_cols=B.SR,
                                                     stream_id_cols=1, seed=seed, layout=L,
                                                     codes_rows=bufs["dy_r"][0], scales_rows=bufs["dy_r"][1],
                                                     codes_cols=bufs["dy_c"][0], scales_cols=bufs["dy_c"][1]),
                    T * O * MX_DUAL_BYTES_PER_ELEM, "GB/s", HBM_PEAK_GBS, "hbm")] + \
                [op for op in ops if not op[0].startswith(("quantize dY", "Hadamard-quantize dY"))]
        cfg = {"workload": "Llama-3-8B o_proj backward, MXFP4: SR on dY, fixed-sign Hadamard-32 on wgrad" +
                           (", dY's two operands from one read (dual producer)" if dual else ""),
               "dgrad_mnk": [T, I, O], "wgrad_mnk": [O, I, T], "layout": layout_name, "input_copies": copies}
        return cfg, ops, 2.0 * T * I * O * 2
    if name in ("mlp_chain", "mlp_chain_fused"):
        # two MXFP4 GEMMs in a row (MLP up then down shapes, tiled layout):
        # mlp_chain writes H = X W1^T in bf16 and quantizes it for GEMM2;
        # mlp_chain_fused has GEMM1's epilogue write H as GEMM2's MXFP4
        # operand directly (fp4_gemm_mx_quant)
        fused = name == "mlp_chain_fused"
        X = gen("qkv", "X", copies)
        W1 = gen("nvfp4", "W", copies)
        W2 = gen("mlp_down", "W", copies)
        M, K = X[0].shape
        N1, N2 = W1[0].shape[0], W2[0].shape[0]
        bx, bw1, bh, bw2 = mx_bufs(M, K), mx_bufs(N1, K), mx_bufs(M, N1), mx_bufs(N2, N1)
        H = None if fused else torch.empty((M, N1), dtype=torch.bfloat16, device=dev)
        C2 = torch.empty((M, N2), dtype=torch.bfloat16, device=dev)
        ops = [
            ("quantize X", qk, lambda s: B.fp4_quantize_mx(X[s % copies], codes=bx[0], scales=bx[1], layout=L),
             M * K * MX_BYTES_PER_ELEM, "GB/s", HBM_PEAK_GBS, "hbm"),
            ("quantize W1", qk, lambda s: B.fp4_quantize_mx(W1[s % copies], codes=bw1[0], scales=bw1[1], layout=L),
             N1 * K * MX_BYTES_PER_ELEM, "GB/s", HBM_PEAK_GBS, "hbm"),
        ]
        if fused:
            ops.append(("GEMM1 X W1^T -> MXFP4 H (fused quantize)", "gemm_mx_kernel",
                        lambda s: B.fp4_gemm_mx_quant(*bx, *bw1, layout=L, m=M, n=N1, c_layout=L, codes=bh[0],
                                                      scales=bh[1]),
                        2.0 * M * N1 * K, "TFLOP/s", FP4_PEAK_TFLOPS, "mfma"))
        else:
            ops += [("GEMM1 X W1^T -> bf16 H", "gemm_mx_kernel",
                     lambda s: B.fp4_gemm_mx(*bx, *bw1, c=H, layout=L, m=M, n=N1), 2.0 * M * N1 * K, "TFLOP/s",
                     FP4_PEAK_TFLOPS, "mfma"),
                    ("quantize H", qk, lambda s: B.fp4_quantize_mx(H, codes=bh[0], scales=bh[1], layout=L),
                     M * N1 * MX_BYTES_PER_ELEM, "GB/s", HBM_PEAK_GBS, "hbm")]
        ops += [
            ("quantize W2", qk, lambda s: B.fp4_quantize_mx(W2[s % copies], codes=bw2[0], scales=bw2[1], layout=L),
             N2 * N1 * MX_BYTES_PER_ELEM, "GB/s", HBM_PEAK_GBS, "hbm"),
            ("GEMM2 H W2^T -> bf16", "gemm_mx_kernel",
             lambda s: B.fp4_gemm_mx(*bh, *bw2, c=C2, layout=L, m=M, n=N2), 2.0 * M * N2 * N1, "TFLOP/s",
             FP4_PEAK_TFLOPS, "mfma"),
        ]
        cfg = {"workload": "MXFP4, two chained GEMMs (MLP up then down shapes), H " +
                           ("quantized in GEMM1's epilogue" if fused else "written in bf16 and quantized by the producer"),
               "gemm1_mnk": [M, N1, K], "gemm2_mnk": [M, N2, N1], "layout": layout_name, "input_copies": copies}
        return cfg, ops, 2.0 * M * N1 * K + 2.0 * M * N2 * N1
    if name in ("mlp_swiglu", "mlp_swiglu_fused"):
        # the whole MLP forward: gate/up GEMM, SwiGLU, down GEMM (tiled
        # layout; the gate/up weight's rows are taken as gate and up
        # interleaved in groups of 32, the layout the fused epilogue reads).
        # mlp_swiglu writes C in bf16, applies fp4_swiglu_bf16 and quantizes
        # H; mlp_swiglu_fused has GEMM1's epilogue apply SwiGLU and write H
        # as GEMM2's MXFP4 operand (fp4_gemm_mx_swiglu_quant)
        fused = name == "mlp_swiglu_fused"
        X = gen("mlp_gate_up", "X", copies)
        W1 = gen("mlp_gate_up", "W", copies)
        W2 = gen("mlp_down", "W", copies)
        M, K = X[0].shape
        N1, N2 = W1[0].shape[0], W2[0].shape[0]
        F = N1 // 2
        bx, bw1, bh, bw2 = mx_bufs(M, K), mx_bufs(N1, K), mx_bufs(M, F), mx_bufs(N2, F)
        C1 = None if fused else torch.empty((M, N1), dtype=torch.bfloat16, device=dev)
        H = None if fused else torch.empty((M, F), dtype=torch.bfloat16, device=dev)
        C2 = torch.empty((M, N2), dtype=torch.bfloat16, device=dev)
        ops = [
            ("quantize X", qk, lambda s: B.fp4_quantize_mx(X[s % copies], codes=bx[0], scales=bx[1], layout=L),
             M * K * MX_BYTES_PER_ELEM, "GB/s", HBM_PEAK_GBS, "hbm"),
            ("quantize W_gate_up", qk,
             lambda s: B.fp4_quantize_mx(W1[s % copies], codes=bw1[0], scales=bw1[1], layout=L),
             N1 * K * MX_BYTES_PER_ELEM, "GB/s", HBM_PEAK_GBS, "hbm"),
        ]
        if fused:
            ops.append(("GEMM gate/up -> SwiGLU -> MXFP4 H (fused)", "gemm_mx_kernel",
                        lambda s: B.fp4_gemm_mx_swiglu_quant(*bx, *bw1, layout=L, m=M, n=N1, h_layout=L,
                                                             codes=bh[0], scales=bh[1]),
                        2.0 * M * N1 * K, "TFLOP/s", FP4_PEAK_TFLOPS, "mfma"))
        else:
            ops += [("GEMM gate/up -> bf16 C", "gemm_mx_kernel",
                     lambda s: B.fp4_gemm_mx(*bx, *bw1, c=C1, layout=L, m=M, n=N1), 2.0 * M * N1 * K, "TFLOP/s",
                     FP4_PEAK_TFLOPS, "mfma"),
                    ("SwiGLU C -> bf16 H", "swiglu_kernel", lambda s: B.fp4_swiglu_bf16(C1, F, pair=32, h=H),
                     M * F * 6, "GB/s", HBM_PEAK_GBS, "hbm"),
                    ("quantize H", qk, lambda s: B.fp4_quantize_mx(H, codes=bh[0], scales=bh[1], layout=L),
                     M * F * MX_BYTES_PER_ELEM, "GB/s", HBM_PEAK_GBS, "hbm")]
        ops += [
            ("quantize W_down", qk, lambda s: B.fp4_quantize_mx(W2[s % copies], codes=bw2[0], scales=bw2[1], layout=L),
             N2 * F * MX_BYTES_PER_ELEM, "GB/s", HBM_PEAK_GBS, "hbm"),
            ("GEMM down H W_down^T -> bf16", "gemm_mx_kernel",
             lambda s: B.fp4_gemm_mx(*bh, *bw2, c=C2, layout=L, m=M, n=N2), 2.0 * M * N2 * F, "TFLOP/s",
             FP4_PEAK_TFLOPS, "mfma"),
        ]
        cfg = {"workload": "Llama-3-8B MLP forward, MXFP4: gate/up GEMM, SwiGLU, down GEMM; H " +
                           ("made and quantized in the gate/up GEMM's epilogue" if fused
                            else "via bf16 C, the SwiGLU kernel and the producer"),
               "gemm1_mnk": [M, N1, K], "gemm2_mnk": [M, N2, F], "layout": layout_name, "input_copies": copies}
        return cfg, ops, 2.0 * M * N1 * K + 2.0 * M * N2 * F
    if name == "nvfp4_wgrad":
        # the o_proj weight gradient in NVFP4 (per-tile domain): dY^T and X^T
        # quantized along tokens with the fixed-sign Hadamard (SR on dY), then
        # dW = (1/32) dY^T X
        dY = gen("backward", "dY", copies)
        X = gen("backward", "X", copies)
        T, O = dY[0].shape
        I = X[0].shape[1]
        mask = synth.sign_mask(synth.HADAMARD_MASK_SEED)
        D = B.NV_TILE128

        def nvbufs(R, Kc):
            cs, ss = B.nv_output_shapes(R, Kc, L)
            return (torch.empty(cs, dtype=torch.uint8, device=dev),
                    torch.empty(ss, dtype=torch.uint8, device=dev),
                    torch.empty(B.nv_tensor_scale_shape(R, Kc, D), dtype=torch.float32, device=dev))

        bd, bx = nvbufs(O, T), nvbufs(I, T)
        dW = torch.empty((O, I), dtype=torch.float32, device=dev)
        ops = [
            ("Hadamard-quantize dY^T (NVFP4 tile, SR)", "nv_quant_cols_kernel",
             lambda s: B.fp4_quantize_nv(dY[s % copies], D, axis=B.ALONG_COLS, round=B.SR, seed=synth.SR_SEED,
                                         stream_id=1, hadamard_mask=mask, codes=bd[0], scales=bd[1],
                                         tensor_scale=bd[2], layout=L),
             T * O * NV_TILE_BYTES_PER_ELEM, "GB/s", HBM_PEAK_GBS, "hbm"),
            ("Hadamard-quantize X^T (NVFP4 tile)", "nv_quant_cols_kernel",
             lambda s: B.fp4_quantize_nv(X[s % copies], D, axis=B.ALONG_COLS, hadamard_mask=mask, codes=bx[0],
                                         scales=bx[1], tensor_scale=bx[2], layout=L),
             T * I * NV_TILE_BYTES_PER_ELEM, "GB/s", HBM_PEAK_GBS, "hbm"),
            ("GEMM NVFP4 wgrad dY^T X (alpha 1/32)", "gemm_nv_fp16_kernel",
             lambda s: B.fp4_gemm_nv(*bd, *bx, D, alpha=1.0 / 32, c=dW, layout=L, m=O, n=I), 2.0 * O * I * T,
             "TFLOP/s", BF16_PEAK_TFLOPS, "mfma"),
        ]
        cfg = {"workload": "Llama-3-8B o_proj weight gradient, NVFP4 per-128x128-tile domain, fixed-sign Hadamard-32 "
                           "along tokens, SR on dY", "wgrad_mnk": [O, I, T], "layout": layout_name,
               "input_copies": copies}
        return cfg, ops, 2.0 * O * I * T
    if name in ("nvfp4_chain", "nvfp4_chain_2pass"):
        # two NVFP4 GEMMs in a row (Llama-3-8B MLP up and down shapes, global
        # domain): the first GEMM's output is the second's A operand.  In
        # nvfp4_chain the first GEMM also reports max |C1| and C1 is quantized
        # in one pass with it; nvfp4_chain_2pass runs the amax pass instead.
        one_pass = name == "nvfp4_chain"
        X = gen("nvfp4", "X", copies)
        W1 = gen("nvfp4", "W", copies)
        W2 = gen("mlp_down", "W", copies)
        M, K = X[0].shape
        N1 = W1[0].shape[0]
        N2 = W2[0].shape[0]
        G = B.NV_GLOBAL

        def nvbufs(R, Kc):
            return (torch.empty((R, Kc // 2), dtype=torch.uint8, device=dev),
                    torch.empty((R, Kc // 16), dtype=torch.uint8, device=dev),
                    torch.empty((1,), dtype=torch.float32, device=dev),
                    torch.empty((max(1, B.fp4q_nv_workspace_bytes(R, Kc, 0, G)),), dtype=torch.uint8, device=dev))

        bx, bw1, bc1, bw2 = nvbufs(M, K), nvbufs(N1, K), nvbufs(M, N1), nvbufs(N2, N1)
        C1 = torch.empty((M, N1), dtype=torch.bfloat16, device=dev)
        C2 = torch.empty((M, N2), dtype=torch.bfloat16, device=dev)
        amax = torch.zeros((1,), dtype=torch.float32, device=dev)

        def q(src, b, **kw):
            return B.fp4_quantize_nv(src, G, codes=b[0], scales=b[1], tensor_scale=b[2], workspace=b[3], **kw)

        def gemm1(s):
            if one_pass:
                amax.zero_()
                B.fp4_gemm_nv(*bx[:3], *bw1[:3], G, out_dtype=torch.bfloat16, c=C1, c_amax=amax)
            else:
                B.fp4_gemm_nv(*bx[:3], *bw1[:3], G, out_dtype=torch.bfloat16, c=C1)

        ops = [
            ("quantize X (NVFP4)", "nv_quant_global (amax + quantize)", lambda s: q(X[s % copies], bx),
             M * K * NV_GLOBAL_BYTES_PER_ELEM, "GB/s", HBM_PEAK_GBS, "hbm"),
            ("quantize W1 (NVFP4)", "nv_quant_global (amax + quantize)", lambda s: q(W1[s % copies], bw1),
             N1 * K * NV_GLOBAL_BYTES_PER_ELEM, "GB/s", HBM_PEAK_GBS, "hbm"),
            ("GEMM1 X W1^T" + (" (+ max |C1|)" if one_pass else ""), "gemm_nv_fp16_kernel", gemm1,
             2.0 * M * N1 * K, "TFLOP/s", BF16_PEAK_TFLOPS, "mfma"),
            ("quantize C1 (NVFP4, " + ("one pass, GEMM1's amax)" if one_pass else "amax pass + quantize)"),
             "nv_quant_global_kernel" if one_pass else "nv_quant_global (amax + quantize)",
             (lambda s: q(C1, bc1, amax=amax)) if one_pass else (lambda s: q(C1, bc1)),
             M * N1 * (NV_GLOBAL_BYTES_PER_ELEM - (2 if one_pass else 0)), "GB/s", HBM_PEAK_GBS, "hbm"),
            ("quantize W2 (NVFP4)", "nv_quant_global (amax + quantize)", lambda s: q(W2[s % copies], bw2),
             N2 * N1 * NV_GLOBAL_BYTES_PER_ELEM, "GB/s", HBM_PEAK_GBS, "hbm"),
            ("GEMM2 C1 W2^T", "gemm_nv_fp16_kernel",
             lambda s: B.fp4_gemm_nv(*bc1[:3], *bw2[:3], G, out_dtype=torch.bfloat16, c=C2),
             2.0 * M * N2 * N1, "TFLOP/s", BF16_PEAK_TFLOPS, "mfma"),
        ]
        cfg = {"workload": "NVFP4 global, two chained GEMMs (MLP up then down shapes), C1 quantized " +
                           ("in one pass with GEMM1's fused amax" if one_pass else "with its own amax pass"),
               "gemm1_mnk": [M, N1, K], "gemm2_mnk": [M, N2, N1], "out": "bf16", "input_copies": copies}
        return cfg, ops, 2.0 * M * N1 * K + 2.0 * M * N2 * N1
    # NVFP4
    domain = B.NV_GLOBAL if name == "nvfp4_global" else B.NV_TILE128
    X = gen("nvfp4", "X", copies)
    W = gen("nvfp4", "W", copies)
    M, K = X[0].shape
    N = W[0].shape[0]
    bufs = {}

    def qnv(tag, src, R):
        ts_shape = B.nv_tensor_scale_shape(R, K, domain)
        cs, ss = B.nv_output_shapes(R, K, L)
        bufs[tag] = (torch.empty(cs, dtype=torch.uint8, device=dev),
                     torch.empty(ss, dtype=torch.uint8, device=dev),
                     torch.empty(ts_shape, dtype=torch.float32, device=dev),
                     torch.empty((max(1, B.fp4q_nv_workspace_bytes(R, K, 0, domain)),), dtype=torch.uint8,
                                 device=dev))
        b = bufs[tag]
        return lambda s: B.fp4_quantize_nv(src[s % copies], domain, codes=b[0], scales=b[1], tensor_scale=b[2],
                                           workspace=b[3] if domain == B.NV_GLOBAL else None, layout=L)

    C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    bpe = NV_GLOBAL_BYTES_PER_ELEM if domain == B.NV_GLOBAL else NV_TILE_BYTES_PER_ELEM
    kname = "nv_quant_global (amax + quantize)" if domain == B.NV_GLOBAL else "nv_quant_tile_kernel"
    ops = [
        ("quantize X (NVFP4)", kname, qnv("x", X, M), M * K * bpe, "GB/s", HBM_PEAK_GBS, "hbm"),
        ("quantize W (NVFP4)", kname, qnv("w", W, N), N * K * bpe, "GB/s", HBM_PEAK_GBS, "hbm"),
        ("GEMM NVFP4 (fp16 MFMA)", "gemm_nv_fp16_kernel",
         lambda s: B.fp4_gemm_nv(bufs["x"][0], bufs["x"][1], bufs["x"][2], bufs["w"][0], bufs["w"][1], bufs["w"][2],
                                 domain, c=C, layout=L, m=M, n=N), 2.0 * M * N * K, "TFLOP/s", BF16_PEAK_TFLOPS,
         "mfma"),
    ]
    cfg = {"workload": f"NVFP4 {'global' if domain == B.NV_GLOBAL else 'per-128x128-tile'} tensor scale",
           "gemm_mnk": [M, N, K], "out": "bf16", "layout": layout_name, "input_copies": copies}
    return cfg, ops, 2.0 * M * N * K


def read_traffic(kernel, workload):
    """HBM bytes per launch from a committed rocprofv3 counter summary, if one
    exists for this kernel and workload and still matches the kernel source
    (`source` lists the files, comma-separated)."""
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    src = vals.get("source")
    if not src or "traffic_bytes" not in vals:
        return None
    if source_hash(src.split(",")) != vals.get("source_sha256_16"):
        return None  # kernel changed since the counters were taken
    return float(vals["traffic_bytes"])


def source_hash(paths):
    """SHA-256 (first 16 hex digits) of the kernel's source files, concatenated
    in the order given, with comments, blank lines and indentation removed
    (a change to the comments does not invalidate the counters)."""
    import hashlib
    import re

    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p.strip())) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update("\n".join(ln.strip() for ln in text.splitlines() if ln.strip()).encode())
    return h.hexdigest()[:16]


def _oracle_quantize_rows(oracle, x, threads):
    """oracle.quantize_mx of bf16 bits x along rows, the rows split over
    `threads` host threads (the oracle's C releases the GIL; rows are
    independent, so the result is the single-threaded one)."""
    import concurrent.futures as cf

    import numpy as np

    if threads <= 1 or x.shape[0] < 2 * threads:
        return oracle.quantize_mx(x)
    parts = np.array_split(np.arange(x.shape[0]), threads)
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        res = list(ex.map(lambda ix: oracle.quantize_mx(x[ix[0]:ix[-1] + 1]), [p for p in parts if p.size]))
    return np.concatenate([r[0] for r in res]), np.concatenate([r[1] for r in res])


def cpu_baseline(workload):
    """The oracle, as it stands, on a bounded slice of one step of the
    workload (MXFP4 forward workloads): every operand cut to half of its
    rows (tokens and output features alike), so each GEMM does 1/4 of its
    flops, timed once on one thread and once on every host core; value = the
    slice's GEMM flops / its time, in TFLOP/s."""
    if workload not in ("qkv", "mlp"):
        return None
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    from fp4_block_scaled_quantizer_amd import synth

    frac = 2
    if workload == "qkv":
        parts = [("qkv", "X", "qkv", "W")]
    else:
        parts = [("mlp_gate_up", "X", "mlp_gate_up", "W"), ("mlp_down", "H", "mlp_down", "W")]
    slices = []
    flops = 0.0
    for ca, ra, cb, rb in parts:
        a = synth.bf16_bits(synth.config_tensor(ca, ra))
        b = synth.bf16_bits(synth.config_tensor(cb, rb))
        a = np.ascontiguousarray(a[:a.shape[0] // frac])
        b = np.ascontiguousarray(b[:b.shape[0] // frac])
        slices.append((a, b))
        flops += 2.0 * a.shape[0] * b.shape[0] * a.shape[1]
    ncores = os.cpu_count() or 1

    def run(threads):
        with threadpool_limits(limits=threads):
            t0 = time.perf_counter()
            for a, b in slices:
                qa = _oracle_quantize_rows(oracle, a, threads)
                qb = _oracle_quantize_rows(oracle, b, threads)
                oracle.gemm_ref(oracle.dequant_mx(*qa), oracle.dequant_mx(*qb), weights=False)
            return time.perf_counter() - t0

    t1 = run(1)
    tn = run(ncores)
    shapes = [[int(a.shape[0]), int(b.shape[0]), int(a.shape[1])] for a, b in slices]
    return {"value": round(flops / tn / 1e12, 4), "unit": "TFLOP/s", "cores": ncores, "kind": "oracle",
            "seconds": round(tn, 3), "single_thread": {"value": round(flops / t1 / 1e12, 4), "seconds": round(t1, 3),
                                                         "cores": 1},
            "sample": f"half of every operand's rows (GEMMs M x N x K = {shapes}, {flops / 1e9:.0f} GFLOP): "
                      "oracle.quantize_mx of both operands (C, rows split over the threads), dequantize, float64 "
                      "numpy matmul; value = the slice's GEMM flops / its time",
            "host_cpu": platform.processor() or platform.machine(), "host_nproc": ncores}


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: --gpus {args.gpus} / WORLD_SIZE {world} is not supported "
              "(this build runs the FP4 producer and GEMM on a single MI355X)", file=sys.stderr)
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    cfg, ops, step_flops = build_workload(args.workload, dev, args.copies, args.layout)
    stream = torch.cuda.current_stream()

    # W warmup steps, then more until the GPU has run for WARM_S seconds: the
    # first ~0.1 s of back-to-back work runs at lower clocks.
    t0 = time.perf_counter()
    s = 0
    while s < args.warmup or time.perf_counter() - t0 < WARM_S:
        for op in ops:
            op[2](s)
        s += 1
        if s % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()

    def ev():
        return torch.cuda.Event(enable_timing=True)

    nops = len(ops)
    # Per-op durations in the step: for each op, K steps with a HIP event pair
    # around that op's launch only.
    op_ms = []
    for i in range(nops):
        evs = [(ev(), ev()) for _ in range(args.steps)]
        for s in range(args.steps):
            for j, op in enumerate(ops):
                if j == i:
                    evs[s][0].record(stream)
                op[2](s)
                if j == i:
                    evs[s][1].record(stream)
        torch.cuda.synchronize()
        op_ms.append([e0.elapsed_time(e1) for e0, e1 in evs])

    # Each op also as a batch of back-to-back launches (no markers at all),
    # for the short producers where even two markers per step matter.
    batch = 20
    batched_ms = []
    for i, op in enumerate(ops):
        b0, b1 = ev(), ev()
        b0.record(stream)
        for r in range(batch):
            op[2](r)
        b1.record(stream)
        torch.cuda.synchronize()
        batched_ms.append(b0.elapsed_time(b1) / batch)

    # The dominant kernel: the kernel name with the most time per step.
    per_kernel = {}
    for i, op in enumerate(ops):
        per_kernel[op[1]] = per_kernel.get(op[1], 0.0) + sum(op_ms[i]) / len(op_ms[i])
    dom_name = max(per_kernel, key=per_kernel.get)
    dom_ops = [i for i, op in enumerate(ops) if op[1] == dom_name]

    # Timed region: K steps launched back to back.
    t_start, t_end = ev(), ev()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for s in range(args.steps):
        for op in ops:
            op[2](s)
    t_end.record(stream)
    enqueue = time.perf_counter() - wall0
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    gpu_ms = t_start.elapsed_time(t_end)
    ms_per_step = gpu_ms / args.steps

    # Roofline pass: the same K steps with an event pair around every launch
    # of the dominant kernel (on the stream it is launched on).
    dom_ev = []
    r_start, r_end = ev(), ev()
    r_start.record(stream)
    for s in range(args.steps):
        for j, op in enumerate(ops):
            if j in dom_ops:
                e0, e1 = ev(), ev()
                e0.record(stream)
                op[2](s)
                e1.record(stream)
                dom_ev.append((j, e0, e1))
            else:
                op[2](s)
    r_end.record(stream)
    torch.cuda.synchronize()
    dom_ms = [(j, e0.elapsed_time(e1)) for j, e0, e1 in dom_ev]
    ms_per_step_marked = r_start.elapsed_time(r_end) / args.steps

    kernels = []
    for i, (label, kname, _, amount, unit, peak, bound) in enumerate(ops):
        durs = op_ms[i]
        avg_ms = sum(durs) / len(durs)
        use_ms = avg_ms if avg_ms > 0.1 else batched_ms[i]
        achieved = amount / (use_ms * 1e-3) / (1e9 if unit == "GB/s" else 1e12)
        kernels.append({"op": label, "kernel": kname, "avg_us": round(avg_ms * 1e3, 2),
                        "avg_us_batched": round(batched_ms[i] * 1e3, 2), "min_us": round(min(durs) * 1e3, 2),
                        "achieved": round(achieved, 1), "unit": unit, "peak": peak,
                        "frac": round(achieved / peak, 4), "bound": bound, "algorithmic": amount})
    d0 = ops[dom_ops[0]]
    unit, peak, bound = d0[4], d0[5], d0[6]
    amount_per_launch = sum(ops[j][3] for j in dom_ops) / len(dom_ops)
    avg_launch_ms = sum(t for _, t in dom_ms) / len(dom_ms)
    achieved = amount_per_launch / (avg_launch_ms * 1e-3) / (1e9 if unit == "GB/s" else 1e12)
    roofline = {"bound": bound, "achieved": round(achieved, 1), "peak": peak, "unit": unit,
                "frac": round(achieved / peak, 4), "traffic": read_traffic(dom_name, args.workload),
                "kernel": dom_name, "ops": [ops[j][0] for j in dom_ops],
                "launches_per_step": len(dom_ops), "avg_launch_us": round(avg_launch_ms * 1e3, 2),
                "algorithmic_per_launch": amount_per_launch,
                "avg_launch_us_by_op": {ops[j][0]: round(1e3 * sum(t for jj, t in dom_ms if jj == j) /
                                                         max(1, sum(1 for jj, _ in dom_ms if jj == j)), 2)
                                        for j in dom_ops}}
    # workloads without a GEMM (a producer alone, the copy calibration) report
    # the dominant kernel's rate
    value = step_flops / (ms_per_step * 1e-3) / 1e12 if step_flops else achieved
    out = {
        "metric": "quantize+FP4 GEMM TFLOP/s (Llama-3-8B shapes)" if step_flops else f"{d0[0]} {unit}",
        "value": round(value, 1),
        "unit": "TFLOP/s" if step_flops else unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp16(e2m1*e4m3) -> f32" if "nvfp4" in args.workload else
                  "e2m1 x e2m1 -> f32 accumulate" if step_flops else
                  "bf16" if args.workload == "copy" else "bf16 -> e2m1 + e8m0"),
        "data": "synthetic",
        "config": cfg,
        "roofline": roofline,
        "kernels": kernels,
        "ms_per_step_roofline_pass": round(ms_per_step_marked, 5),
        "wall_s_timed": round(wall, 4),
        "host_enqueue_us_per_step": round(enqueue / args.steps * 1e6, 1),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.workload)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
