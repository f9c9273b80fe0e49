"""Every call enqueues on the caller's stream: a producer and a GEMM on a
side stream see the work queued before them on that stream, and a QKV-like
step (quantize X, quantize W, GEMM) captured into a HIP graph replays
correctly several times, with eager work between the replays, against the
eager result of each replay's inputs."""
import numpy as np
import pytest
import torch

from tests.gpu_common import B, announce, assert_bytes_equal, device, np_u8, oracle, synth

pytestmark = pytest.mark.gpu


def test_calls_follow_the_caller_stream():
    dev = device()
    announce("side stream ordering")
    M, N, K = 512, 384, 1024
    x0 = synth.activation(M, K, 601)
    x1 = synth.activation(M, K, 602)
    w = synth.weight(N, K, 603).to(dev)
    x = x0.to(dev)
    x1d = x1.to(dev)
    big = torch.randn((4096, 4096), device=dev)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        # a long kernel, then the new input, then the library calls: all on s
        for _ in range(4):
            big = big @ big * 1e-3
        x.copy_(x1d)
        codes, scales = B.fp4_quantize_mx(x, stream=s)
        bw = B.fp4_quantize_mx(w, stream=s)
        c = B.fp4_gemm_mx(codes, scales, *bw, stream=s)
    s.synchronize()
    oc, os_ = oracle.quantize_mx(synth.bf16_bits(x1))
    assert_bytes_equal(np_u8(codes), oc, "codes of the input written just before on the same stream")
    assert_bytes_equal(np_u8(scales), os_, "scales")
    ref = B.fp4_gemm_mx(torch.from_numpy(oc).to(dev), torch.from_numpy(os_).to(dev), *bw)
    torch.cuda.synchronize()
    assert torch.equal(c, ref)


def test_graph_capture_and_replay():
    dev = device()
    announce("graph capture of quantize X, quantize W, GEMM")
    M, N, K = 1024, 768, 2048
    L = B.LAYOUT_TILED
    x = synth.activation(M, K, 611).to(dev)
    w = synth.weight(N, K, 612).to(dev)
    cx, sx = B.mx_output_shapes(M, K, L)
    cw, sw = B.mx_output_shapes(N, K, L)
    bx = (torch.empty(cx, dtype=torch.uint8, device=dev), torch.empty(sx, dtype=torch.uint8, device=dev))
    bw = (torch.empty(cw, dtype=torch.uint8, device=dev), torch.empty(sw, dtype=torch.uint8, device=dev))
    c = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    def step():
        B.fp4_quantize_mx(x, codes=bx[0], scales=bx[1], layout=L)
        B.fp4_quantize_mx(w, codes=bw[0], scales=bw[1], layout=L)
        B.fp4_gemm_mx(*bx, *bw, c=c, layout=L, m=M, n=N)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        # new inputs written eagerly between replays
        x.copy_(synth.activation(M, K, 620 + rep).to(dev))
        w.copy_(synth.weight(N, K, 630 + rep).to(dev))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = c.clone()
        step()  # the same step, eagerly
        torch.cuda.synchronize()
        assert torch.equal(got, c), f"replay {rep} differs from the eager step"
        assert bool(torch.isfinite(got.float()).all())
