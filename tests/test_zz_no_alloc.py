"""fp4_quantize_nv_noalloc (the library's own 4 KiB workspace instead of a
caller's) against fp4_quantize_nv with a caller workspace, through the C ABI:
byte for byte, both axes and domains, RNE and SR, two calls in a row with the
second on a smaller operand (the shared buffer keeps the first call's
partial maxima, which must not leak into the second), and a third call after
a different-shaped one on the other axis."""
import numpy as np
import pytest
import torch

from tests.gpu_common import B, announce, assert_bytes_equal, device, np_u8, oracle, synth

pytestmark = pytest.mark.gpu


def both(x, domain, axis, rnd):
    ref = B.fp4_quantize_nv(x, domain, axis=axis, round=rnd, seed=7, stream_id=1)
    got = B.fp4_quantize_nv_noalloc(x, domain, axis=axis, round=rnd, seed=7, stream_id=1)
    return ref, got


def same(ref, got, what):
    assert_bytes_equal(np_u8(got[0]), np_u8(ref[0]), f"{what} codes")
    assert_bytes_equal(np_u8(got[1]), np_u8(ref[1]), f"{what} scales")
    assert np.array_equal(got[2].cpu().numpy().view(np.uint32), ref[2].cpu().numpy().view(np.uint32)), what


@pytest.mark.parametrize("domain", [0, 1])
@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("rnd", [0, 1])
def test_noalloc_equals_workspace_call_twice(domain, axis, rnd):
    dev = device()
    announce(f"nv noalloc domain={domain} axis={axis} round={rnd}")
    # first call: a large operand (1024 partial maxima in the global domain),
    # one huge outlier so that its amax would dominate a stale partial
    big = synth.activation(2048, 4096, 91)
    big[5, 7] = 3.0e4
    ref1, got1 = both(big.to(dev), domain, axis, rnd)
    # second call, smaller and with a much smaller amax
    small = synth.weight(384, 512, 92)
    ref2, got2 = both(small.to(dev), domain, axis, rnd)
    torch.cuda.synchronize()
    same(ref1, got1, "first call")
    same(ref2, got2, "second call")
    # and the second call against the oracle
    oc, os_, ots = oracle.quantize_nv(synth.bf16_bits(small), axis=axis, sr=bool(rnd), seed=7, stream=1,
                                      domain=domain)
    assert_bytes_equal(np_u8(got2[0]), oc, "oracle codes")
    assert_bytes_equal(np_u8(got2[1]), os_, "oracle scales")
    assert np.array_equal(got2[2].cpu().numpy().view(np.uint32), ots.view(np.uint32))


def test_noalloc_allocates_nothing_and_errors():
    dev = device()
    announce("nv noalloc: no allocation during the call; argument errors")
    x = synth.activation(256, 1024, 93).to(dev)
    codes = torch.empty((256, 512), dtype=torch.uint8, device=dev)
    scales = torch.empty((256, 64), dtype=torch.uint8, device=dev)
    ts = torch.empty((1,), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    L = B.lib()
    stream = torch.cuda.current_stream().cuda_stream
    before = torch.cuda.memory_stats().get("allocation.all.allocated", 0)
    st = L.fp4_quantize_nv_noalloc(x.data_ptr(), 256, 1024, 1024, 0, 0, 0, 0, 0, codes.data_ptr(),
                                   scales.data_ptr(), ts.data_ptr(), 0, stream)
    torch.cuda.synchronize()
    assert st == B.OK
    assert torch.cuda.memory_stats().get("allocation.all.allocated", 0) == before
    ref = B.fp4_quantize_nv(x, 0)
    torch.cuda.synchronize()
    assert torch.equal(codes, ref[0]) and torch.equal(scales, ref[1]) and torch.equal(ts, ref[2])
    # the same argument checks as fp4_quantize_nv
    assert L.fp4_quantize_nv_noalloc(x.data_ptr(), 256, 1000, 1024, 0, 0, 0, 0, 0, codes.data_ptr(),
                                     scales.data_ptr(), ts.data_ptr(), 0, stream) == B.ESHAPE
    # the tiled layout needs K % 128 == 0 (here K = 1000 is rejected before any launch)
    assert L.fp4_quantize_nv_noalloc(x.data_ptr(), 256, 1000, 1024, 0, 0, 0, 0, 0, codes.data_ptr(),
                                     scales.data_ptr(), ts.data_ptr(), 1, stream) == B.ESHAPE
    assert L.fp4_quantize_nv_noalloc(None, 256, 1024, 1024, 0, 0, 0, 0, 0, codes.data_ptr(),
                                     scales.data_ptr(), ts.data_ptr(), 0, stream) == B.EINVAL
