"""macaq_linear_noalloc (no workspace: the library's own scratch) against
macaq_linear (caller's workspace) on the same inputs, through the C ABI.
Both run the same kernels, so the outputs must be the same bits: two calls
in a row, the second on a smaller input (the scratch keeps the first call's
contents), then a decode shape whose split-K partial sums also live in the
scratch, and the call captured in a HIP graph and replayed with other calls
in between. A size beyond the scratch is refused before anything is
enqueued."""
import ctypes

import numpy as np
import pytest
import torch

from mxfp4_w4a4_post_amd import binding, inputs

pytestmark = pytest.mark.gpu

EWORKSPACE = 3


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    binding.load_library()
    return torch.device("cuda:0")


def _layer(case, dev):
    a, r = binding.make_multipliers(binding.calibrate(case.xcal.to(dev)), case.b)
    return a, binding.prepare_weights(case.w.to(dev), r, case.b)


def _both(case, dev, out_dtype):
    x = case.x.to(dev)
    a, pw = _layer(case, dev)
    y_ref = binding.linear(x, a, case.b, pw, out_dtype=out_dtype)
    y = torch.full_like(y_ref, float("nan"))
    binding.linear_noalloc(x, a, case.b, pw, out=y)
    torch.cuda.synchronize()
    return y, y_ref


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_noalloc_equals_linear_two_calls(dev, out_dtype):
    big = inputs.linear_case(2, 1)                          # M=2048, K=4096, N=14336 (wide tiles)
    small = inputs.linear_case(1, 0, M=300, K=1024, N=600)  # ragged, after the big call
    for case in (big, small):
        print("[noalloc] %s %s" % (case.name, out_dtype), flush=True)
        y, y_ref = _both(case, dev, out_dtype)
        assert torch.equal(y, y_ref), case.name


def test_noalloc_decode_split_k(dev):
    for M in (64, 8):
        case = inputs.linear_case(3, 1, M=M)  # K=25600, N=5120: split K, partial sums in the scratch
        print("[noalloc] %s" % case.name, flush=True)
        y, y_ref = _both(case, dev, torch.bfloat16)
        assert torch.equal(y, y_ref), case.name


def test_noalloc_in_a_graph(dev):
    """A caller that captures its work in a HIP graph (the kind of caller the
    entry point is for): the captured call, replayed with other no-allocation
    calls in between that overwrite the scratch, equals the eager call every
    time (each call writes what it reads from the scratch before reading it)."""
    case = inputs.linear_case(3, 1, M=64)          # K=25600, N=5120: split-K partials in the scratch too
    other = inputs.linear_case(1, 0, M=300, K=1024, N=600)
    print("[noalloc] graph %s, between replays %s" % (case.name, other.name), flush=True)
    x, xo = case.x.to(dev), other.x.to(dev)
    a, pw = _layer(case, dev)
    ao, pwo = _layer(other, dev)
    y_ref = binding.linear(x, a, case.b, pw, out_dtype=torch.bfloat16)
    y = torch.empty_like(y_ref)
    yo = torch.empty(other.M, other.N, dtype=torch.bfloat16, device=dev)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        binding.linear_noalloc(x, a, case.b, pw, out=y)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        binding.linear_noalloc(x, a, case.b, pw, out=y)
    for i in range(3):
        y.fill_(float("nan"))
        binding.linear_noalloc(xo, ao, other.b, pwo, out=yo)   # overwrites the scratch
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_ref), "replay %d differs from the eager call" % i


def test_noalloc_refuses_beyond_scratch(dev):
    lib = binding.load_library()
    M, K, N = 16384, 28672, 8192
    need = lib.macaq_linear_workspace_size(M, K, N)
    assert need > binding.NOALLOC_SCRATCH_BYTES
    fake = 0x10000  # aligned, never dereferenced: the size check comes before anything is enqueued
    st = lib.macaq_linear_noalloc(fake, M, K, K, None, 0, fake, fake, N, fake, 0, N, None)
    assert st == EWORKSPACE
    assert "scratch" in lib.macaq_last_error().decode()
