"""Streaming preparation of a layer stack gives exactly what layer-by-layer
preparation gives (multipliers and packed weights bit for bit), with device
memory bounded by two layers whatever the stack's depth."""
import numpy as np
import pytest
import torch

import oracle
from mxfp4_w4a4_post_amd import binding, inputs, streaming
from parity_util import bits, log, packed_to_row_major

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    binding.load_library()
    return torch.device("cuda:0")


def test_streamed_stack_matches_oracle(dev):
    shapes = [(256, 256), (96, 512), (320, 256), (64, 768), (256, 256)]
    layers = []
    for i, (N, K) in enumerate(shapes):
        c = inputs.linear_case(1, 0, M=1, K=K, N=N)
        layers.append(streaming.HostLayer(c.w.pin_memory(), c.xcal.pin_memory()))
    log("streamed stack of %d layers" % len(layers))
    prep = streaming.StreamingPreparer(dev, max(n for n, _ in shapes), max(k for _, k in shapes), inputs.CALIB_ROWS)
    out = prep.run(layers, 32)
    for L, P in zip(layers, out):
        a_o, r_o = oracle.multipliers(oracle.calibrate(bits(L.xcal)), 32)
        c_o, s_o = oracle.prepare_weights(bits(L.w), r_o, 32)
        assert np.array_equal(P.a.numpy().view(np.uint32), a_o.view(np.uint32))
        assert np.array_equal(P.r.numpy().view(np.uint32), r_o.view(np.uint32))
        c_g, s_g = packed_to_row_major(binding.Packed(P.codes, P.scales, P.N, P.K))
        assert np.array_equal(c_g, c_o) and np.array_equal(s_g, s_o)


def test_streamed_memory_does_not_grow_with_depth(dev):
    N, K = 1024, 2048
    gen = torch.Generator(device=dev)
    gen.manual_seed(1)
    layers = [streaming.HostLayer((torch.randn(N, K, generator=gen, device=dev) * 0.02).to(torch.bfloat16).cpu()
                                  .pin_memory(),
                                  torch.randn(64, K, generator=gen, device=dev).to(torch.bfloat16).cpu().pin_memory())
              for _ in range(12)]
    torch.cuda.synchronize()
    prep = streaming.StreamingPreparer(dev, N, K, 64)
    prep.run(layers[:2], 32)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats(dev)
    base = torch.cuda.memory_allocated(dev)
    prep.run(layers[:3], 32)
    peak3 = torch.cuda.max_memory_allocated(dev) - base
    torch.cuda.reset_peak_memory_stats(dev)
    prep.run(layers, 32)
    peak12 = torch.cuda.max_memory_allocated(dev) - base
    log("peak extra device bytes: 3 layers %d, 12 layers %d (one layer's weights: %d)" % (peak3, peak12, 2 * N * K))
    assert peak12 <= peak3 + 65536
