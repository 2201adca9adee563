"""Stress canary for the persistent GEMM kernels.

Every GEMM launch here is persistent: a grid of at most one (or two)
workgroups per compute unit walks the output tiles, and each workgroup
starts loading its next tile while it stores the last. The stress hook
(macaq_debug_limit_workgroups) caps the grid, so each workgroup walks many
more tiles, in another order and another interleaving with the others. Each
output tile is still computed whole, by one workgroup, in a fixed order, so
the outputs must be bit-identical to those of the planned grid; a
difference would expose a race between consecutive tiles of one workgroup
(LDS or registers reused before the previous tile is done with them).
Covered: the wide prefill kernel, the 128 x 256 prefill kernel, split-K
decode, the grouped layer and the MoE block (gate/up with its SwiGLU
epilogue, down, combine).
"""
import numpy as np
import pytest
import torch

from mxfp4_w4a4_post_amd import binding, inputs
from parity_util import log

pytestmark = pytest.mark.gpu

CAPS = [1, 5, 37, 200]


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    binding.load_library()
    return torch.device("cuda:0")


@pytest.fixture
def uncapped():
    binding.limit_workgroups(0)
    yield
    binding.limit_workgroups(0)


def _bf16(shape, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(*shape, generator=g) * scale).to(torch.bfloat16)


def _layer(N, K, b, dev, seed):
    w = _bf16((N, K), seed, 0.02).to(dev)
    xcal = _bf16((64, K), seed + 1).to(dev)
    return binding.prepare_layer(w, xcal, b)


def _compare_under_caps(run, what):
    ref = run()
    torch.cuda.synchronize()
    for cap in CAPS:
        binding.limit_workgroups(cap)
        got = run()
        torch.cuda.synchronize()
        binding.limit_workgroups(0)
        same = all(torch.equal(g, r) for g, r in zip(got, ref)) if isinstance(ref, tuple) else torch.equal(got, ref)
        assert same, "%s: output changed with the grid capped at %d workgroups" % (what, cap)
    log("%s: bit-identical with the grid capped at %s workgroups" % (what, CAPS))


@pytest.mark.parametrize("M,N,K,b,what", [
    (4096, 4096, 1024, 32, "wide 256 x 256 tiles"),
    (1000, 3000, 1024, 64, "128 x 256 tiles, ragged"),
    (16, 4096, 8192, 32, "decode, split-K"),
    (64, 5120, 25600, 32, "decode, split-K, large K"),
])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_linear_stress(dev, uncapped, M, N, K, b, what, out_dtype):
    log("stress linear %s M=%d N=%d K=%d b=%d %s" % (what, M, N, K, b, out_dtype))
    lay = _layer(N, K, b, dev, M + N)
    x = _bf16((M, K), 7 + M).to(dev)
    _compare_under_caps(lambda: lay(x, out_dtype=out_dtype), "linear " + what)


def test_grouped_stress(dev, uncapped):
    E, T, K, N, b = 8, 3000, 1024, 1536, 32
    log("stress grouped T=%d E=%d K=%d N=%d" % (T, E, K, N))
    rng = np.random.default_rng(3)
    cuts = np.sort(rng.integers(0, T, size=E - 1))
    cuts[2] = cuts[1]  # an empty expert
    off = torch.from_numpy(np.concatenate([[0], cuts, [T]]).astype(np.int32)).to(dev)
    w = binding.empty_grouped_weights(E, N, K, dev)
    a = torch.empty(E, K, dtype=torch.float32, device=dev)
    for e in range(E):
        lay = _layer(N, K, b, dev, 100 + e)
        ex = binding.expert(w, e)
        ex.codes.copy_(lay.w.codes)
        ex.scales.copy_(lay.w.scales)
        a[e] = lay.a
    x = _bf16((T, K), 11).to(dev)
    _compare_under_caps(lambda: binding.linear_grouped(x, off, a, b, w), "grouped")


def test_moe_block_stress(dev, uncapped):
    c = inputs.moe_block_case(tokens=512, experts=16, top_k=4, hidden=1024, ffn=512, b=32)
    log("stress MoE block T=%d E=%d k=%d H=%d F=%d" % (c.T, c.E, c.k, c.H, c.F))
    lay = binding.prepare_moe(c.w_gate.to(dev), c.w_up.to(dev), c.w_dn.to(dev), c.xcal_gu.to(dev),
                              c.xcal_dn.to(dev), c.b)
    ids = torch.from_numpy(c.ids).to(dev)
    w = torch.from_numpy(c.w).to(dev)
    x = c.x.to(dev)

    def run():
        off, tok, pos = binding.moe_route(ids, c.E)
        dn = binding.moe_gate_up(x, c.k, tok, off, lay.a_gu, c.b, lay.wgu, lay.a_dn)
        return dn.codes.clone(), dn.scales.clone(), lay(x, ids, w, out_dtype=torch.float32)

    _compare_under_caps(run, "MoE block")
