"""Flip-Refinement on the GPU vs the CPU oracle, through the C ABI.

Every decision is taken in fp64 with sums in index order on both sides, so
the Hessian, the refined codes and the move counts are compared bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
from mxfp4_w4a4_post_amd import binding, inputs
from parity_util import bits, log, packed_to_row_major, row_major_to_gemm_layout

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    binding.load_library()
    return torch.device("cuda:0")


def _rows(R, K, seed, outliers=2, factor=20.0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((R, K)).astype(np.float32)
    x[:, rng.choice(K, outliers, replace=False)] *= factor
    return inputs.to_bf16(x)


@pytest.mark.parametrize("R,K,b", [(64, 256, 32), (48, 512, 64), (40, 1024, 128), (33, 320, 0), (64, 4096, 32)])
def test_hessian_bit_exact(dev, R, K, b):
    log("hessian R=%d K=%d b=%d" % (R, K, b))
    x = _rows(R, K, R + K + b)
    xb = bits(x)
    s = oracle.calibrate(xb)
    a, _ = oracle.multipliers(s, b)
    H_o = oracle.hessian(xb, a if b else None, b)
    H_g = binding.hessian(x.to(dev), torch.from_numpy(a).to(dev) if b else None, b)
    torch.cuda.synchronize()
    assert np.array_equal(H_g.cpu().numpy().view(np.uint64), H_o.view(np.uint64))


@pytest.mark.parametrize("R,K,b,factor", [(129, 1024, 0, 1e4), (70, 2048, 32, 3e3)])
def test_hessian_bit_exact_wide_range(dev, R, K, b, factor):
    """Channels spanning four decades and a ragged row count, so the fp64
    sums cancel and round at very different magnitudes: the matrix-core
    Hessian must still equal the oracle's sequential fused sums bit for bit."""
    log("hessian wide range R=%d K=%d b=%d factor=%g" % (R, K, b, factor))
    rng = np.random.default_rng(R * K)
    x = rng.standard_normal((R, K)).astype(np.float32)
    x *= np.exp(rng.uniform(0.0, np.log(factor), K)).astype(np.float32)
    x[:, ::7] *= -1.0
    xt = inputs.to_bf16(x)
    xb = bits(xt)
    s = oracle.calibrate(xb)
    a, _ = oracle.multipliers(s, b)
    H_o = oracle.hessian(xb, a if b else None, b)
    H_g = binding.hessian(xt.to(dev), torch.from_numpy(a).to(dev) if b else None, b)
    torch.cuda.synchronize()
    assert np.array_equal(H_g.cpu().numpy().view(np.uint64), H_o.view(np.uint64))


def _refine_case(dev, N, K, b, cap, f32=False, seed=0, R=96, H_np=None):
    rng = np.random.default_rng(seed)
    x = _rows(R, K, seed + 1)
    xb = bits(x)
    s = oracle.calibrate(xb)
    a, r = oracle.multipliers(s, b)
    w32 = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    w = torch.from_numpy(w32) if f32 else inputs.to_bf16(w32)
    wn = w.numpy() if f32 else bits(w)
    rr = r if b else None
    codes, scales = oracle.prepare_weights(wn, rr, b)
    H = H_np if H_np is not None else oracle.hessian(xb, a if b else None, b)
    out_o, flips_o = oracle.flip_refine(wn, rr, b, H, cap, codes, scales)
    c_t, s_t = row_major_to_gemm_layout(codes, scales)
    packed = binding.Packed(torch.from_numpy(c_t).to(dev), torch.from_numpy(s_t).to(dev), N, K)
    flips = binding.flip_refine(w.to(dev), torch.from_numpy(r).to(dev) if b else None, b,
                                torch.from_numpy(np.ascontiguousarray(H)).to(dev), cap, packed)
    torch.cuda.synchronize()
    out_g, sc_g = packed_to_row_major(packed)
    assert np.array_equal(sc_g, scales), "scales changed"
    assert np.array_equal(flips.cpu().numpy(), flips_o), (flips.cpu().numpy()[:8], flips_o[:8])
    assert np.array_equal(out_g, out_o), "%d code bytes differ" % int(np.count_nonzero(out_g != out_o))
    return flips_o


@pytest.mark.parametrize("N,K,b,cap,f32", [
    (64, 256, 32, 64, False),
    (40, 512, 64, 1000, False),   # runs until no move helps
    (24, 1024, 128, 16, True),    # fp32 weights
    (17, 320, 0, 32, False),      # plain MXFP4, ragged K
    (8, 2048, 32, 0, False),      # cap 0: nothing moves
    (6, 4096, 32, 48, False),     # two element pairs per thread
])
def test_flip_refine_bit_exact(dev, N, K, b, cap, f32):
    log("flip_refine N=%d K=%d b=%d cap=%d f32=%s" % (N, K, b, cap, f32))
    flips = _refine_case(dev, N, K, b, cap, f32, seed=N + K)
    if cap:
        assert flips.sum() > 0


def test_flip_refine_wide_rows(dev):
    """K = 20480 (16 element pairs per thread); H is the fp64 Gram of random
    rows computed here in numpy (any symmetric H serves the comparison)."""
    K, N = 20480, 2
    log("flip_refine wide K=%d" % K)
    rng = np.random.default_rng(11)
    xt = rng.standard_normal((12, K))
    H = xt.T @ xt
    flips = _refine_case(dev, N, K, 32, 24, seed=3, H_np=H)
    assert flips.sum() > 0


@pytest.mark.parametrize("K", [3072, 6144, 12288, 14336, 16384])
def test_flip_refine_row_layouts(dev, K):
    """Row lengths that take each workgroup layout of the move kernel: 256
    threads with the last pairs past K (3072), 1024 threads with 3, 6, 7 and 8
    element pairs per thread (6144 ragged, 12288, 14336, 16384). H is the fp64
    Gram of random rows computed here in numpy."""
    N = 2
    log("flip_refine row layout K=%d" % K)
    rng = np.random.default_rng(K)
    xt = rng.standard_normal((12, K))
    H = xt.T @ xt
    flips = _refine_case(dev, N, K, 32, 24, seed=K, H_np=H)
    assert flips.sum() > 0


def test_flip_refine_prefill_layer_sampled(dev):
    """A prefill 8B-shaped layer (4096 x 4096, b = 32) refined whole on the GPU;
    the oracle refines a sample of rows (rows are independent)."""
    c = inputs.linear_case(2, 0, M=16)
    K, N, b = c.K, c.N, c.b
    log("flip_refine prefill layer N=%d K=%d" % (N, K))
    xcal = inputs.activations(2, 0, 512, K, stream=1)
    xb = bits(c.xcal)
    a, r = oracle.multipliers(oracle.calibrate(xb), b)
    H_o = oracle.hessian(bits(xcal), a, b)
    w = c.w.to(dev)
    r_d = torch.from_numpy(r).to(dev)
    packed = binding.prepare_weights(w, r_d, b)
    H_g = binding.hessian(xcal.to(dev), torch.from_numpy(a).to(dev), b)
    torch.cuda.synchronize()
    assert np.array_equal(H_g.cpu().numpy().view(np.uint64), H_o.view(np.uint64))
    codes0, scales0 = packed_to_row_major(packed)
    flips = binding.flip_refine(w, r_d, b, H_g, 64, packed).cpu().numpy()
    torch.cuda.synchronize()
    out_g, _ = packed_to_row_major(packed)
    rows = np.sort(np.random.default_rng(2).choice(N, 6, replace=False))
    out_o, flips_o = oracle.flip_refine(bits(c.w)[rows], r, b, H_o, 64, codes0[rows], scales0[rows])
    log("rows %s flips %s" % (list(rows), list(flips_o)))
    assert np.array_equal(flips[rows], flips_o)
    assert np.array_equal(out_g[rows], out_o)
