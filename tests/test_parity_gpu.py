"""HIP path vs the CPU oracle, element by element, through the C ABI.

Small cases run whole on both sides; full-size workloads run whole on the GPU
(in the launch configuration the benchmark times) and are compared on sampled
rows and columns that the oracle computes one by one (rows of a linear layer
and rows of W' are independent).
"""
import dataclasses
import functools
import json
import os

import numpy as np
import pytest
import torch

import oracle
from mxfp4_w4a4_post_amd import binding, inputs
from parity_util import (REL_L2_TOL, accumulation_bound, assert_bf16_bracket, assert_elementwise, assert_quant_equal,
                         bits, log, np_u8, packed_to_row_major, rel_l2, row_major_to_gemm_layout, tile_sample)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    binding.load_library()
    return torch.device("cuda:0")


@functools.lru_cache(maxsize=4)
def cached_case(cfg, shape, M=None):
    return inputs.linear_case(cfg, shape, M=M)


def case_with_block(cfg, shape, b, M=None):
    return dataclasses.replace(cached_case(cfg, shape, M), b=b)


def gpu_layer(case, dev, b=None):
    b = case.b if b is None else b
    xcal = case.xcal.to(dev)
    s = binding.calibrate(xcal)
    a, r = binding.make_multipliers(s, b)
    return s, a, r


def oracle_layer(case, b=None):
    b = case.b if b is None else b
    s = oracle.calibrate(bits(case.xcal))
    a, r = oracle.multipliers(s, b)
    return s, a, r


# ---------------------------------------------------------------------------
# Calibration and multipliers: bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("quarters", [0, 1, 2, 4])
def test_calibrate_variants_bit_exact(dev, quarters):
    log("calibrate variant quarters=%d" % quarters)
    xcal = inputs.calibration(2, 0, 4096)
    x = xcal.clone()
    x[:, 7] = 0
    s_g = binding.calibrate(x.to(dev), quarters)
    s_o = oracle.calibrate_pow(bits(x), quarters)
    assert np.array_equal(s_g.cpu().numpy().view(np.uint32), s_o.view(np.uint32))

@pytest.mark.parametrize("cfg,shape,K", [(1, 0, 256), (2, 0, 4096), (3, 1, 25600), (5, 1, 28672)])
def test_calibrate_and_multipliers_bit_exact(dev, cfg, shape, K):
    log("calibrate cfg=%d K=%d" % (cfg, K))
    xcal = inputs.calibration(cfg, shape, K)
    s_g = binding.calibrate(xcal.to(dev))
    s_o = oracle.calibrate(bits(xcal))
    assert np.array_equal(s_g.cpu().numpy().view(np.uint32), s_o.view(np.uint32))
    for b in (0, 32, 64, 128):
        a_g, r_g = binding.make_multipliers(s_g, b)
        a_o, r_o = oracle.multipliers(s_o, b)
        assert np.array_equal(a_g.cpu().numpy().view(np.uint32), a_o.view(np.uint32)), b
        assert np.array_equal(r_g.cpu().numpy().view(np.uint32), r_o.view(np.uint32)), b


# ---------------------------------------------------------------------------
# Activation transform + MXFP4: bit-exact codes and scales
# ---------------------------------------------------------------------------

QUANT_CASES = [
    (1, 0, None, 32), (1, 0, None, 64), (1, 0, None, 128), (1, 0, None, 0),
    (2, 0, None, 32), (2, 2, 512, 32),
    (3, 1, 64, 32), (3, 0, 1, 32),
    (5, 0, 1024, 32), (5, 0, 1024, 64), (5, 1, 256, 128),
]


@pytest.mark.parametrize("cfg,shape,M,b", QUANT_CASES)
def test_quant_act_bit_exact(dev, cfg, shape, M, b):
    case = inputs.linear_case(cfg, shape, M=M, b=b, with_weights=False)
    log("quant_act %s" % case.name)
    _, a_g, _ = gpu_layer(case, dev)
    _, a_o, _ = oracle_layer(case)
    use_scale = b != 0
    x_d = case.x.to(dev)
    c_g, s_g = binding.quant_act(x_d, a_g if use_scale else None, b)
    c_o, s_o = oracle.quant_rows(bits(case.x), a_o if use_scale else None, b)
    t_o = oracle.transform_rows(bits(case.x), a_o if use_scale else None, b)
    assert_quant_equal(np_u8(c_g), np_u8(s_g), c_o, s_o, t_o, case.name)
    # the GEMM layout holds the same codes, with zero padding
    pk = binding.quant_act(x_d, a_g if use_scale else None, b, layout="gemm")
    c_t, s_t = packed_to_row_major(pk)
    assert np.array_equal(c_t, np_u8(c_g)) and np.array_equal(s_t, np_u8(s_g))


def test_quant_act_hand_worked_groups(dev):
    """The hand-worked MX groups through the GPU row quantizer (fp32 input, no
    transform), against the stored expected bytes."""
    cases = json.load(open(os.path.join(GOLDEN, "mx_hand_worked.json")))["cases"]
    w = torch.tensor([c["values"] for c in cases], dtype=torch.float32, device=dev)
    codes, scales = packed_to_row_major(binding.prepare_weights(w, None, 0))
    for i, c in enumerate(cases):
        assert int(scales[i, 0]) == c["scale"], c["what"]
        assert list(np_u8(codes[i])) == c["bytes"], c["what"]


def test_quant_edge_values(dev):
    """Zero rows, ties, -0, saturation, tiny and subnormal groups, and large
    magnitudes, with and without the transform."""
    K = 256
    rng = np.random.default_rng(5)
    rows = []
    rows.append(np.zeros(K, np.float32))
    rows.append(-np.zeros(K, np.float32))
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, 7.99, 8.0], np.float32)
    rows.append(np.resize(np.concatenate([mids, -mids]), K).astype(np.float32))
    rows.append((rng.standard_normal(K) * 1e-38).astype(np.float32))
    rows.append((rng.standard_normal(K) * (3e38 / 1024)).astype(np.float32))
    rows.append((np.float32(2.0) ** rng.integers(-140, 120, size=K).astype(np.float32)).astype(np.float32))
    x = np.stack(rows).astype(np.float32)
    for b in (0, 32, 128):
        log("quant edge b=%d" % b)
        c_g, s_g = packed_to_row_major(binding.prepare_weights(torch.from_numpy(x).to(dev), None, b))
        c_o, s_o = oracle.quant_rows(x, None, b)
        t_o = oracle.transform_rows(x, None, b)
        finite = np.all(np.isfinite(t_o), axis=1)
        assert_quant_equal(np_u8(c_g)[finite], np_u8(s_g)[finite], c_o[finite], s_o[finite], t_o[finite],
                           "edge b=%d" % b)


# ---------------------------------------------------------------------------
# Prepared weights: bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cfg,shape,N,b,f32", [(1, 0, None, 32, False), (2, 0, 1024, 32, False),
                                               (2, 2, 256, 32, True), (5, 0, 256, 128, False),
                                               (3, 0, 512, 32, False)])
def test_prepare_weights_bit_exact(dev, cfg, shape, N, b, f32):
    case = inputs.linear_case(cfg, shape, M=1, b=b, N=N)
    log("prepare_weights %s f32=%s" % (case.name, f32))
    _, _, r_g = gpu_layer(case, dev)
    _, _, r_o = oracle_layer(case)
    w = case.w.float() if f32 else case.w
    c_g, s_g = packed_to_row_major(binding.prepare_weights(w.to(dev), r_g, b))
    w_np = w.numpy() if f32 else bits(w)
    c_o, s_o = oracle.prepare_weights(w_np, r_o, b)
    t_o = oracle.transform_rows(w_np, r_o, b)
    assert_quant_equal(np_u8(c_g), np_u8(s_g), c_o, s_o, t_o, case.name)


# ---------------------------------------------------------------------------
# The GEMM on MXFP4 operands
# ---------------------------------------------------------------------------

GEMM_SHAPES = [(16, 256, 256), (17, 300, 352), (1, 64, 32), (130, 520, 1056), (300, 260, 96), (8, 512, 8192),
               (64, 1024, 4096), (257, 513, 768), (33, 2048, 2560), (1024, 512, 512)]


@pytest.mark.parametrize("M,N,K", GEMM_SHAPES)
def test_gemm_random_codes(dev, M, N, K):
    log("gemm M=%d N=%d K=%d" % (M, N, K))
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    ac = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    as_ = rng.integers(118, 136, size=(M, K // 32), dtype=np.uint8)
    wc = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    ws = rng.integers(118, 136, size=(N, K // 32), dtype=np.uint8)
    def packed(c, sc):
        tc, ts = row_major_to_gemm_layout(c, sc)
        return binding.Packed(torch.from_numpy(tc).to(dev), torch.from_numpy(ts).to(dev), c.shape[0], 2 * c.shape[1])

    pa, pw = packed(ac, as_), packed(wc, ws)
    y = binding.linear_plain_gemm(pa, pw, out_dtype=torch.float32)
    y_o = oracle.gemm_codes(ac, as_, wc, ws)
    bound = accumulation_bound(oracle, ac, as_, wc, ws, K)
    assert_elementwise(y.cpu().numpy(), y_o, bound, "gemm fp32 %d %d %d" % (M, N, K))
    err = rel_l2(y.cpu().numpy(), y_o)
    assert err <= REL_L2_TOL, err
    y16 = binding.linear_plain_gemm(pa, pw, out_dtype=torch.bfloat16)
    assert_bf16_bracket(y16, y_o, bound, "gemm bf16 %d %d %d" % (M, N, K))


# Shapes with at least 256 tiles of 256 x 256 (and K a multiple of 1024):
# the wide-tile kernel, with ragged last m- and n-tiles (N a multiple of 8).
WIDE_SHAPES = [(4100, 4104, 1024), (4096, 4096, 2048), (2048, 14336, 4096), (3000, 6152, 1024)]


@pytest.mark.parametrize("M,N,K", WIDE_SHAPES)
def test_gemm_wide_tiles_random_codes(dev, M, N, K):
    """The wide-tile GEMM on random codes: every output row of a sample that
    holds a row of every 256-row tile (and the last row), all columns, each
    within its accumulation bound, in fp32 and bf16."""
    log("gemm wide M=%d N=%d K=%d" % (M, N, K))
    rng = np.random.default_rng(M + 3 * N + 7 * K)
    ac = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    as_ = rng.integers(118, 136, size=(M, K // 32), dtype=np.uint8)
    wc = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    ws = rng.integers(118, 136, size=(N, K // 32), dtype=np.uint8)

    def packed(c, sc):
        tc, ts = row_major_to_gemm_layout(c, sc)
        return binding.Packed(torch.from_numpy(tc).to(dev), torch.from_numpy(ts).to(dev), c.shape[0], 2 * c.shape[1])

    pa, pw = packed(ac, as_), packed(wc, ws)
    y = binding.linear_plain_gemm(pa, pw, out_dtype=torch.float32)
    y16 = binding.linear_plain_gemm(pa, pw, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = tile_sample(M, 256, rng, extra=(0,))
    y_o = oracle.gemm_codes(ac[rows], as_[rows], wc, ws)
    bound = accumulation_bound(oracle, ac[rows], as_[rows], wc, ws, K)
    got = y.cpu().numpy()[rows]
    assert_elementwise(got, y_o, bound, "gemm wide fp32")
    assert rel_l2(got, y_o) <= REL_L2_TOL
    assert_bf16_bracket(y16.cpu()[torch.from_numpy(rows)], y_o, bound, "gemm wide bf16")
    # the same call again is bit-identical
    y2 = binding.linear_plain_gemm(pa, pw, out_dtype=torch.float32)
    assert torch.equal(y, y2)


# ---------------------------------------------------------------------------
# The layer
# ---------------------------------------------------------------------------

def check_linear(case, dev, rows=None, cols=None, b=None):
    """GPU: the whole layer. Oracle: rows x cols of it (all when None)."""
    b = case.b if b is None else b
    _, a_g, r_g = gpu_layer(case, dev, b)
    _, a_o, r_o = oracle_layer(case, b)
    x_d = case.x.to(dev)
    w_d = case.w.to(dev)
    pw = binding.prepare_weights(w_d, r_g, b)
    wc_g, ws_g = packed_to_row_major(pw)
    y_g = binding.linear(x_d, a_g, b, pw, out_dtype=torch.float32)
    y_g16 = binding.linear(x_d, a_g, b, pw, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rows = np.arange(case.M) if rows is None else np.asarray(rows)
    cols = np.arange(case.N) if cols is None else np.asarray(cols)
    xb = bits(case.x)[rows]
    wb = bits(case.w)[cols]
    wc_o, ws_o = oracle.prepare_weights(wb, r_o, b)
    assert_quant_equal(wc_g[cols], ws_g[cols], wc_o, ws_o, oracle.transform_rows(wb, r_o, b),
                       case.name + " W'")
    ac_o, as_o = oracle.quant_rows(xb, a_o, b)
    y_o = oracle.gemm_codes(ac_o, as_o, wc_o, ws_o)
    bound = accumulation_bound(oracle, ac_o, as_o, wc_o, ws_o, case.K)
    got = y_g.cpu().numpy()[np.ix_(rows, cols)]
    assert_elementwise(got, y_o, bound, case.name + " fp32")
    err = rel_l2(got, y_o)
    log("%s rel-L2 %.3g on %dx%d outputs" % (case.name, err, len(rows), len(cols)))
    assert err <= REL_L2_TOL, err
    assert_bf16_bracket(y_g16.cpu()[torch.from_numpy(rows)][:, torch.from_numpy(cols)], y_o, bound,
                        case.name + " bf16")
    return y_g


def test_linear_tiny_full(dev):
    case = inputs.linear_case(1, 0)
    log("linear %s" % case.name)
    y1 = check_linear(case, dev)
    # determinism: the same call twice is bit-identical
    _, a_g, r_g = gpu_layer(case, dev)
    pw = binding.prepare_weights(case.w.to(dev), r_g, case.b)
    y2 = binding.linear(case.x.to(dev), a_g, case.b, pw, out_dtype=torch.float32)
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("b", [0, 64, 128])
def test_linear_tiny_blocks(dev, b):
    case = inputs.linear_case(1, 0, b=b)
    log("linear %s" % case.name)
    if b == 0:
        # plain MXFP4: no multiply, no Hadamard on either side
        x_d, w_d = case.x.to(dev), case.w.to(dev)
        pw = binding.prepare_weights(w_d, None, 0)
        y = binding.linear(x_d, None, 0, pw, out_dtype=torch.float32)
        wc_o, ws_o = oracle.prepare_weights(bits(case.w), None, 0)
        y_o = oracle.linear(bits(case.x), None, 0, wc_o, ws_o)
        assert np.array_equal(packed_to_row_major(pw)[0], wc_o)
        assert rel_l2(y.cpu().numpy(), y_o) <= REL_L2_TOL
    else:
        check_linear(case, dev, b=b)


@pytest.mark.parametrize("M,K,N", [(17, 96, 40), (1, 32, 16), (65, 352, 264), (300, 1024, 600), (129, 768, 2048)])
def test_linear_ragged(dev, M, K, N):
    """Ragged M, N and K (K a multiple of 32 but not of the 256-element step)."""
    case = inputs.linear_case(1, 0, M=M, K=K, N=N, b=32)
    log("linear ragged %s" % case.name)
    check_linear(case, dev)


def test_linear_strided_and_empty(dev):
    case = inputs.linear_case(1, 0, M=20, K=256, N=48)
    _, a_g, r_g = gpu_layer(case, dev)
    pw = binding.prepare_weights(case.w.to(dev), r_g, case.b)
    xpad = torch.zeros(20, 256 + 64, dtype=torch.bfloat16, device=dev)
    xpad[:, :256] = case.x.to(dev)
    ypad = torch.full((20, 48 + 16), 7.0, dtype=torch.float32, device=dev)
    binding.linear(xpad[:, :256], a_g, case.b, pw, out=ypad[:, :48])
    y = binding.linear(case.x.to(dev), a_g, case.b, pw, out_dtype=torch.float32)
    assert torch.equal(ypad[:, :48], y)
    assert torch.all(ypad[:, 48:] == 7.0)
    empty = binding.linear(torch.empty(0, 256, dtype=torch.bfloat16, device=dev), a_g, case.b, pw)
    assert empty.shape == (0, 48)


@pytest.mark.parametrize("shape", [0, 1, 2])
def test_linear_prefill_8b(dev, shape):
    """The whole layer on the GPU; the oracle on a row of every 128-row tile
    (and the first and last rows) by every column."""
    case = cached_case(2, shape)
    log("linear %s" % case.name)
    rng = np.random.default_rng(100 + shape)
    check_linear(case, dev, tile_sample(case.M, 128, rng, extra=(0,)), None)


@pytest.mark.parametrize("shape", [0, 1])
@pytest.mark.parametrize("M", [1, 8, 32, 64])
def test_linear_decode_32b(dev, M, shape):
    case = inputs.linear_case(3, shape, M=M)
    log("linear %s" % case.name)
    rng = np.random.default_rng(200 + M + shape)
    rows = np.arange(M) if M <= 8 else np.sort(rng.choice(M, 8, replace=False))
    cols = np.sort(rng.choice(case.N, 512, replace=False))
    check_linear(case, dev, rows, cols)


@pytest.mark.parametrize("shape,b", [(0, 32), (1, 32), (0, 64), (1, 64), (0, 128), (1, 128)])
def test_linear_prefill_large(dev, shape, b):
    """The whole layer on the GPU as the benchmark runs it; the oracle on a
    row of every 256-row tile by every column (so every output tile is
    checked), each output within its accumulation bound."""
    case = case_with_block(5, shape, b)
    log("linear %s" % case.name)
    rng = np.random.default_rng(300 + shape + b)
    rows = tile_sample(case.M, 256, rng, extra=(0,)) if b == 32 else np.sort(rng.choice(case.M, 12, replace=False))
    cols = None if b == 32 else np.sort(rng.choice(case.N, 512, replace=False))
    check_linear(case, dev, rows, cols, b=b)


# ---------------------------------------------------------------------------
# Grouped (MoE) layer
# ---------------------------------------------------------------------------

def grouped_gpu(mc, dev, b, out_dtype=torch.float32):
    E, K = mc.E, mc.K
    xcal = mc.xcal.to(dev)
    a = torch.empty(E, K, dtype=torch.float32, device=dev)
    r = torch.empty(E, K, dtype=torch.float32, device=dev)
    for e in range(E):
        s = binding.calibrate(xcal[e])
        a[e], r[e] = binding.make_multipliers(s, b)
    w = mc.w.to(dev)
    pw = binding.empty_grouped_weights(E, mc.N, K, dev)
    for e in range(E):
        binding.prepare_weights(w[e], r[e], b, out=binding.expert(pw, e))
    off = torch.from_numpy(mc.offsets).to(dev)
    y = binding.linear_grouped(mc.x.to(dev), off, a, b, pw, out_dtype=out_dtype)
    return y, a, pw


def oracle_expert(mc, e, b):
    s = oracle.calibrate(bits(mc.xcal[e]))
    a, r = oracle.multipliers(s, b)
    wc, ws = oracle.prepare_weights(bits(mc.w[e]), r, b)
    return a, wc, ws


def test_linear_grouped_small_full(dev):
    mc = inputs.moe_case("gate_up", tokens=64, experts=8)
    log("grouped small T=%d E=%d counts=%s" % (mc.T, mc.E, list(mc.counts)))
    y, a, pw = grouped_gpu(mc, dev, 32)
    a_o = np.zeros((mc.E, mc.K), np.float32)
    wc_o = np.zeros((mc.E, mc.N, mc.K // 2), np.uint8)
    ws_o = np.zeros((mc.E, mc.N, mc.K // 32), np.uint8)
    for e in range(mc.E):
        a_o[e], wc_o[e], ws_o[e] = oracle_expert(mc, e, 32)
        c_e, s_e = packed_to_row_major(binding.expert(pw, e))
        assert np.array_equal(c_e, wc_o[e]) and np.array_equal(s_e, ws_o[e]), e
    y_o = oracle.linear_grouped(bits(mc.x), mc.offsets, a_o, 32, wc_o, ws_o)
    assert rel_l2(y.cpu().numpy(), y_o) <= REL_L2_TOL


def test_linear_grouped_empty_experts(dev):
    """Experts with no rows, and a single-row expert."""
    E, K, N = 5, 256, 96
    off = np.array([0, 0, 40, 40, 41, 300], np.int32)
    T = int(off[-1])
    rng = np.random.default_rng(9)
    x = inputs.to_bf16(rng.standard_normal((T, K)).astype(np.float32))
    a_o = (rng.random((E, K)) + 0.5).astype(np.float32)
    wc_o = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    ws_o = rng.integers(118, 134, size=(E, N, K // 32), dtype=np.uint8)
    tiles = [row_major_to_gemm_layout(wc_o[e], ws_o[e]) for e in range(E)]
    pw = binding.Packed(torch.from_numpy(np.stack([t[0] for t in tiles])).to(dev),
                        torch.from_numpy(np.stack([t[1] for t in tiles])).to(dev), N, K)
    y = binding.linear_grouped(x.to(dev), torch.from_numpy(off).to(dev), torch.from_numpy(a_o).to(dev), 32, pw,
                               out_dtype=torch.float32)
    y_o = oracle.linear_grouped(bits(x), off, a_o, 32, wc_o, ws_o)
    assert rel_l2(y.cpu().numpy(), y_o) <= REL_L2_TOL


@pytest.mark.parametrize("proj", ["gate_up", "down"])
def test_linear_grouped_moe_full(dev, proj):
    mc = inputs.moe_case(proj)
    log("grouped MoE %s T=%d E=%d K=%d N=%d" % (proj, mc.T, mc.E, mc.K, mc.N))
    y, a, pw = grouped_gpu(mc, dev, 32, out_dtype=torch.float32)
    torch.cuda.synchronize()
    counts = mc.counts
    experts = sorted(set([int(np.argmax(counts)), int(np.argmin(counts))] +
                         list(np.random.default_rng(7).choice(mc.E, 6, replace=False))))
    yc = y.cpu().numpy()
    for e in experts:
        lo, hi = int(mc.offsets[e]), int(mc.offsets[e + 1])
        if hi == lo:
            continue
        rows = np.unique(np.concatenate([[lo, hi - 1], np.random.default_rng(e).integers(lo, hi, 4)]))
        a_o, wc_o, ws_o = oracle_expert(mc, e, 32)
        assert np.array_equal(packed_to_row_major(binding.expert(pw, e))[0], wc_o), e
        y_o = oracle.linear(bits(mc.x)[rows], a_o, 32, wc_o, ws_o)
        err = rel_l2(yc[rows], y_o)
        assert err <= REL_L2_TOL, (e, err)


def _grouped_bf16_vs_f32(dev, x, off, a, pw):
    """The grouped layer's bf16 output is its fp32 output rounded to nearest
    even: the same accumulators, only the epilogue differs (bf16 rows go out
    through LDS and are written during the next tile's steps)."""
    y32 = binding.linear_grouped(x, off, a, 32, pw, out_dtype=torch.float32)
    y16 = binding.linear_grouped(x, off, a, 32, pw, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    want = y32.to(torch.bfloat16)
    bad = int((y16.view(torch.int16) != want.view(torch.int16)).sum())
    assert bad == 0, "%d of %d bf16 outputs differ from the rounded fp32 outputs" % (bad, y16.numel())


def test_linear_grouped_bf16_output_moe_down(dev):
    """MoE down projection (32768 expert rows, N = 2048, K = 768): many tiles
    per workgroup and ragged expert tails."""
    mc = inputs.moe_case("down")
    log("grouped bf16 vs fp32 output, down T=%d E=%d K=%d N=%d" % (mc.T, mc.E, mc.K, mc.N))
    _, a, pw = grouped_gpu(mc, dev, 32)
    _grouped_bf16_vs_f32(dev, mc.x.to(dev), torch.from_numpy(mc.offsets).to(dev), a, pw)


@pytest.mark.parametrize("N", [96, 200, 100])
def test_linear_grouped_bf16_output_ragged(dev, N):
    """Ragged N (a partial last column tile; N = 100 takes the path without
    16-byte row alignment), empty and single-row experts."""
    E, K = 6, 512
    off = np.array([0, 0, 300, 301, 301, 700, 1000], np.int32)
    T = int(off[-1])
    log("grouped bf16 vs fp32 output, ragged N=%d T=%d" % (N, T))
    rng = np.random.default_rng(N)
    x = inputs.to_bf16(rng.standard_normal((T, K)).astype(np.float32))
    a = torch.from_numpy((rng.random((E, K)) + 0.5).astype(np.float32)).to(dev)
    wc = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    ws = rng.integers(118, 134, size=(E, N, K // 32), dtype=np.uint8)
    tiles = [row_major_to_gemm_layout(wc[e], ws[e]) for e in range(E)]
    pw = binding.Packed(torch.from_numpy(np.stack([t[0] for t in tiles])).to(dev),
                        torch.from_numpy(np.stack([t[1] for t in tiles])).to(dev), N, K)
    _grouped_bf16_vs_f32(dev, x.to(dev), torch.from_numpy(off).to(dev), a, pw)


@pytest.mark.parametrize("E", [4096, 4100])
def test_linear_grouped_many_experts(dev, E):
    """Thousands of experts, most empty or with a single row: the tile map is
    written entry by entry from the experts' tile prefix (up to 4096 experts)
    or by each expert's own thread beyond that."""
    K, N = 64, 32
    rng = np.random.default_rng(E)
    counts = np.zeros(E, np.int64)
    hot = rng.choice(E, 40, replace=False)
    counts[hot] = rng.integers(1, 300, size=40)
    counts[rng.choice(E, 200, replace=False)] += 1
    off = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    T = int(off[-1])
    log("grouped E=%d T=%d" % (E, T))
    x = inputs.to_bf16(rng.standard_normal((T, K)).astype(np.float32))
    a_o = (rng.random((E, K)) + 0.5).astype(np.float32)
    wc_o = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    ws_o = rng.integers(118, 134, size=(E, N, K // 32), dtype=np.uint8)
    tiles = [row_major_to_gemm_layout(wc_o[e], ws_o[e]) for e in range(E)]
    pw = binding.Packed(torch.from_numpy(np.stack([t[0] for t in tiles])).to(dev),
                        torch.from_numpy(np.stack([t[1] for t in tiles])).to(dev), N, K)
    y = binding.linear_grouped(x.to(dev), torch.from_numpy(off).to(dev), torch.from_numpy(a_o).to(dev), 32, pw,
                               out_dtype=torch.float32)
    y_o = oracle.linear_grouped(bits(x), off, a_o, 32, wc_o, ws_o)
    assert rel_l2(y.cpu().numpy(), y_o) <= REL_L2_TOL
