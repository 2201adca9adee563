"""MoE block on the GPU vs the CPU oracle, through the C ABI.

Routing is compared bit for bit.

The down projection's MXFP4 input comes out of the gate/up GEMM's epilogue,
where gate and up are fp32 sums and SiLU a fast exp2 / reciprocal; the
oracle has exact sums and an fp64 SiLU rounded once to fp32. Both sides then
take the same fp32 transform and quantizer, so the GPU's down input must
equal the oracle's except where a transformed value lies within the two
sides' difference of a rounding midpoint (or a group's largest magnitude
within it of a power of two). Every code and scale that differs is checked
against a rigorous per-element bound on that difference (moe_util:
dn_input_bound, check_slips); over the full MoE workload, every routed row,
at most 1e-5 of the codes may differ.

The down projection and the combine are then checked on the GPU's own down
input, per output: against the oracle's fp64 GEMM over those codes, each
expert row rounded to bf16 and summed with the routing weights in fp64,
within a bound made of the fp32 accumulation, a bf16 row rounding that may
fall the other way near a midpoint, and the fp32 combine
(moe_util.down_combine_reference); bf16 outputs lie in
[RN_bf16(y - B), RN_bf16(y + B)].
"""
import dataclasses
import functools

import numpy as np
import pytest
import torch

import oracle
from moe_util import check_down_input, down_combine_reference, oracle_prepare
from mxfp4_w4a4_post_amd import binding, inputs
from parity_util import (assert_bf16_bracket, assert_elementwise, bits, gemm_layout_to_row_major, log, padded,
                         row_major_to_gemm_layout, tile_sample)

pytestmark = pytest.mark.gpu

# largest fraction of down-input codes that may differ from the oracle's over
# the full MoE workload (each one also within its bound)
DN_SLIP_FRACTION = 1e-5


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    binding.load_library()
    return torch.device("cuda:0")


@functools.lru_cache(maxsize=2)
def small_case(T, E, k, H, F, b):
    return inputs.moe_block_case(tokens=T, experts=E, top_k=k, hidden=H, ffn=F, b=b)


@functools.lru_cache(maxsize=2)
def small_prep(T, E, k, H, F, b):
    return oracle_prepare(oracle, small_case(T, E, k, H, F, b))


def gpu_layer(c, dev):
    if c.b == 0:
        return binding.prepare_moe(c.w_gate.to(dev), c.w_up.to(dev), c.w_dn.to(dev), None, None, 0)
    return binding.prepare_moe(c.w_gate.to(dev), c.w_up.to(dev), c.w_dn.to(dev), c.xcal_gu.to(dev),
                               c.xcal_dn.to(dev), c.b)


def dn_row_major(p, R, F):
    """Row-major codes/scales of the down input (rows < R); its K padding must be zero."""
    RP, KP = padded(R, F)
    codes, scales = gemm_layout_to_row_major(p.codes.cpu().numpy(), p.scales.cpu().numpy(), R, F,
                                             check_padding=False)
    full_c, full_s = gemm_layout_to_row_major(p.codes.cpu().numpy(), p.scales.cpu().numpy(), RP, KP,
                                              check_padding=False)
    assert not full_c[:R, F // 2:].any() and not full_s[:R, F // 32:].any(), "K padding of the down input"
    return codes, scales


def check_outputs(c, prep, d_codes, d_scales, tokens, y32=None, y16=None, what=""):
    """GPU outputs of these tokens (fp32 and / or bf16) against the chained
    reference on the down input (d_codes, d_scales)."""
    y_ref, bound = down_combine_reference(oracle, c, prep, d_codes, d_scales, tokens)
    if y32 is not None:
        assert_elementwise(y32, y_ref, bound, what + " fp32")
    if y16 is not None:
        assert_bf16_bracket(y16, y_ref, bound, what + " bf16")
    return y_ref


# ---------------------------------------------------------------------------
# Routing: bit-exact
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T,k,E,bad", [(1, 1, 1, False), (37, 3, 5, True), (64, 8, 16, False), (300, 2, 700, True),
                                       (0, 4, 8, False),       # no entries
                                       (700, 3, 4096, True),   # 3 chunks of 1024 entries, the last ragged
                                       (5001, 8, 64, True),    # 40 chunks, ragged tail
                                       (2048, 8, 1, False)])   # one expert takes every entry
def test_route_bit_exact(dev, T, k, E, bad):
    log("route T=%d k=%d E=%d bad=%s" % (T, k, E, bad))
    rng = np.random.default_rng(T + 10 * k + E)
    ids = rng.integers(0, E, size=(T, k), dtype=np.int32)
    if bad:
        ids[rng.random((T, k)) < 0.1] = -1
        ids[rng.random((T, k)) < 0.05] = E
    off, tok, pos = binding.moe_route(torch.from_numpy(ids).to(dev), E)
    o_off, o_tok, o_pos = oracle.moe_route(ids, E)
    n = int(o_off[-1])
    assert np.array_equal(off.cpu().numpy(), o_off)
    assert np.array_equal(pos.cpu().numpy(), o_pos)
    tg = tok.cpu().numpy()
    assert np.array_equal(tg[:n], o_tok[:n])
    assert np.all(tg[n:] == 0)


def test_route_moe_workload(dev):
    spec = inputs.MOE
    ids, _ = inputs.moe_topk(spec["tokens"], spec["experts"], spec["top_k"], spec["zipf"])
    log("route MoE workload T=%d" % ids.shape[0])
    off, tok, pos = binding.moe_route(torch.from_numpy(ids).to(dev), spec["experts"])
    o_off, o_tok, o_pos = oracle.moe_route(ids, spec["experts"])
    assert np.array_equal(off.cpu().numpy(), o_off)
    assert np.array_equal(tok.cpu().numpy(), o_tok)
    assert np.array_equal(pos.cpu().numpy(), o_pos)


# ---------------------------------------------------------------------------
# Gate/up with the SwiGLU epilogue, down + combine, the whole block
# ---------------------------------------------------------------------------

BLOCK_CASES = [
    (64, 8, 4, 256, 256, 32),
    (37, 5, 3, 512, 96, 32),    # ragged experts, F not a multiple of 256 (K padding written by the epilogue)
    (48, 6, 2, 256, 256, 64),
    (40, 4, 3, 256, 384, 128),
    (50, 7, 2, 256, 160, 0),    # plain MXFP4 (no multipliers, no Hadamard)
]


@pytest.mark.parametrize("T,E,k,H,F,b", BLOCK_CASES)
def test_gate_up_down_input(dev, T, E, k, H, F, b):
    log("moe gate/up T=%d E=%d k=%d H=%d F=%d b=%d" % (T, E, k, H, F, b))
    c = small_case(T, E, k, H, F, b)
    prep = small_prep(T, E, k, H, F, b)
    lay = gpu_layer(c, dev)
    x = c.x.to(dev)
    off, tok, pos = binding.moe_route(torch.from_numpy(c.ids).to(dev), E)
    dn = binding.moe_gate_up(x, k, tok, off, lay.a_gu, b, lay.wgu, lay.a_dn)
    torch.cuda.synchronize()
    g_c, g_s = dn_row_major(dn, T * k, F)
    st, _, _ = check_down_input(oracle, c, prep, g_c, g_s)
    assert st.rows == T * k
    log("down input: %s" % st)


@pytest.mark.parametrize("T,E,k,H,F,b", BLOCK_CASES[:4])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_down_combine_on_oracle_inputs(dev, T, E, k, H, F, b, out_dtype):
    log("moe down/combine T=%d E=%d k=%d H=%d F=%d b=%d %s" % (T, E, k, H, F, b, out_dtype))
    c = small_case(T, E, k, H, F, b)
    prep = small_prep(T, E, k, H, F, b)
    lay = gpu_layer(c, dev)
    _, hc, hs = oracle.moe_block(bits(c.x), c.ids, c.w, E, *prep, b, threads=4)
    cod, sca = row_major_to_gemm_layout(hc, hs)
    dn = binding.Packed(torch.from_numpy(cod).to(dev), torch.from_numpy(sca).to(dev), T * k, F)
    off, tok, pos = binding.moe_route(torch.from_numpy(c.ids).to(dev), E)
    y = binding.moe_down_combine(dn, off, pos, torch.from_numpy(c.w).to(dev), lay.wdn, out_dtype=out_dtype)
    torch.cuda.synchronize()
    y = y.float().cpu().numpy()
    if out_dtype == torch.float32:
        check_outputs(c, prep, hc, hs, np.arange(T), y32=y, what="down/combine")
    else:
        check_outputs(c, prep, hc, hs, np.arange(T), y16=y, what="down/combine")


def run_block(c, prep, lay, dev, ids_np, what):
    """The block through moe_block (fp32 and bf16 outputs, the fp32 one
    twice) and its down input through moe_gate_up; the down input within its
    bounds, the outputs within theirs on that down input, and tokens whose
    down input equals the oracle's against the oracle block's own output."""
    ids = torch.from_numpy(ids_np).to(dev)
    w = torch.from_numpy(c.w).to(dev)
    x = c.x.to(dev)
    y = lay(x, ids, w, out_dtype=torch.float32)
    y2 = lay(x, ids, w, out_dtype=torch.float32)  # a second call on a fresh workspace
    yb = lay(x, ids, w, out_dtype=torch.bfloat16)
    off, tok, pos = binding.moe_route(ids, c.E)
    dn = binding.moe_gate_up(x, c.k, tok, off, lay.a_gu, c.b, lay.wgu, lay.a_dn)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    g_c, g_s = dn_row_major(dn, c.T * c.k, c.F)
    cc = dataclasses.replace(c, ids=ids_np)
    st, o_c, o_s = check_down_input(oracle, cc, prep, g_c, g_s)
    log("%s down input: %s" % (what, st))
    tokens = np.arange(c.T)
    y_ref = check_outputs(cc, prep, g_c, g_s, tokens, y32=y.cpu().numpy(), y16=yb, what=what)
    y_o, _, _ = oracle.moe_block(bits(c.x), ids_np, c.w, c.E, *prep, c.b, threads=4)
    p = pos.cpu().numpy().reshape(c.T, c.k)
    row_diff = (g_c != o_c).any(axis=1) | (g_s != o_s).any(axis=1)
    clean = np.array([not row_diff[p[t][p[t] >= 0]].any() for t in range(c.T)], bool)
    assert np.array_equal(y_ref[clean], y_o[clean]), "%s: chained reference vs the oracle block" % what


@pytest.mark.parametrize("T,E,k,H,F,b", BLOCK_CASES)
def test_block_end_to_end(dev, T, E, k, H, F, b):
    log("moe block T=%d E=%d k=%d H=%d F=%d b=%d" % (T, E, k, H, F, b))
    c = small_case(T, E, k, H, F, b)
    run_block(c, small_prep(T, E, k, H, F, b), gpu_layer(c, dev), dev, c.ids, "block")


def test_block_ids_out_of_range(dev):
    """Entries with an id outside [0, E) take no row and add nothing."""
    c = small_case(64, 8, 4, 256, 256, 32)
    ids = c.ids.copy()
    ids[::7, 1] = -3
    ids[::5, 2] = c.E + 2
    log("moe block with %d bad ids" % int(np.count_nonzero((ids < 0) | (ids >= c.E))))
    run_block(c, small_prep(64, 8, 4, 256, 256, 32), gpu_layer(c, dev), dev, ids, "block with bad ids")


@pytest.mark.timeout(900)
def test_block_moe_workload(dev):
    """The MoE workload at full size (4096 tokens, 128 experts, top-8, hidden
    2048, expert FFN 768, b = 32), run whole on the GPU as the benchmark runs
    it. The down input of every routed row is checked against the oracle's
    (equal, or within its bound, at most 1e-5 of the codes differing); the
    bf16 output of one token in every 64, plus the last, against the chained
    reference on the GPU's down input."""
    c = inputs.moe_block_case()
    log("moe block workload T=%d E=%d k=%d H=%d F=%d" % (c.T, c.E, c.k, c.H, c.F))
    lay = gpu_layer(c, dev)
    ids = torch.from_numpy(c.ids).to(dev)
    w = torch.from_numpy(c.w).to(dev)
    ws = torch.empty(binding.moe_workspace_size(c.T, c.k, c.E, c.H, c.F), dtype=torch.uint8, device=dev)
    x = c.x.to(dev)
    y = lay(x, ids, w, out_dtype=torch.bfloat16, workspace=ws)
    off, tok, pos = binding.moe_route(ids, c.E)
    dn = binding.moe_gate_up(x, c.k, tok, off, lay.a_gu, c.b, lay.wgu, lay.a_dn, workspace=ws)
    torch.cuda.synchronize()
    g_c, g_s = dn_row_major(dn, c.T * c.k, c.F)
    y = y.float().cpu().numpy()
    log("oracle: preparing %d experts" % c.E)
    prep = oracle_prepare(oracle, c)
    log("oracle: down input of every routed row")
    st, o_c, o_s = check_down_input(oracle, c, prep, g_c, g_s)
    log("workload down input: %s (fraction %.2e)" % (st, st.code_diffs / max(st.codes, 1)))
    assert st.rows == c.T * c.k
    assert st.code_diffs <= DN_SLIP_FRACTION * st.codes, str(st)
    assert st.scale_diffs <= DN_SLIP_FRACTION * st.scales, str(st)
    sample = tile_sample(c.T, 64, np.random.default_rng(44))
    log("oracle: outputs of %d tokens" % sample.size)
    check_outputs(c, prep, g_c, g_s, sample, y16=y[sample], what="workload sample")
    # the oracle's own block on a few of them (the chained reference's pin at size)
    few = sample[:8]
    want = np.zeros(c.T, bool)
    want[few] = True
    y_o, hc, hs = oracle.moe_block(bits(c.x), c.ids, c.w, c.E, *prep, c.b, want=want)
    rows = pos.cpu().numpy().reshape(c.T, c.k)[few].reshape(-1)
    assert np.array_equal(hc[rows], o_c[rows]) and np.array_equal(hs[rows], o_s[rows])
