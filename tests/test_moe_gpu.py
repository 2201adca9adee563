"""MoE block on the GPU vs the CPU oracle, through the C ABI.

Routing is compared bit for bit. The down projection's MXFP4 input comes out
of the gate/up GEMM's epilogue, where gate and up are fp32 sums on the GPU and
fp64 sums in the oracle: the codes and scales are decided in fp32 on both
sides, but from values that may differ in their last bits, so a code sitting
within a few ulp of a rounding midpoint (or a group whose amax sits at a power
of two) may land on the neighbouring value. The tests bound that fraction and
check the dequantized inputs and the outputs by relative L2 error. The down
projection and the combine are checked on the oracle's own down inputs.
"""
import functools

import numpy as np
import pytest
import torch

import oracle
from moe_util import bf16_round, oracle_prepare
from mxfp4_w4a4_post_amd import binding, inputs
from parity_util import REL_L2_TOL, bits, gemm_layout_to_row_major, log, padded, rel_l2, row_major_to_gemm_layout

pytestmark = pytest.mark.gpu

# fraction of down-input codes / scales allowed to differ from the oracle's
# (decisions taken in fp32 on values that differ in their last bits)
DN_SLIP_FRACTION = 1e-4


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    binding.load_library()
    return torch.device("cuda:0")


@functools.lru_cache(maxsize=2)
def small_case(T, E, k, H, F, b):
    return inputs.moe_block_case(tokens=T, experts=E, top_k=k, hidden=H, ffn=F, b=b)


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


def split_tokens(gc, gs, oc, os_, pos, T, k):
    """Tokens whose k rows of down input equal the oracle's bit for bit, and
    the rest (rows with a slipped code or scale)."""
    bad_row = (gc != oc).any(axis=1) | (gs != os_).any(axis=1)
    p = np.asarray(pos).reshape(T, k)
    bad = np.zeros(T, bool)
    for t in range(T):
        rows = p[t][p[t] >= 0]
        bad[t] = bool(bad_row[rows].any()) if rows.size else False
    return ~bad, bad


def assert_y_close(y, y_o, clean, what, bf16=False):
    """Tokens with identical down inputs: rel-L2 within the output tolerance
    (against the oracle rounded to bf16 for bf16 output). Tokens with a
    slipped down-input code: each within 5% (one E2M1 step of one of the
    F inputs of one of its k rows)."""
    ref = bf16_round(y_o) if bf16 else np.asarray(y_o, np.float64)
    got = np.asarray(y, np.float64)
    if clean.any():
        err = rel_l2(got[clean], ref[clean])
        assert err <= REL_L2_TOL, "%s: rel-L2 %.3e over %d tokens" % (what, err, int(clean.sum()))
    for t in np.nonzero(~clean)[0]:
        e = rel_l2(got[t], ref[t])
        assert e <= 5e-2, "%s: token %d with a slipped down-input code off by %.3e" % (what, t, e)


def assert_dn_close(gc, gs, oc, os_, what):
    n_s = int(np.count_nonzero(gs != os_))
    assert n_s <= max(1, DN_SLIP_FRACTION * gs.size), "%s: %d of %d scales differ" % (what, n_s, gs.size)
    n_c = int(np.count_nonzero(gc != oc))
    assert n_c <= max(2, DN_SLIP_FRACTION * gc.size * 2), "%s: %d of %d code bytes differ" % (what, n_c, gc.size)
    if n_s or n_c:
        log("%s: %d scales and %d code bytes differ" % (what, n_s, n_c))
    dg = oracle.dequant_rows(gc, gs)
    do = oracle.dequant_rows(oc, os_)
    assert rel_l2(dg, do) <= REL_L2_TOL, what


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
    lay = gpu_layer(c, dev)
    a_gu, gc, gs, a_dn, dc, ds = oracle_prepare(oracle, c)
    _, hc, hs = oracle.moe_block(bits(c.x), c.ids, c.w, E, a_gu, gc, gs, a_dn, dc, ds, b, threads=4)
    x = c.x.to(dev)
    off, tok, pos = binding.moe_route(torch.from_numpy(c.ids).to(dev), E)
    dn = binding.moe_gate_up(x, k, tok, off, lay.a_gu, b, lay.wgu, lay.a_dn)
    torch.cuda.synchronize()
    R = T * k
    g_c, g_s = dn_row_major(dn, R, F)
    assert_dn_close(g_c, g_s, hc, hs, "down input")


@pytest.mark.parametrize("T,E,k,H,F,b", BLOCK_CASES[:3])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_down_combine_on_oracle_inputs(dev, T, E, k, H, F, b, out_dtype):
    log("moe down/combine T=%d E=%d k=%d H=%d F=%d b=%d %s" % (T, E, k, H, F, b, out_dtype))
    c = small_case(T, E, k, H, F, b)
    lay = gpu_layer(c, dev)
    a_gu, gc, gs, a_dn, dc, ds = oracle_prepare(oracle, c)
    y_o, hc, hs = oracle.moe_block(bits(c.x), c.ids, c.w, E, a_gu, gc, gs, a_dn, dc, ds, b, threads=4)
    R = T * k
    cod, sca = row_major_to_gemm_layout(hc, hs)
    dn = binding.Packed(torch.from_numpy(cod).to(dev), torch.from_numpy(sca).to(dev), R, F)
    off, tok, pos = binding.moe_route(torch.from_numpy(c.ids).to(dev), E)
    y = binding.moe_down_combine(dn, off, pos, torch.from_numpy(c.w).to(dev), lay.wdn, out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert_y_close(y.float().cpu().numpy(), y_o, np.ones(T, bool), "down/combine", out_dtype == torch.bfloat16)


@pytest.mark.parametrize("T,E,k,H,F,b", BLOCK_CASES)
def test_block_end_to_end(dev, T, E, k, H, F, b):
    log("moe block T=%d E=%d k=%d H=%d F=%d b=%d" % (T, E, k, H, F, b))
    c = small_case(T, E, k, H, F, b)
    lay = gpu_layer(c, dev)
    a_gu, gc, gs, a_dn, dc, ds = oracle_prepare(oracle, c)
    y_o, _, _ = oracle.moe_block(bits(c.x), c.ids, c.w, E, a_gu, gc, gs, a_dn, dc, ds, b, threads=4)
    _, hc, hs = oracle.moe_block(bits(c.x), c.ids, c.w, E, a_gu, gc, gs, a_dn, dc, ds, b, threads=4)
    ids = torch.from_numpy(c.ids).to(dev)
    w = torch.from_numpy(c.w).to(dev)
    x = c.x.to(dev)
    y = lay(x, ids, w, out_dtype=torch.float32)
    y2 = lay(x, ids, w, out_dtype=torch.float32)  # a second call on a fresh workspace
    yb = lay(x, ids, w, out_dtype=torch.bfloat16)
    off, tok, pos = binding.moe_route(ids, E)
    dn = binding.moe_gate_up(x, k, tok, off, lay.a_gu, b, lay.wgu, lay.a_dn)
    torch.cuda.synchronize()
    g_c, g_s = dn_row_major(dn, T * k, F)
    clean, _ = split_tokens(g_c, g_s, hc, hs, pos.cpu().numpy(), T, k)
    assert_y_close(y.cpu().numpy(), y_o, clean, "block fp32")
    assert_y_close(yb.float().cpu().numpy(), y_o, clean, "block bf16", bf16=True)
    assert torch.equal(y, y2)


def test_block_ids_out_of_range(dev):
    """Entries with an id outside [0, E) take no row and add nothing."""
    c = small_case(64, 8, 4, 256, 256, 32)
    lay = gpu_layer(c, dev)
    ids = c.ids.copy()
    ids[::7, 1] = -3
    ids[::5, 2] = c.E + 2
    log("moe block with %d bad ids" % int(np.count_nonzero((ids < 0) | (ids >= c.E))))
    a_gu, gc, gs, a_dn, dc, ds = oracle_prepare(oracle, c)
    y_o, hc, hs = oracle.moe_block(bits(c.x), ids, c.w, c.E, a_gu, gc, gs, a_dn, dc, ds, c.b, threads=4)
    ids_d = torch.from_numpy(ids).to(dev)
    x = c.x.to(dev)
    y = lay(x, ids_d, torch.from_numpy(c.w).to(dev), out_dtype=torch.float32)
    off, tok, pos = binding.moe_route(ids_d, c.E)
    dn = binding.moe_gate_up(x, c.k, tok, off, lay.a_gu, c.b, lay.wgu, lay.a_dn)
    torch.cuda.synchronize()
    n = int(off[-1].item())
    g_c, g_s = dn_row_major(dn, c.T * c.k, c.F)
    clean, _ = split_tokens(g_c[:n], g_s[:n], hc[:n], hs[:n], pos.cpu().numpy(), c.T, c.k)
    assert_y_close(y.cpu().numpy(), y_o, clean, "block with bad ids")


def test_block_moe_workload_sampled(dev):
    """The MoE workload at full size (4096 tokens, 128 experts, top-8, hidden
    2048, expert FFN 768, b = 32), run whole on the GPU as the benchmark runs
    it; the oracle computes a sample of tokens (their rows only)."""
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
    rng = np.random.default_rng(44)
    sample = np.sort(rng.choice(c.T, size=12, replace=False))
    want = np.zeros(c.T, bool)
    want[sample] = True
    used = np.unique(c.ids[sample])
    a_gu, gc, gs, a_dn, dc, ds = oracle_prepare(oracle, c, experts=used)
    y_o, hc, hs = oracle.moe_block(bits(c.x), c.ids, c.w, c.E, a_gu, gc, gs, a_dn, dc, ds, c.b, want=want)
    p = pos.cpu().numpy()
    rows = p.reshape(c.T, c.k)[sample].reshape(-1)
    g_c, g_s = dn_row_major(dn, c.T * c.k, c.F)
    assert_dn_close(g_c[rows], g_s[rows], hc[rows], hs[rows], "sampled down input")
    clean, _ = split_tokens(g_c, g_s, hc, hs, p, c.T, c.k)
    clean = clean[sample]
    log("sampled tokens %s, %d with identical down inputs" % (list(sample[:4]), int(clean.sum())))
    assert_y_close(y.float().cpu().numpy()[sample], y_o[sample], clean, "workload sample", bf16=True)
