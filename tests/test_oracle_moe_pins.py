"""Pins of the oracle's MoE block to things other than itself.

Routing is checked against numpy's stable lexsort and by brute force;
SiLU * up against closed forms (SiLU(0) = 0, SiLU(g) - SiLU(-g) = g) and a
layout probe of the stacked gate/up columns; the combine against exact row
selection and a numpy restatement; the whole block against a restatement
that takes only the already pinned quantizer and dequantizer from the oracle
and does the routing, gathering, matmuls, SiLU, bf16 rounding and combine in
numpy, and against the dense layer when there is one expert and k = 1.
"""
import numpy as np
import pytest
from mxfp4_w4a4_post_amd import inputs

from moe_util import bf16_round as _bf16_round, oracle_prepare as _prepare_case


def _np_route(ids, E):
    """Independent restatement: stable sort of entries by expert id."""
    flat = ids.reshape(-1)
    n = flat.size
    valid = (flat >= 0) & (flat < E)
    order = np.lexsort((np.arange(n), np.where(valid, flat, E)))
    order = order[valid[order]]
    counts = np.bincount(flat[valid], minlength=E)
    off = np.zeros(E + 1, np.int64)
    off[1:] = np.cumsum(counts)
    pos = np.full(n, -1, np.int64)
    pos[order] = np.arange(order.size)
    return off, order // ids.shape[1], pos


@pytest.mark.parametrize("T,k,E", [(1, 1, 1), (7, 3, 5), (64, 8, 16), (33, 2, 40)])
def test_route_matches_stable_sort(orc, T, k, E):
    rng = np.random.default_rng(T * 100 + k * 10 + E)
    ids = rng.integers(0, E, size=(T, k), dtype=np.int32)
    off, row_token, pos = orc.moe_route(ids, E)
    eoff, etok, epos = _np_route(ids, E)
    assert np.array_equal(off, eoff)
    assert np.array_equal(pos, epos)
    assert np.array_equal(row_token[:off[-1]], etok)
    # inverse maps: row pos[i] holds entry i's token and lies in its expert's range
    for i, r in enumerate(pos):
        assert row_token[r] == i // k
        e = ids.reshape(-1)[i]
        assert off[e] <= r < off[e + 1]


def test_route_skips_ids_out_of_range(orc):
    ids = np.array([[0, 3], [-1, 1], [2, 0]], np.int32)
    off, row_token, pos = orc.moe_route(ids, 3)
    assert off.tolist() == [0, 2, 3, 4]
    assert pos.tolist() == [0, -1, -1, 2, 3, 1]
    assert row_token[:4].tolist() == [0, 2, 1, 2]


def test_route_empty_experts(orc):
    ids = np.full((5, 2), 3, np.int32)
    off, row_token, pos = orc.moe_route(ids, 6)
    assert off.tolist() == [0, 0, 0, 0, 10, 10, 10]
    assert pos.tolist() == list(range(10))
    assert row_token.tolist() == [0, 0, 1, 1, 2, 2, 3, 3, 4, 4]


def _stack(g, u):
    """[R, F] gate and up outputs -> [R, 2F] with alternating 32-column blocks."""
    R, F = g.shape
    return np.stack([g.reshape(R, F // 32, 32), u.reshape(R, F // 32, 32)], axis=2).reshape(R, 2 * F)


def test_silu_closed_forms(orc):
    g = np.linspace(-20.0, 20.0, 64 * 5).reshape(5, 64)
    ones = np.ones_like(g)
    hp = orc.silu_mul(_stack(g, ones)).astype(np.float64)
    hn = orc.silu_mul(_stack(-g, ones)).astype(np.float64)
    # SiLU(g) - SiLU(-g) = g; each side is one fp32 rounding of the exact value
    tol = 2.0 * np.spacing(np.maximum(np.abs(hp), np.abs(hn)).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs((hp - hn) - g) <= tol + 1e-300)
    z = orc.silu_mul(_stack(np.zeros((1, 32)), np.full((1, 32), 7.0)))
    assert np.all(z == 0.0)
    # SiLU(1) = 1 / (1 + e^-1)
    one = orc.silu_mul(_stack(np.ones((1, 32)), np.full((1, 32), 2.0)))
    assert np.all(one == np.float32(2.0 / (1.0 + np.exp(-1.0))))
    # far right SiLU(g) = g in fp32, far left it vanishes
    big = orc.silu_mul(_stack(np.full((1, 32), 40.0), np.full((1, 32), 3.0)))
    assert np.all(big == np.float32(120.0))
    small = orc.silu_mul(_stack(np.full((1, 32), -200.0), np.ones((1, 32))))
    assert np.all(small == 0) and np.all(np.signbit(small))


def test_silu_mul_layout(orc):
    """Channel c takes gate column 64 (c // 32) + c % 32 and up column + 32."""
    R, F = 3, 96
    gu = np.zeros((R, 2 * F))
    for c in range(F):
        gu[:, 64 * (c // 32) + c % 32] = 40.0 + c           # gate: SiLU = itself
        gu[:, 64 * (c // 32) + 32 + c % 32] = np.arange(1, R + 1)  # up: row number
    h = orc.silu_mul(gu)
    expect = (40.0 + np.arange(F))[None, :] * np.arange(1, R + 1)[:, None]
    assert np.array_equal(h, expect.astype(np.float32))


def test_combine_selects_and_weights(orc):
    rng = np.random.default_rng(3)
    rows = rng.standard_normal((10, 7)).astype(np.float32)
    pos = np.array([[3, 9, -1], [0, 0, 5]], np.int32)
    onehot = np.array([[1, 0, 0], [0, 0, 1]], np.float32)
    y = orc.moe_combine(rows, pos, onehot)
    assert np.array_equal(y[0], rows[3].astype(np.float64))
    assert np.array_equal(y[1], rows[5].astype(np.float64))
    w = rng.random((2, 3)).astype(np.float32)
    y = orc.moe_combine(rows, pos, w)
    expect = np.zeros((2, 7))
    for t in range(2):
        for j in range(3):
            if pos[t, j] >= 0:
                expect[t] += np.float64(w[t, j]) * rows[pos[t, j]].astype(np.float64)
    assert np.allclose(y, expect, rtol=1e-15, atol=0)


def test_moe_block_matches_restatement(orc):
    c = inputs.moe_block_case(tokens=40, experts=6, top_k=3, hidden=64, ffn=64)
    a_gu, gc, gs, a_dn, dc, ds = _prepare_case(orc, c)
    x = inputs.bf16_bits(c.x)
    y, hc, hs = orc.moe_block(x, c.ids, c.w, c.E, a_gu, gc, gs, a_dn, dc, ds, c.b, threads=2)

    # restatement: numpy routing, the pinned quantizer / dequantizer per row,
    # numpy matmuls, SiLU, bf16 rows and combine
    off, row_token, pos = _np_route(c.ids, c.E)
    R = c.T * c.k
    rows = np.zeros((R, c.H))
    for e in range(c.E):
        sl = slice(off[e], off[e + 1])
        if off[e + 1] == off[e]:
            continue
        xe = x[row_token[sl]]
        qc, qs = orc.quant_rows(xe, a_gu[e], c.b)
        gu = orc.dequant_rows(qc, qs) @ orc.dequant_rows(gc[e], gs[e]).T
        g = np.concatenate([gu[:, 64 * j: 64 * j + 32] for j in range(c.F // 32)], axis=1)
        u = np.concatenate([gu[:, 64 * j + 32: 64 * j + 64] for j in range(c.F // 32)], axis=1)
        h = (g / (1.0 + np.exp(-g)) * u).astype(np.float32)
        hq, hsq = orc.quant_rows(h, a_dn[e], c.b)
        assert np.array_equal(hc[sl], hq) and np.array_equal(hs[sl], hsq)
        rows[sl] = _bf16_round(orc.dequant_rows(hq, hsq) @ orc.dequant_rows(dc[e], ds[e]).T)
    expect = np.zeros((c.T, c.H))
    for t in range(c.T):
        for j in range(c.k):
            expect[t] += np.float64(c.w[t, j]) * rows[pos[t * c.k + j]]
    assert np.allclose(y, expect, rtol=1e-12, atol=1e-12)


def test_moe_block_single_expert_is_dense_chain(orc):
    """E = 1, k = 1, weight 1: the block is linear -> SiLU * up -> linear."""
    c = inputs.moe_block_case(tokens=12, experts=1, top_k=1, hidden=64, ffn=32)
    a_gu, gc, gs, a_dn, dc, ds = _prepare_case(orc, c)
    x = inputs.bf16_bits(c.x)
    w1 = np.ones((c.T, 1), np.float32)
    y, _, _ = orc.moe_block(x, c.ids, w1, 1, a_gu, gc, gs, a_dn, dc, ds, c.b, threads=1)
    gu = orc.linear(x, a_gu[0], c.b, gc[0], gs[0], threads=1)
    h = orc.silu_mul(gu)
    hq, hs = orc.quant_rows(h, a_dn[0], c.b)
    yd = orc.gemm_codes(hq, hs, dc[0], ds[0], threads=1)
    assert np.array_equal(y, _bf16_round(yd))


def test_moe_block_token_subset(orc):
    c = inputs.moe_block_case(tokens=24, experts=4, top_k=2, hidden=64, ffn=64)
    a_gu, gc, gs, a_dn, dc, ds = _prepare_case(orc, c)
    x = inputs.bf16_bits(c.x)
    y, hc, hs = orc.moe_block(x, c.ids, c.w, c.E, a_gu, gc, gs, a_dn, dc, ds, c.b, threads=2)
    want = np.zeros(c.T, bool)
    want[[0, 5, 23]] = True
    ys, hcs, hss = orc.moe_block(x, c.ids, c.w, c.E, a_gu, gc, gs, a_dn, dc, ds, c.b, want=want, threads=2)
    assert np.array_equal(ys[want], y[want])
    assert np.all(ys[~want] == 0)
    _, _, pos = orc.moe_route(c.ids, c.E)
    rows = pos.reshape(c.T, c.k)[want].reshape(-1)
    assert np.array_equal(hcs[rows], hc[rows]) and np.array_equal(hss[rows], hs[rows])
