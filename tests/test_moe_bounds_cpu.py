"""Pins of the MoE parity machinery (CPU only).

The GPU MoE tests rebuild the oracle's block step by step (to see the
gate/up sums and h behind any down-input code that differs) and check the
GPU's down projection and combine on the GPU's own down input. These tests
pin that machinery before any GPU result is judged by it:

  - the step-by-step rebuild gives the oracle block's own down inputs, and
    the chained down/combine reference on those inputs its own output, bit
    for bit;
  - the slip check accepts codes quantized from values the bound allows
    (a simulated fp32 gate/up + SiLU, and h perturbed by up to 0.9 of the
    bound), and rejects planted mistakes: a code moved one step away from a
    tie, a code moved two steps, a scale moved off a group whose largest
    magnitude is far from a power of two, a zero with the wrong sign;
  - the E2M1 / E8M0 helpers against the oracle's own quantizer;
  - the down/combine bound holds for a simulated fp32 down GEMM (chunked
    fp32 sums), bf16 rows and an fp32 fused multiply-add combine, and a
    planted output error outside it is caught.
"""
import numpy as np
import pytest

from moe_util import (check_slips, down_combine_reference, dn_input_bound, e2m1_index, e8m0_code,
                      oracle_down_inputs, oracle_prepare, rn_bf16, split_gate_up)
from mxfp4_w4a4_post_amd import inputs
from parity_util import accumulation_bound, assert_elementwise, unpack

CASES = [(64, 8, 4, 256, 256, 32), (37, 5, 3, 512, 96, 32), (40, 4, 3, 256, 384, 128), (50, 7, 2, 256, 160, 0)]


def _case(T, E, k, H, F, b):
    return inputs.moe_block_case(tokens=T, experts=E, top_k=k, hidden=H, ffn=F, b=b)


@pytest.mark.parametrize("T,E,k,H,F,b", CASES)
def test_rebuild_matches_block(orc, T, E, k, H, F, b):
    c = _case(T, E, k, H, F, b)
    prep = oracle_prepare(orc, c)
    y_o, hc_o, hs_o = orc.moe_block(inputs.bf16_bits(c.x), c.ids, c.w, E, *prep, b)
    hc = np.zeros_like(hc_o)
    hs = np.zeros_like(hs_o)
    for e, rows, ac, as_, gu, h, c_, s_ in oracle_down_inputs(orc, c, prep):
        hc[rows], hs[rows] = c_, s_
    assert np.array_equal(hc, hc_o) and np.array_equal(hs, hs_o)
    y, bound = down_combine_reference(orc, c, prep, hc, hs, np.arange(T))
    assert np.array_equal(y, y_o)
    assert np.all(bound > 0)


def test_rn_bf16_matches_torch(orc):
    import torch
    rng = np.random.default_rng(5)
    v = rng.standard_normal(20000) * np.exp2(rng.integers(-30, 30, 20000))
    # fp64 values round to fp32 first, then to bf16, as torch does in two steps
    ref = torch.from_numpy(v).float().to(torch.bfloat16).float().numpy().astype(np.float64)
    assert np.array_equal(rn_bf16(v), ref)
    # ties to even: 1 + 2^-8 lies between 1 and 1 + 2^-7
    assert rn_bf16(np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8]))[0] == 1.0
    assert rn_bf16(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2.0 ** -6


def test_e2m1_e8m0_match_oracle_quantizer(orc):
    """Round a group whose largest magnitude fixes the scale: the helpers give
    the oracle quantizer's codes and scale."""
    rng = np.random.default_rng(6)
    rows = rng.standard_normal((512, 32)).astype(np.float32) * np.float32(3.0)
    rows[:64] = np.round(rows[:64] * 4) / 4          # many exact ties
    rows[64:80] = 0.0
    codes, scales = orc.quant_rows(rows, None, 0)
    amax = np.max(np.abs(rows.astype(np.float64)), axis=1)
    sc = e8m0_code(amax)
    assert np.array_equal(sc, scales[:, 0].astype(np.int64))
    X = np.ldexp(1.0, sc - 127)[:, None]
    idx = e2m1_index(np.abs(rows) / X)
    nib = unpack(codes)
    assert np.array_equal(idx, nib & 7)


def _perturbed_codes(orc, h, dh, a, b, theta):
    hp = (h.astype(np.float64) + theta * dh).astype(np.float32)
    return orc.quant_rows(hp, a, b)


def _h_bound(gu, b_gu):
    """Per element bound on |h_gpu - h_oracle| alone (the dn term of
    dn_input_bound with a = 1, b = 0)."""
    return dn_input_bound(gu, b_gu, np.zeros((gu.shape[0], gu.shape[1] // 2), np.float32), None, 0)


@pytest.mark.parametrize("T,E,k,H,F,b", CASES)
def test_slip_check_accepts_values_within_bound(orc, T, E, k, H, F, b):
    c = _case(T, E, k, H, F, b)
    prep = oracle_prepare(orc, c)
    rng = np.random.default_rng(T + F)
    n_diff = 0
    for e, rows, ac, as_, gu, h, hc, hs in oracle_down_inputs(orc, c, prep):
        ad = None if prep[3] is None else prep[3][e]
        b_gu = accumulation_bound(orc, ac, as_, prep[1][e], prep[2][e], H)
        t = orc.transform_rows(h, ad, b)
        dt = dn_input_bound(gu, b_gu, h, ad, b)
        assert check_slips(hc, hs, hc, hs, t, dt) == (0, 0)
        # gate/up rounded to fp32 and an fp32 SiLU
        g32, u32 = (v.astype(np.float32) for v in split_gate_up(gu))
        s32 = g32 / (np.float32(1) + np.exp(-g32))
        h32 = (s32 * u32).astype(np.float32)
        c32, s32c = orc.quant_rows(h32, ad, b)
        check_slips(c32, s32c, hc, hs, t, dt)
        # h moved by up to 0.9 of its own bound
        dh = _h_bound(gu, b_gu)
        theta = rng.choice([-0.9, 0.9], size=h.shape)
        cp, sp = _perturbed_codes(orc, h, dh, ad, b, theta)
        nc, ns = check_slips(cp, sp, hc, hs, t, dt)
        n_diff += nc + ns
    print("codes / scales moved by a perturbation within the bound: %d" % n_diff)


def _first_case(orc):
    c = _case(64, 8, 4, 256, 256, 32)
    prep = oracle_prepare(orc, c)
    e, rows, ac, as_, gu, h, hc, hs = next(iter(oracle_down_inputs(orc, c, prep)))
    ad = prep[3][e]
    b_gu = accumulation_bound(orc, ac, as_, prep[1][e], prep[2][e], c.H)
    t = orc.transform_rows(h, ad, c.b).astype(np.float64)
    dt = dn_input_bound(gu, b_gu, h, ad, c.b)
    return hc, hs, t, dt


def _set_nibble(codes, r, j, v):
    out = codes.copy()
    byte = out[r, j // 2]
    out[r, j // 2] = (byte & 0xF0) | v if j % 2 == 0 else (byte & 0x0F) | (v << 4)
    return out


def test_slip_check_rejects_planted_mistakes(orc):
    hc, hs, t, dt = _first_case(orc)
    nib = unpack(hc)
    X = np.ldexp(1.0, np.repeat(hs.astype(np.int64), 32, axis=1) - 127)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    dist = np.min(np.abs(np.abs(t)[..., None] / X[..., None] - mids), axis=-1) * X
    # a code one step up, far from any tie (magnitude 1 .. 4, room to move)
    far = (dist > 100 * dt) & ((nib & 7) >= 2) & ((nib & 7) <= 5)
    r, j = np.argwhere(far)[0]
    with pytest.raises(AssertionError, match="no value within the bound"):
        check_slips(_set_nibble(hc, r, j, int(nib[r, j]) + 1), hs, hc, hs, t, dt)
    # two steps, even where a tie is near (the bound scaled up to cover one step)
    with pytest.raises(AssertionError):
        check_slips(_set_nibble(hc, r, j, int(nib[r, j]) + 2), hs, hc, hs, t, dt * 1e4)
    # a scale one up on a group whose largest magnitude is far from a power of two
    amax = np.max(np.abs(t).reshape(t.shape[0], -1, 32), axis=2)
    frac = amax / np.exp2(np.floor(np.log2(amax)))
    rg, g = np.argwhere((frac > 1.2) & (frac < 1.8))[0]
    hs2 = hs.copy()
    hs2[rg, g] += 1
    with pytest.raises(AssertionError, match="scales outside"):
        check_slips(hc, hs2, hc, hs, t, dt)


def test_slip_check_accepts_a_tie(orc):
    """A code at an exact tie may go either way when the bound reaches it."""
    t = np.zeros((1, 32))
    t[0, 0] = 6.0                     # fixes the scale at 2^0
    t[0, 1] = 1.25                    # tie between 1 (even) and 1.5
    codes, scales = orc.quant_rows(t.astype(np.float32), None, 0)
    assert unpack(codes)[0, 1] == 2
    moved = _set_nibble(codes, 0, 1, 3)
    dt = np.full((1, 32), 1e-6)
    assert check_slips(moved, scales, codes, scales, t, dt) == (1, 0)
    with pytest.raises(AssertionError):
        check_slips(moved, scales, codes, scales, t, np.zeros((1, 32)) + 2.0 ** -149)


def test_slip_check_zero_sign(orc):
    """A small negative value rounds to -0 (code 8); +0 is accepted only when
    the bound reaches a non-negative value."""
    t = np.zeros((1, 32))
    t[0, 0] = 6.0
    t[0, 2] = -0.1
    codes, scales = orc.quant_rows(t.astype(np.float32), None, 0)
    assert unpack(codes)[0, 2] == 8
    flipped = _set_nibble(codes, 0, 2, 0)
    with pytest.raises(AssertionError, match="no value within the bound"):
        check_slips(flipped, scales, codes, scales, t, np.full((1, 32), 0.01))
    assert check_slips(flipped, scales, codes, scales, t, np.full((1, 32), 0.2)) == (1, 0)


def _chunked_fp32_gemm(orc, ac, as_, wc, ws):
    """fp32 GEMM in the shape of the GPU's: exact 64-element partial sums,
    each rounded to fp32, added in order in fp32."""
    A = orc.dequant_rows(ac, as_)
    W = orc.dequant_rows(wc, ws)
    M, K = A.shape
    C = K // 64
    parts = np.einsum("mck,nck->mnc", A.reshape(M, C, 64), W.reshape(W.shape[0], C, 64)).astype(np.float32)
    acc = np.zeros(parts.shape[:2], np.float32)
    for q in range(C):
        acc = (acc.astype(np.float64) + parts[:, :, q]).astype(np.float32)
    return acc


@pytest.mark.parametrize("T,E,k,H,F,b", [CASES[0], CASES[2], (48, 6, 2, 256, 256, 64)])
def test_down_combine_bound_holds_for_fp32_pipeline(orc, T, E, k, H, F, b):
    c = _case(T, E, k, H, F, b)
    prep = oracle_prepare(orc, c)
    _, hc, hs = orc.moe_block(inputs.bf16_bits(c.x), c.ids, c.w, E, *prep, b)
    tokens = np.arange(T)
    y_ref, bound = down_combine_reference(orc, c, prep, hc, hs, tokens)
    off, tok, pos = orc.moe_route(c.ids, E)
    rows = np.zeros((T * k, H), np.float64)
    for e in range(E):
        r = np.arange(off[e], off[e + 1])
        if r.size:
            rows[r] = rn_bf16(_chunked_fp32_gemm(orc, hc[r], hs[r], prep[4][e], prep[5][e]).astype(np.float64))
    p = pos.reshape(T, k)
    y = np.zeros((T, H), np.float32)
    for j in range(k):
        ok = p[:, j] >= 0
        fma = c.w[:, j].astype(np.float64)[:, None] * rows[np.where(ok, p[:, j], 0)] + y.astype(np.float64)
        y = np.where(ok[:, None], fma.astype(np.float32), y)
    assert_elementwise(y, y_ref, bound, "simulated fp32 down/combine")
    planted = y.astype(np.float64).copy()
    planted[3, 7] = y_ref[3, 7] + 2 * bound[3, 7]
    with pytest.raises(AssertionError, match="outside their accumulation bound"):
        assert_elementwise(planted, y_ref, bound, "planted")
