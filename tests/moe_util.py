"""Oracle-side preparation of MoE block cases, shared by the oracle pins and
the GPU parity tests (numpy and the oracle only)."""
import numpy as np
import torch

from mxfp4_w4a4_post_amd import inputs


def stack_rows(wg, wu):
    """[F, H] gate and up weight rows -> [2F, H], alternating blocks of 32 rows."""
    F, H = wg.shape
    return np.stack([wg.reshape(F // 32, 32, H), wu.reshape(F // 32, 32, H)], axis=1).reshape(2 * F, H)


def bf16_round(v):
    return torch.from_numpy(np.asarray(v, np.float64)).float().bfloat16().float().numpy().astype(np.float64)


def oracle_prepare(orc, c, experts=None, workers=8):
    """Per expert (all, or only those in `experts`): calibrate, multipliers,
    prepared stacked gate/up and down weights (row-major codes and scales).
    Experts left out keep zero weights and unit multipliers. Experts are
    prepared on `workers` threads (the oracle's calls release the GIL);
    each writes only its own slices."""
    from concurrent.futures import ThreadPoolExecutor
    bits = inputs.bf16_bits
    E, F, H, b = c.E, c.F, c.H, c.b
    a_gu = np.ones((E, H), np.float32)
    a_dn = np.ones((E, F), np.float32)
    gc = np.zeros((E, 2 * F, H // 2), np.uint8)
    gs = np.zeros((E, 2 * F, H // 32), np.uint8)
    dc = np.zeros((E, H, F // 2), np.uint8)
    ds = np.zeros((E, H, F // 32), np.uint8)

    def one(e):
        if b == 0:
            gc[e], gs[e] = orc.prepare_weights(stack_rows(bits(c.w_gate[e]), bits(c.w_up[e])), None, 0)
            dc[e], ds[e] = orc.prepare_weights(bits(c.w_dn[e]), None, 0)
            return
        a, r = orc.multipliers(orc.calibrate(bits(c.xcal_gu[e])), b)
        a_gu[e] = a
        gc[e], gs[e] = orc.prepare_weights(stack_rows(bits(c.w_gate[e]), bits(c.w_up[e])), r, b)
        a, r = orc.multipliers(orc.calibrate(bits(c.xcal_dn[e])), b)
        a_dn[e] = a
        dc[e], ds[e] = orc.prepare_weights(bits(c.w_dn[e]), r, b)

    todo = range(E) if experts is None else sorted(set(int(v) for v in experts))
    with ThreadPoolExecutor(max_workers=max(1, workers)) as ex:
        list(ex.map(one, todo))
    if b == 0:
        return None, gc, gs, None, dc, ds
    return a_gu, gc, gs, a_dn, dc, ds


# ---------------------------------------------------------------------------
# The down projection's input: where the GPU may differ from the oracle, and
# by how much
# ---------------------------------------------------------------------------
#
# On the GPU the gate/up GEMM's epilogue forms h = SiLU(g) * u from fp32
# sums and a fast exp2 / reciprocal SiLU; the oracle forms it from exact
# sums with an fp64 SiLU, rounded once to fp32. Both then take the same fp32
# transform and quantizer. A code can therefore differ only where a
# transformed value lies within the two sides' difference of a rounding
# midpoint, and a scale only where a group's largest magnitude lies within
# it of a power of two. dn_input_bound() bounds that difference per element;
# check_slips() requires every GPU code and scale to be one that some value
# within the bound rounds to.

U32 = 2.0 ** -24
SILU_SLOPE = 1.1  # |d/dg g sigma(g)| <= 1.0999 for every real g
_E2M1_MIDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def e2m1_index(m):
    """E2M1 magnitude index (0 .. 7) of m >= 0 already divided by the block
    scale: nearest of 0, .5, 1, 1.5, 2, 3, 4, 6, ties to the even index,
    saturating at 6 (the OCP MX v1.0 element rounding)."""
    m = np.asarray(m, np.float64)
    i = np.searchsorted(_E2M1_MIDS, m, side="left")
    tie = (i < 7) & (_E2M1_MIDS[np.minimum(i, 6)] == m)
    return i + (tie & (i % 2 == 1))


def e8m0_code(amax):
    """Scale code of a group with largest magnitude amax: floor(log2 amax) - 2
    biased by 127, clamped at 0 (also for an all-zero group)."""
    amax = np.asarray(amax, np.float64)
    _, e = np.frexp(amax)
    return np.where(amax > 0, np.clip(e.astype(np.int64) - 3 + 127, 0, 254), 0)


def _ladder(t, X):
    """Signed E2M1 ladder position of t rounded at block scale X (-0 and +0
    both 0): monotone in t."""
    i = e2m1_index(np.abs(t) / X)
    return np.where(t < 0, -i, i)


def rn_bf16(v):
    """Round fp64 values to fp32, then to the nearest bf16 (8 significant
    bits, ties to even), as a device rounds its fp32 result and as the
    oracle rounds an expert row; normal range only. Both steps are monotone."""
    m, e = np.frexp(np.asarray(v, np.float64).astype(np.float32).astype(np.float64))
    return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)


def split_gate_up(gu):
    """Stacked gate/up outputs [n, 2F] (blocks of 32 gate then 32 up
    columns) -> (gate [n, F], up [n, F])."""
    n, F2 = gu.shape
    q = np.asarray(gu).reshape(n, F2 // 64, 2, 32)
    return q[:, :, 0].reshape(n, F2 // 2), q[:, :, 1].reshape(n, F2 // 2)


def dn_input_bound(gu, b_gu, h, a, b):
    """Per element, a bound on |t_gpu - t_oracle| for the transformed down
    inputs S_b(a * h) of rows whose exact gate/up sums are gu [n, 2F] (fp64,
    the oracle's), with the GPU's fp32 gate/up sums within b_gu of them, and
    the oracle's h [n, F] (fp32).

    The GPU's SiLU: e^-g as exp2(g * RN32(-log2 e)) (argument error
    2|g|u, the exp2 taken as within 2 ulp, i.e. 4u), 1 + e^-g (u), a
    reciprocal within 2 ulp (4u), then g * r and (.) * up (u each): relative
    error at most (2.1 |g| + 12) u with u = 2^-24. Where g < -80 the GPU's
    e^-g may overflow and its SiLU come out as zero, so the whole value is
    allowed there. With |SiLU'| <= 1.1, the GPU's h lies within
    dh = P (1 + eta) - |SiLU(g) up| (1 - u) of the oracle's, where
    P = (|SiLU(g)| + 1.1 B_g)(|up| + B_u). The transform is linear with
    entries of magnitude one (the 1/sqrt(b) is in a), so the difference
    carries through as sum_k |a_k| dh_k over the element's block, plus each
    side's own fp32 roundings (one multiply and log2 b butterfly stages):
    gamma_L sum_k |a_k| |h_k| each, with L = 1 + log2 b."""
    gu = np.asarray(gu, np.float64)
    g, up = split_gate_up(gu)
    bg, bu = split_gate_up(np.asarray(b_gu, np.float64))
    n, F = g.shape
    with np.errstate(over="ignore"):
        s = g / (1.0 + np.exp(-g))
    P = (np.abs(s) + SILU_SLOPE * bg) * (np.abs(up) + bu)
    eta = (2.1 * (np.abs(g) + bg) + 12.0) * U32
    dh = P * (1.0 + eta) - np.abs(s * up) * (1.0 - U32)
    dh = np.where(g - bg < -80.0, dh + P, dh)
    bb = max(int(b), 1)
    am = np.ones(F) if a is None else np.abs(np.asarray(a, np.float64))
    L = (0 if a is None else 1) + int(np.log2(bb))
    gam = L * U32 / (1.0 - L * U32)

    def block_sum(v):
        return np.repeat(v.reshape(n, F // bb, bb).sum(axis=2), bb, axis=1)

    z = am * dh
    zh = am * (np.abs(np.asarray(h, np.float64)) + dh)
    return block_sum(z) * (1.0 + U32) + 2.0 * gam * block_sum(zh) + 2.0 ** -149


def check_slips(g_codes, g_scales, o_codes, o_scales, t, dt, what=""):
    """Every GPU code and scale of these rows must be what some transformed
    value within dt of the oracle's t (fp32) quantizes to: scale codes in
    [e8m0(max(|t| - dt)), e8m0(max(|t| + dt))] per group; each element, at
    the GPU's scale X, on the signed E2M1 ladder between RN((t - dt) / X) and
    RN((t + dt) / X), with a zero's sign bit matching a value of that sign in
    the interval; a code that differs under an equal scale one step from the
    oracle's. Returns (code elements that differ, scales that differ)."""
    from parity_util import unpack
    t = np.asarray(t, np.float64)
    dt = np.asarray(dt, np.float64)
    n, F = t.shape
    G = F // 32
    gn = unpack(np.asarray(g_codes, np.uint8)).reshape(n, G, 32).astype(np.int64)
    on = unpack(np.asarray(o_codes, np.uint8)).reshape(n, G, 32).astype(np.int64)
    gp = np.where(gn & 8, -(gn & 7), gn & 7)
    op = np.where(on & 8, -(on & 7), on & 7)
    t3 = t.reshape(n, G, 32)
    d3 = dt.reshape(n, G, 32)
    gs = np.asarray(g_scales, np.int64).reshape(n, G)
    os_ = np.asarray(o_scales, np.int64).reshape(n, G)
    lo_s = e8m0_code(np.max(np.maximum(np.abs(t3) - d3, 0.0), axis=2))
    hi_s = e8m0_code(np.max(np.abs(t3) + d3, axis=2))
    bad_s = (gs < lo_s) | (gs > hi_s)
    if bad_s.any():
        r, q = np.argwhere(bad_s)[0]
        raise AssertionError("%s: %d scales outside their reachable range; first row %d group %d: got %d, reachable "
                             "%d .. %d (oracle %d)" % (what, int(bad_s.sum()), r, q, gs[r, q], lo_s[r, q],
                                                       hi_s[r, q], os_[r, q]))
    X = np.ldexp(1.0, gs - 127)[:, :, None]
    lo = _ladder(t3 - d3, X)
    hi = _ladder(t3 + d3, X)
    zero = (gn & 7) == 0
    neg = (gn & 8) != 0
    bad = (gp < lo) | (gp > hi)
    bad |= zero & neg & (t3 - d3 > 0)
    bad |= zero & ~neg & (t3 + d3 < 0)
    bad |= (gs == os_)[:, :, None] & (np.abs(gp - op) > 1)
    if bad.any():
        r, q, j = np.argwhere(bad)[0]
        raise AssertionError("%s: %d codes that no value within the bound rounds to; first row %d element %d: got "
                             "%d, oracle %d, t %r, bound %r, scale %d (oracle %d)"
                             % (what, int(bad.sum()), r, 32 * q + j, gn[r, q, j], on[r, q, j], t3[r, q, j],
                                d3[r, q, j], gs[r, q], os_[r, q]))
    return int(np.count_nonzero(gn != on)), int(np.count_nonzero(gs != os_))


class DnStats:
    def __init__(self):
        self.rows = self.codes = self.code_diffs = self.scales = self.scale_diffs = self.rows_diff = 0

    def __str__(self):
        return ("%d rows, %d of %d codes and %d of %d scales differ (%d rows)"
                % (self.rows, self.code_diffs, self.codes, self.scale_diffs, self.scales, self.rows_diff))


def oracle_down_inputs(orc, c, prep, want=None):
    """Per expert: (rows, act codes, act scales, gate/up fp64 [n, 2F], h fp32,
    down codes, down scales) for its routed rows (of wanted tokens only, when
    `want` is given): the oracle's gate/up layer, SiLU * up, and the down
    projection's quantizer, step by step."""
    a_gu, gc, gs, a_dn, _, _ = prep
    off, tok, _ = orc.moe_route(c.ids, c.E)
    xb = inputs.bf16_bits(c.x)
    for e in range(c.E):
        rows = np.arange(off[e], off[e + 1])
        if want is not None:
            rows = rows[want[tok[rows]]]
        if not rows.size:
            continue
        ac, as_ = orc.quant_rows(xb[tok[rows]], None if a_gu is None else a_gu[e], c.b)
        gu = orc.gemm_codes(ac, as_, gc[e], gs[e])
        h = orc.silu_mul(gu)
        hc, hs = orc.quant_rows(h, None if a_dn is None else a_dn[e], c.b)
        yield e, rows, ac, as_, gu, h, hc, hs


def check_down_input(orc, c, prep, g_codes, g_scales, want=None, what="down input"):
    """The GPU's down input (row-major codes / scales of every routed row)
    against the oracle's: equal, or within dn_input_bound (check_slips).
    Returns (DnStats, the oracle's codes, the oracle's scales)."""
    from parity_util import accumulation_bound
    a_dn = prep[3]
    st = DnStats()
    o_c = np.zeros_like(g_codes)
    o_s = np.zeros_like(g_scales)
    for e, rows, ac, as_, gu, h, hc, hs in oracle_down_inputs(orc, c, prep, want):
        o_c[rows], o_s[rows] = hc, hs
        st.rows += rows.size
        st.codes += 2 * hc.size
        st.scales += hs.size
        diff = (g_codes[rows] != hc).any(axis=1) | (g_scales[rows] != hs).any(axis=1)
        if not diff.any():
            continue
        d = np.nonzero(diff)[0]
        ad = None if a_dn is None else a_dn[e]
        b_gu = accumulation_bound(orc, ac[d], as_[d], prep[1][e], prep[2][e], c.H)
        t = orc.transform_rows(h[d], ad, c.b)
        dt = dn_input_bound(gu[d], b_gu, h[d], ad, c.b)
        nc, ns = check_slips(g_codes[rows[d]], g_scales[rows[d]], hc[d], hs[d], t, dt,
                             "%s (expert %d)" % (what, e))
        st.code_diffs += nc
        st.scale_diffs += ns
        st.rows_diff += d.size
    return st, o_c, o_s


def down_combine_reference(orc, c, prep, d_codes, d_scales, tokens):
    """Reference and per-output bound for the down projection and combine of
    the given tokens, on the down input (d_codes, d_scales) of every routed
    row (row-major): each expert row D = the oracle's fp64 GEMM over those
    codes, rounded to bf16; y = sum_j w[t, j] * RN_bf16(D_j) in fp64 in slot
    order. The GPU's row is RN_bf16 of an fp32 sum within B (the
    accumulation bound) of D, so within Delta = the larger step from
    RN_bf16(D) to RN_bf16(D -+ B) of the reference row; its combine adds k
    fp32 fused multiply-adds. Bound: sum_j |w| Delta_j +
    gamma_k sum_j |w| (|RN_bf16(D_j)| + Delta_j)."""
    from parity_util import accumulation_bound
    dc, ds = prep[4], prep[5]
    T, k, H, F = c.T, c.k, c.H, c.F
    tokens = np.asarray(tokens, np.int64)
    off, tok, pos = orc.moe_route(c.ids, c.E)
    p = pos.reshape(T, k)
    need = np.zeros(T, bool)
    need[tokens] = True
    rows = np.nonzero(need[tok[:off[-1]]])[0]
    slot = np.full(max(int(off[-1]), 1), -1, np.int64)
    slot[rows] = np.arange(rows.size)
    d_ref = np.zeros((rows.size, H))
    delta = np.zeros((rows.size, H))
    for e in range(c.E):
        r = rows[(rows >= off[e]) & (rows < off[e + 1])]
        if not r.size:
            continue
        D = orc.gemm_codes(d_codes[r], d_scales[r], dc[e], ds[e])
        B = accumulation_bound(orc, d_codes[r], d_scales[r], dc[e], ds[e], F)
        d = rn_bf16(D)
        d_ref[slot[r]] = d
        delta[slot[r]] = np.maximum(rn_bf16(D + B) - d, d - rn_bf16(D - B))
    y = np.zeros((tokens.size, H))
    mag = np.zeros((tokens.size, H))
    dev = np.zeros((tokens.size, H))
    for j in range(k):
        r = p[tokens, j]
        ok = r >= 0
        s = slot[np.where(ok, r, 0)]
        wj = c.w[tokens, j].astype(np.float64)[:, None]
        y += np.where(ok[:, None], wj * d_ref[s], 0.0)
        mag += np.where(ok[:, None], np.abs(wj) * (np.abs(d_ref[s]) + delta[s]), 0.0)
        dev += np.where(ok[:, None], np.abs(wj) * delta[s], 0.0)
    gam = k * U32 / (1.0 - k * U32)
    return y, dev + gam * mag + k * 2.0 ** -149
