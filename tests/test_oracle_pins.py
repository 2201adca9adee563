"""Pins of the CPU oracle to things other than itself.

Each test checks the oracle against a closed form, a library routine, a
hand-worked value or brute force, chosen so that a plausible slip (a dropped
term, a wrong sign or index, a transposed operand, the wrong direction of the
per-channel scale, the wrong stage order) fails at least one of them.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def f32_bits(x):
    return int(np.array([x], np.float32).view(np.uint32)[0])


def bits_f32(u):
    return float(np.array([u], np.uint32).view(np.float32)[0])


def next_up(x):
    return float(np.nextafter(np.float32(x), np.float32(np.inf)))


def next_down(x):
    return float(np.nextafter(np.float32(x), np.float32(-np.inf)))


def is_nearest_f32(value: float, exact: Fraction) -> bool:
    """value is an fp32 nearest to `exact` (compared in exact rationals)."""
    d = abs(Fraction(value) - exact)
    return d <= abs(Fraction(next_up(value)) - exact) and d <= abs(Fraction(next_down(value)) - exact)


# ---------------------------------------------------------------------------
# Block-Hadamard
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("b", [32, 64, 128])
def test_fwht_equals_sylvester_matrix(orc, b):
    """The transform of the unit vectors gives Sylvester's H_b (scipy's
    natural-order construction), so S_b[i][j] = (-1)^popcount(i & j)."""
    eye = np.eye(b, dtype=np.float32)
    t = orc.transform_rows(eye, None, b)  # row j is S_b e_j = column j of S_b
    S = t.T
    ref = scipy.linalg.hadamard(b).astype(np.float32)
    assert np.array_equal(S, ref)
    i = np.arange(b)
    pop = np.vectorize(lambda v: bin(v).count("1"))(i[:, None] & i[None, :])
    assert np.array_equal(S, np.where(pop % 2 == 0, 1.0, -1.0).astype(np.float32))


@pytest.mark.parametrize("b", [32, 64, 128])
def test_hadamard_orthogonal_in_integers(orc, b):
    S = orc.transform_rows(np.eye(b, dtype=np.float32), None, b).astype(np.int64)
    assert np.array_equal(S @ S.T, b * np.eye(b, dtype=np.int64))


def test_fwht_worked_example(orc):
    """[1, 2, 3, 4] under the order-4 Sylvester matrix is [10, -2, -4, 0]; with the
    vector zero-padded to a 32-block, row i of S_32 restricted to j < 4 equals row
    i mod 4 of S_4, so the 32 outputs repeat that pattern."""
    v = np.zeros((1, 32), np.float32)
    v[0, :4] = [1, 2, 3, 4]
    t = orc.transform_rows(v, None, 32)[0]
    assert np.array_equal(t, np.tile(np.array([10, -2, -4, 0], np.float32), 8))


@pytest.mark.parametrize("b", [32, 64, 128])
def test_fwht_twice_is_b_times_identity(orc, b):
    rng = np.random.default_rng(7)
    v = rng.integers(-8, 9, size=(3, 2 * b)).astype(np.float32)
    t = orc.transform_rows(v, None, b)
    tt = orc.transform_rows(t, None, b)
    assert np.array_equal(tt, b * v)


def test_blocks_are_contiguous_and_independent(orc):
    """Each aligned b-block of K is transformed on its own."""
    rng = np.random.default_rng(8)
    v = rng.integers(-8, 9, size=(2, 128)).astype(np.float32)
    whole = orc.transform_rows(v, None, 32)
    for j in range(4):
        part = orc.transform_rows(np.ascontiguousarray(v[:, 32 * j:32 * (j + 1)]), None, 32)
        assert np.array_equal(whole[:, 32 * j:32 * (j + 1)], part)
    H = scipy.linalg.hadamard(32)
    assert np.array_equal(whole[:, 32:64], (v[:, 32:64].astype(np.int64) @ H.T).astype(np.float32))


def test_stage_order_rounding(orc):
    """The fp32 rounding follows stages of span 1, 2, 4, ... in that order.
    With v = [1, e, 0, e, 0...], e = 2^-24: span 1 gives 1 + e -> 1 (a tie,
    to even) and 0 + e = e; span 2 gives 1 + e -> 1 again. Output 0 is exactly
    1.0. (Span 2 first would give 1 and 2e, then 1 + 2e = 1 + 2^-23.)"""
    e = 2.0 ** -24
    v = np.zeros((1, 32), np.float32)
    v[0, 0], v[0, 1], v[0, 3] = 1.0, e, e
    t = orc.transform_rows(v, None, 32)[0]
    assert t[0] == np.float32(1.0)


def test_multiply_comes_before_hadamard(orc):
    """t = S_b (m * x): with m a power of two per channel and integer x the
    result is exact and equals the integer matrix product."""
    rng = np.random.default_rng(9)
    x = rng.integers(-4, 5, size=(2, 64)).astype(np.float32)
    m = (2.0 ** rng.integers(-2, 3, size=64)).astype(np.float32)
    t = orc.transform_rows(x, m, 64)
    H = scipy.linalg.hadamard(64).astype(np.float64)
    assert np.array_equal(t.astype(np.float64), (x.astype(np.float64) * m) @ H.T)


# ---------------------------------------------------------------------------
# Per-channel scale and multipliers
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("b,bits", [(32, 0x3E3504F3), (64, 0x3E000000), (128, 0x3DB504F3)])
def test_c_b_is_rounded_inverse_sqrt(orc, b, bits):
    """c_b = RN32(1/sqrt(b)): 1/sqrt(32) = sqrt(2)/8 and 1/sqrt(128) = sqrt(2)/16,
    whose fp32 roundings are 0x3E3504F3 and 0x3DB504F3; 1/sqrt(64) = 0.125."""
    a, r = orc.multipliers(np.ones(4, np.float32), b)
    assert all(f32_bits(v) == bits for v in a) and all(f32_bits(v) == bits for v in r)
    # the exact value: c^2 * b brackets 1 within one fp32 ulp of c
    c = Fraction(bits_f32(bits))
    lo, hi = Fraction(next_down(float(c))), Fraction(next_up(float(c)))
    assert ((c + lo) / 2) ** 2 * b <= 1 <= ((c + hi) / 2) ** 2 * b


def test_multipliers_correctly_rounded(orc):
    rng = np.random.default_rng(10)
    s = (rng.random(200) * 10 + 0.01).astype(np.float32)
    for b in (0, 32, 64, 128):
        a, r = orc.multipliers(s, b)
        c = Fraction(1) if b == 0 else Fraction(float(orc.multipliers(np.ones(1, np.float32), b)[0][0]))
        for k in range(0, 200, 7):
            assert is_nearest_f32(float(a[k]), c / Fraction(float(s[k])))
            assert is_nearest_f32(float(r[k]), c * Fraction(float(s[k])))


def test_calibrate_is_rounded_sqrt_of_column_max(orc):
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((64, 96)) * 3).astype(np.float32)
    x[:, 5] = 0.0
    x[17, 9] = -40.0  # a negative outlier sets the max of |x|
    s = orc.calibrate(x)
    assert s[5] == 1.0
    for k in range(96):
        if k == 5:
            continue
        mx = Fraction(float(np.max(np.abs(x[:, k]))))
        v = Fraction(float(s[k]))
        # v is the fp32 nearest to sqrt(mx): the two half-ulp neighbours bracket it
        lo = (v + Fraction(next_down(float(v)))) / 2
        hi = (v + Fraction(next_up(float(v)))) / 2
        assert lo * lo <= mx <= hi * hi
    assert f32_bits(s[9]) == f32_bits(np.float32(math.sqrt(40.0)))
    # order of the rows does not matter; bf16 input gives the same as its fp32 widening
    assert np.array_equal(orc.calibrate(x[::-1].copy()), s)
    xb = (x.view(np.uint32) >> 16).astype(np.uint16)
    xw = (xb.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(orc.calibrate(xb), orc.calibrate(xw))


# ---------------------------------------------------------------------------
# MX encoding
# ---------------------------------------------------------------------------

def _golden_cases():
    with open(os.path.join(GOLDEN, "mx_hand_worked.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["what"][:40])
def test_mx_hand_worked(orc, case):
    v = np.array([case["values"]], np.float32)
    codes, scales = orc.quant_rows(v, None, 0)
    assert int(scales[0, 0]) == case["scale"]
    assert list(codes[0]) == case["bytes"]
    unpacked = [(byte >> (4 * h)) & 0xF for byte in codes[0] for h in (0, 1)]
    assert unpacked == case["codes"]


def _rint_e2m1(u: np.ndarray) -> np.ndarray:
    """E2M1 round-to-nearest-even through numpy's rint (round half to even):
    below 2 the grid step is 0.5, in [2, 4) it is 1, in [4, 8) it is 2; the
    rounded value is then saturated at 6 and mapped to its code."""
    step = np.where(u < 2, 0.5, np.where(u < 4, 1.0, 2.0))
    q = np.rint(u / step) * step
    q = np.minimum(q, 6.0)
    lut = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    return np.searchsorted(lut, q)


def test_e2m1_rounding_against_rint(orc):
    """Magnitudes on a fine grid over [0, 8) and one ulp either side of every
    midpoint, with the scale pinned to 1 by a 7.5 in each group."""
    grid = np.arange(0, 8, 1 / 128, dtype=np.float64)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    extra = np.concatenate([mids, np.nextafter(mids.astype(np.float32), 0), np.nextafter(mids.astype(np.float32), 9)])
    u = np.concatenate([grid, extra.astype(np.float64)]).astype(np.float32)
    n_groups = int(np.ceil(len(u) / 31))
    vals = np.zeros(n_groups * 31, np.float32)
    vals[:len(u)] = u
    rows = np.concatenate([np.full((n_groups, 1), 7.5, np.float32), vals.reshape(n_groups, 31)], axis=1)
    codes, scales = orc.quant_rows(rows.reshape(1, -1), None, 0)
    assert np.all(scales == 127)
    c = np.stack([codes[0] & 0xF, codes[0] >> 4], axis=1).reshape(n_groups, 32)[:, 1:].reshape(-1)
    expect = _rint_e2m1(vals.astype(np.float64))
    assert np.array_equal(c, expect)


def test_scale_brackets_amax(orc):
    """Away from the clamp the E8M0 scale X satisfies 4 X <= amax < 8 X,
    i.e. the block maximum lands in E2M1's top binade."""
    rng = np.random.default_rng(12)
    v = (rng.standard_normal((8, 32 * 64)) * np.exp(rng.uniform(-20, 20, size=(8, 1)))).astype(np.float32)
    codes, scales = orc.quant_rows(v, None, 0)
    g = v.reshape(8, 64, 32)
    amax = np.abs(g).max(axis=2).astype(np.float64)
    X = np.ldexp(1.0, scales.astype(np.int64) - 127)
    assert np.all(4 * X <= amax) and np.all(amax < 8 * X)


def test_quantizer_properties(orc):
    rng = np.random.default_rng(13)
    v = (rng.standard_normal((4, 256)) * 2).astype(np.float32)
    c0, s0 = orc.quant_rows(v, None, 0)
    # Q(-v): only sign bits change
    c1, s1 = orc.quant_rows(-v, None, 0)
    assert np.array_equal(s1, s0) and np.array_equal(c1, c0 ^ 0x88)
    # Q(2^j v): same codes, scale moves by j
    for j in (-5, 3, 40):
        cj, sj = orc.quant_rows((v * np.float32(2.0 ** j)).astype(np.float32), None, 0)
        assert np.array_equal(cj, c0) and np.array_equal(sj.astype(int), s0.astype(int) + j)
    # permuting inside a group permutes the codes
    perm = rng.permutation(32)
    vp = v.reshape(4, 8, 32)[:, :, perm].reshape(4, 256)
    cp, sp = orc.quant_rows(vp, None, 0)

    def unpack(c):
        return np.stack([c & 0xF, c >> 4], axis=-1).reshape(4, 8, 32)

    assert np.array_equal(sp, s0) and np.array_equal(unpack(cp), unpack(c0)[:, :, perm])
    # Q(dq(Q(v))) = Q(v)
    dq = orc.dequant_rows(c0, s0).astype(np.float32)
    c2, s2 = orc.quant_rows(dq, None, 0)
    assert np.array_equal(c2, c0) and np.array_equal(s2, s0)


def test_dequant_brute_force(orc):
    rng = np.random.default_rng(14)
    codes = rng.integers(0, 256, size=(3, 32), dtype=np.uint8)
    scales = rng.integers(100, 150, size=(3, 2), dtype=np.uint8)
    out = orc.dequant_rows(codes, scales)
    for r in range(3):
        for k in range(64):
            nib = (int(codes[r, k // 2]) >> (4 * (k % 2))) & 0xF
            mag = E2M1[nib & 7] * Fraction(2) ** (int(scales[r, k // 32]) - 127)
            assert Fraction(float(out[r, k])) == (-mag if nib & 8 else mag)


# ---------------------------------------------------------------------------
# GEMM over codes
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,K,N", [(4, 32, 32), (4, 64, 64), (3, 96, 5)])
def test_gemm_codes_brute_force(orc, M, K, N):
    """Exact rational dot products of decoded codes equal the fp64 result."""
    rng = np.random.default_rng(M * 1000 + K + N)
    ac = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    as_ = rng.integers(118, 136, size=(M, K // 32), dtype=np.uint8)
    wc = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    ws = rng.integers(118, 136, size=(N, K // 32), dtype=np.uint8)

    def dec(c, s, r, k):
        nib = (int(c[r, k // 2]) >> (4 * (k % 2))) & 0xF
        mag = E2M1[nib & 7] * Fraction(2) ** (int(s[r, k // 32]) - 127)
        return -mag if nib & 8 else mag

    y = orc.gemm_codes(ac, as_, wc, ws, threads=2)
    assert y.shape == (M, N)
    for m in range(M):
        for n in range(N):
            exact = sum(dec(ac, as_, m, k) * dec(wc, ws, n, k) for k in range(K))
            assert Fraction(float(y[m, n])) == exact


# ---------------------------------------------------------------------------
# The transformed pair reproduces y = W x
# ---------------------------------------------------------------------------

def test_transform_pair_exact_before_quantization(orc):
    """With b = 64 (c_b = 1/8) and per-channel scales that are powers of two,
    every fp32 step is exact, so (H D W^T)-side and (H D x)-side products give
    W x exactly in fp64."""
    rng = np.random.default_rng(15)
    K, N, M = 128, 16, 4
    s = (2.0 ** rng.integers(-2, 3, size=K)).astype(np.float32)
    a, r = orc.multipliers(s, 64)
    x = rng.integers(-6, 7, size=(M, K)).astype(np.float32)
    w = rng.integers(-6, 7, size=(N, K)).astype(np.float32)
    tx = orc.transform_rows(x, a, 64).astype(np.float64)
    tw = orc.transform_rows(w, r, 64).astype(np.float64)
    assert np.array_equal(tx @ tw.T, x.astype(np.float64) @ w.astype(np.float64).T)


@pytest.mark.parametrize("b", [32, 64, 128])
def test_transform_pair_close_before_quantization(orc, b):
    """Random data: the pair agrees with W x to fp32 transform accuracy."""
    rng = np.random.default_rng(16 + b)
    K, N, M = 512, 64, 8
    xcal = rng.standard_normal((64, K)).astype(np.float32)
    xcal[:, 3] *= 50
    s = orc.calibrate(xcal)
    a, r = orc.multipliers(s, b)
    x = rng.standard_normal((M, K)).astype(np.float32)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    tx = orc.transform_rows(x, a, b).astype(np.float64)
    tw = orc.transform_rows(w, r, b).astype(np.float64)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    assert np.linalg.norm(tx @ tw.T - ref) / np.linalg.norm(ref) < 1e-5


def _grid_pair(rng, M, N, K, s):
    """x and w whose transformed rows land exactly on MXFP4 grids (b = 64):
    targets t have two non-zeros per 32-group, 2 and +-1 (or 0), so their
    quantization is lossless; x_k = (S t)_k s_k / 8, w_k = (S u)_k / (8 s_k)."""
    S = scipy.linalg.hadamard(64).astype(np.float64)

    def targets(rows):
        t = np.zeros((rows, K))
        for r_ in range(rows):
            for g in range(K // 32):
                i, j = rng.choice(32, size=2, replace=False)
                t[r_, 32 * g + i] = 2.0 * rng.choice([-1, 1])
                t[r_, 32 * g + j] = rng.choice([-1.0, 0.0, 1.0])
        return t

    def unblock(t):
        return (t.reshape(t.shape[0], K // 64, 64) @ S.T).reshape(t.shape[0], K)

    tx, tw = targets(M), targets(N)
    x = unblock(tx) * s / 8
    w = unblock(tw) / (8 * s)
    return x, w, tx, tw


def test_linear_end_to_end_exact_on_grid(orc):
    """y = W' Q(H D x) equals W x exactly when the transformed rows are
    representable: this pins the direction of D (activations divided by s),
    the multiply-then-Hadamard order, the packing and the GEMM together."""
    rng = np.random.default_rng(17)
    M, N, K = 5, 24, 256
    s = (2.0 ** rng.integers(-1, 2, size=K)).astype(np.float64)
    x, w, tx, tw = _grid_pair(rng, M, N, K, s)
    xb = x.astype(np.float32)
    assert np.array_equal(xb.astype(np.float64), x)
    xbits = (xb.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((xbits.astype(np.uint32) << 16).view(np.float32), xb)  # exact in bf16
    a, r = orc.multipliers(s.astype(np.float32), 64)
    wc, ws = orc.prepare_weights(w.astype(np.float32), r, 64)
    y = orc.linear(xbits, a, 64, wc, ws, threads=2)
    assert np.array_equal(y, x @ w.T)
    assert np.array_equal(y, tx @ tw.T)
    # the literal "multiply the activations by s" reading does not reproduce W x
    wc2, ws2 = orc.prepare_weights(w.astype(np.float32), a, 64)
    y2 = orc.linear(xbits, r, 64, wc2, ws2, threads=2)
    assert not np.allclose(y2, x @ w.T, rtol=1e-3)


def test_linear_matches_quant_then_gemm(orc):
    rng = np.random.default_rng(18)
    x = (rng.standard_normal((6, 128))).astype(np.float32)
    xbits = (x.view(np.uint32) >> 16).astype(np.uint16)
    w = (rng.standard_normal((10, 128)) * 0.02).astype(np.float32)
    s = orc.calibrate(xbits)
    a, r = orc.multipliers(s, 32)
    wc, ws = orc.prepare_weights(w, r, 32)
    ac, as_ = orc.quant_rows(xbits, a, 32)
    assert np.array_equal(orc.linear(xbits, a, 32, wc, ws), orc.gemm_codes(ac, as_, wc, ws))


def test_linear_grouped_is_per_expert(orc):
    rng = np.random.default_rng(19)
    E, K, N = 4, 64, 8
    off = np.array([0, 3, 3, 10, 12], np.int32)  # expert 1 has no rows
    x = rng.standard_normal((12, K)).astype(np.float32)
    xbits = (x.view(np.uint32) >> 16).astype(np.uint16)
    a = (rng.random((E, K)) + 0.5).astype(np.float32)
    wc = rng.integers(0, 256, size=(E, N, K // 2), dtype=np.uint8)
    ws = rng.integers(120, 130, size=(E, N, K // 32), dtype=np.uint8)
    y = orc.linear_grouped(xbits, off, a, 32, wc, ws)
    for e in range(E):
        lo, hi = off[e], off[e + 1]
        if hi == lo:
            continue
        ye = orc.linear(np.ascontiguousarray(xbits[lo:hi]), a[e], 32, wc[e], ws[e])
        assert np.array_equal(y[lo:hi], ye)
    with pytest.raises(ValueError):
        orc.linear_grouped(xbits, np.array([0, 3, 2, 10, 12], np.int32), a, 32, wc, ws)


def test_quantization_error_prefers_dividing_by_s(orc):
    """Evidence for the reading of D on the tiny workload's distribution:
    dividing the activations by s (and multiplying weight columns by it)
    gives a smaller output error than the other direction or no D."""
    rng = np.random.default_rng(20)
    K, N, M = 256, 256, 16
    chans = rng.choice(K, 4, replace=False)
    xcal = rng.standard_normal((64, K)).astype(np.float32)
    x = rng.standard_normal((M, K)).astype(np.float32)
    xcal[:, chans] *= 50
    x[:, chans] *= 50
    xbits = (x.view(np.uint32) >> 16).astype(np.uint16)
    xw = (xbits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    ref = xw @ w.astype(np.float64).T
    s = orc.calibrate(xcal)

    def err(amul, wmul, b):
        wc, ws = orc.prepare_weights(w, wmul, b)
        y = orc.linear(xbits, amul, b, wc, ws)
        return np.linalg.norm(y - ref) / np.linalg.norm(ref)

    a, r = orc.multipliers(s, 32)
    e_div = err(a, r, 32)
    e_mul = err(r, a, 32)
    e_none = err(*orc.multipliers(np.ones(K, np.float32), 32), 32)
    assert e_div < e_none < e_mul
