"""Pins of the oracle's Hessian and Flip-Refinement to things other than
themselves: the Hessian against numpy's product of the (pinned) transformed
rows; the refinement against closed forms (a diagonal Hessian leaves
round-to-nearest alone, a zero cap changes nothing), against an independent
numpy restatement of the greedy rule that evaluates every candidate move's
objective from scratch, and against the properties the method promises (the
objective never increases, the result is a local minimum under single
adjacent moves, the block scales stay, the held-out output error drops).
"""
import numpy as np
import pytest

from mxfp4_w4a4_post_amd import inputs

LUT = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _index(codes):
    """signed E2M1 index (-7..7) of every element of row-major packed codes"""
    nib = np.stack([codes & 0xF, codes >> 4], axis=-1).reshape(codes.shape[0], -1).astype(np.int64)
    mag = nib & 7
    return np.where(nib & 8, -mag, mag)


def _values(m, scales):
    v = np.sign(m) * LUT[np.abs(m)]
    return v * np.exp2(np.repeat(scales.astype(np.float64) - 127.0, 32, axis=1))


def _objective(wt, m, scales, H):
    e = wt.astype(np.float64) - _values(m, scales)
    return np.einsum("nk,kj,nj->n", e, H, e)


def _case(K=64, N=6, R=256, b=32, seed=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((R, K)).astype(np.float32)
    x[:, rng.choice(K, 2, replace=False)] *= 20.0
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    return inputs.bf16_bits(inputs.to_bf16(x)), inputs.bf16_bits(inputs.to_bf16(w)), b


def _prepared(orc, xb, wb, b):
    a, r = orc.multipliers(orc.calibrate(xb), b)
    codes, scales = orc.prepare_weights(wb, r, b)
    wt = orc.transform_rows(wb, r, b)
    return a, r, codes, scales, wt


def test_hessian_is_gram_of_transformed_rows(orc):
    xb, wb, b = _case()
    a, r = orc.multipliers(orc.calibrate(xb), b)
    H = orc.hessian(xb, a, b)
    xt = orc.transform_rows(xb, a, b).astype(np.float64)
    ref = xt.T @ xt
    assert np.allclose(H, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    assert np.array_equal(H, H.T)  # same products, same order
    assert np.linalg.eigvalsh(H).min() > -1e-9 * np.abs(H).max()


def test_refine_zero_cap_changes_nothing(orc):
    xb, wb, b = _case()
    a, r, codes, scales, _ = _prepared(orc, xb, wb, b)
    out, flips = orc.flip_refine(wb, r, b, orc.hessian(xb, a, b), 0, codes, scales)
    assert np.array_equal(out, codes) and not flips.any()


def test_refine_diagonal_hessian_keeps_round_to_nearest(orc):
    """With H diagonal the objective splits per element, and round-to-nearest
    (ties at exact midpoints cost nothing to keep) is already optimal."""
    xb, wb, b = _case()
    _, r, codes, scales, _ = _prepared(orc, xb, wb, b)
    K = codes.shape[1] * 2
    rng = np.random.default_rng(5)
    for H in (np.eye(K), np.diag(rng.uniform(0.1, 10.0, K))):
        out, flips = orc.flip_refine(wb, r, b, H, 1000, codes, scales)
        assert not flips.any() and np.array_equal(out, codes)


def test_refine_never_increases_and_ends_in_local_minimum(orc):
    xb, wb, b = _case(seed=3)
    a, r, codes, scales, wt = _prepared(orc, xb, wb, b)
    H = orc.hessian(xb, a, b)
    m0 = _index(codes)
    before = _objective(wt, m0, scales, H)
    prev = before
    for cap in (1, 2, 5, 10, 20, 10000):
        out, flips = orc.flip_refine(wb, r, b, H, cap, codes, scales)
        obj = _objective(wt, _index(out), scales, H)
        assert np.all(obj <= prev * (1 + 1e-12) + 1e-18), cap
        assert np.all(flips <= cap)
        prev = obj
    m = _index(out)
    assert np.any(m != m0)
    assert np.all(np.abs(m - m0).sum(axis=1) <= flips)
    scale_tol = 1e-9 * np.abs(prev).max()
    for n in range(m.shape[0]):
        for k in range(m.shape[1]):
            for d in (-1, 1):
                if not -7 <= m[n, k] + d <= 7:
                    continue
                mm = m[n:n + 1].copy()
                mm[0, k] += d
                assert _objective(wt[n:n + 1], mm, scales[n:n + 1], H)[0] >= prev[n] - scale_tol


def _numpy_greedy(wt, codes, scales, H, cap):
    """Independent restatement: each step evaluates every single adjacent move
    by the full objective and takes the best (lowest k, then down, on ties)."""
    m = _index(codes)
    out = []
    for n in range(m.shape[0]):
        row = m[n:n + 1].copy()
        cur = _objective(wt[n:n + 1], row, scales[n:n + 1], H)[0]
        for _ in range(cap):
            best, arg = cur, None
            for k in range(row.shape[1]):
                for d in (-1, 1):
                    if not -7 <= row[0, k] + d <= 7:
                        continue
                    row[0, k] += d
                    val = _objective(wt[n:n + 1], row, scales[n:n + 1], H)[0]
                    row[0, k] -= d
                    if val < best:
                        best, arg = val, (k, d)
            if arg is None:
                break
            row[0, arg[0]] += arg[1]
            cur = best
        out.append(row[0])
    return np.array(out)


def test_refine_matches_numpy_greedy(orc):
    xb, wb, b = _case(K=64, N=4, seed=7)
    a, r, codes, scales, wt = _prepared(orc, xb, wb, b)
    H = orc.hessian(xb, a, b)
    out, flips = orc.flip_refine(wb, r, b, H, 12, codes, scales)
    assert np.array_equal(_index(out), _numpy_greedy(wt, codes, scales, H, 12))


def test_refine_canonical_codes_only_where_moved(orc):
    """Moved elements take the canonical code of their index; the rest keep
    their bits (a -0 that never moves stays 0x8)."""
    xb, wb, b = _case(seed=9)
    a, r, codes, scales, _ = _prepared(orc, xb, wb, b)
    out, _ = orc.flip_refine(wb, r, b, orc.hessian(xb, a, b), 30, codes, scales)
    nib0 = np.stack([codes & 0xF, codes >> 4], axis=-1).reshape(codes.shape[0], -1)
    nib1 = np.stack([out & 0xF, out >> 4], axis=-1).reshape(out.shape[0], -1)
    moved = _index(codes) != _index(out)
    assert np.array_equal(nib1[~moved], nib0[~moved])
    mm = _index(out)[moved]
    assert np.array_equal(nib1[moved], np.where(mm < 0, 8 - mm, mm))


def test_refine_lowers_heldout_output_error(orc):
    """Refined on enough calibration rows, the prepared weights reproduce W x
    better than round-to-nearest on fresh rows of the same distribution."""
    K, N = 128, 16
    c = inputs.linear_case(1, 0, M=64, K=K, N=N)
    xcal = inputs.bf16_bits(inputs.activations(1, 0, 2048, K, stream=1))
    xb = inputs.bf16_bits(c.xcal)
    wb = inputs.bf16_bits(c.w)
    a, r = orc.multipliers(orc.calibrate(xb), 32)
    codes, scales = orc.prepare_weights(wb, r, 32)
    out, flips = orc.flip_refine(wb, r, 32, orc.hessian(xcal, a, 32), 64, codes, scales)
    assert flips.sum() > 0
    xe = inputs.bf16_bits(c.x)
    xt = orc.transform_rows(xe, a, 32).astype(np.float64)
    exact = xe.view(np.uint16).astype(np.uint32) << 16
    y = exact.view(np.float32).astype(np.float64) @ wb.astype(np.uint32).__lshift__(16).view(np.float32).T

    def err(cds):
        q = orc.dequant_rows(cds, scales)
        return np.linalg.norm(xt @ q.T - y)

    assert err(out) < 0.97 * err(codes)
