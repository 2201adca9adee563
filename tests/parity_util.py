"""Comparison helpers for the GPU parity tests (HIP path vs the CPU oracle)."""
import sys

import numpy as np
import torch

# Output tolerance: relative L2 error of the fp32 output against the oracle's
# fp64 accumulation of the same codes.
REL_L2_TOL = 1e-3
# Code tolerance: at most this fraction of codes may differ, each by one step
# of magnitude at a rounding tie within one fp32 ulp of the oracle's value.
CODE_SLIP_FRACTION = 1e-5


def log(msg: str):
    print("[parity] " + msg, flush=True)
    sys.stdout.flush()


def np_u8(t) -> np.ndarray:
    if isinstance(t, np.ndarray):
        return t
    return t.detach().cpu().numpy()


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def rel_l2(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def unpack(codes: np.ndarray) -> np.ndarray:
    return np.stack([codes & 0xF, codes >> 4], axis=-1).reshape(codes.shape[0], -1)


_MIDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def assert_quant_equal(g_codes, g_scales, o_codes, o_scales, t_oracle=None, what=""):
    """Scales bit-exact; codes bit-exact except for the allowed tie slips."""
    g_codes, o_codes = np.asarray(g_codes), np.asarray(o_codes)
    assert np.array_equal(np.asarray(g_scales), np.asarray(o_scales)), "%s: E8M0 scales differ" % what
    if np.array_equal(g_codes, o_codes):
        return
    gu, ou = unpack(g_codes), unpack(o_codes)
    bad = np.argwhere(gu != ou)
    frac = len(bad) / gu.size
    assert t_oracle is not None, "%s: %d codes differ and no pre-quant values to check ties against" % (what, len(bad))
    assert frac <= CODE_SLIP_FRACTION, "%s: %d codes differ (%.2e of all)" % (what, len(bad), frac)
    sc = np.asarray(o_scales).astype(np.int64)
    for r, k in bad:
        gcode, ocode = int(gu[r, k]), int(ou[r, k])
        assert (gcode & 8) == (ocode & 8) and abs((gcode & 7) - (ocode & 7)) == 1, \
            "%s: code %d vs %d at (%d, %d) not adjacent" % (what, gcode, ocode, r, k)
        t = np.float32(t_oracle[r, k])
        u = abs(float(t)) * 2.0 ** (127 - sc[r, k // 32])
        ulp = float(np.spacing(np.float32(abs(t)))) * 2.0 ** (127 - sc[r, k // 32])
        assert np.min(np.abs(_MIDS - u)) <= ulp, "%s: slip at (%d, %d) is not at a tie" % (what, r, k)


def abs_codes(codes) -> np.ndarray:
    """The same packed E2M1 codes with both sign bits cleared: |value|."""
    return np.asarray(codes, np.uint8) & np.uint8(0x77)


def accumulation_bound(oracle, a_codes, a_scales, w_codes, w_scales, K: int) -> np.ndarray:
    """Per-output bound on the fp32 accumulation error of the GPU GEMM.

    Every product of two E2M1 values at E8M0 scales is exact in fp32, so
    the GPU's result differs from the exact sum only by the roundings of
    its fp32 additions. Each partial sum is bounded by
    S[m, n] = sum_k |a_mk| |w_nk| (the oracle's GEMM over the codes with
    the sign bits cleared), so with at most 4 roundings per 64-element
    matrix-core step plus the split-K partial sums (at most K/1024 + 2)
    the error is at most n_r * 2^-24 * S[m, n] (first-order bound, each
    rounding off by at most half an ulp of a value below S: the classical
    gamma_n bound of recursive summation)."""
    n_r = 4 * -(-K // 64) + -(-K // 1024) + 2
    u = 2.0 ** -24
    S = oracle.gemm_codes(abs_codes(a_codes), a_scales, abs_codes(w_codes), w_scales)
    return (n_r * u / (1.0 - n_r * u)) * S + 2.0 ** -149


def assert_elementwise(got, ref, bound, what=""):
    """Every output within its own bound of the oracle's exact value."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    err = np.abs(got - ref)
    bad = err > bound
    if bad.any():
        i = np.unravel_index(int(np.argmax(err - bound)), err.shape)
        raise AssertionError("%s: %d of %d outputs outside their accumulation bound; worst at %s: got %r, oracle "
                             "%r, bound %r" % (what, int(bad.sum()), bad.size, i, got[i], ref[i], bound[i]))


def _bf16_round(v: np.ndarray) -> np.ndarray:
    """Round to nearest even bf16 (through fp32, both roundings monotone)."""
    return torch.from_numpy(np.asarray(v, np.float64)).float().to(torch.bfloat16).float().numpy().astype(np.float64)


def assert_bf16_bracket(y_bf16, y_ref, bound, what=""):
    """bf16 outputs against the oracle: each must be RN_bf16 of some value
    within its accumulation bound of the exact result, i.e. lie in
    [RN_bf16(y - B), RN_bf16(y + B)] (rounding is monotone). With B below
    half a bf16 ulp this is RN_bf16(y) itself, or its neighbour when y sits
    within B of a rounding midpoint."""
    got = y_bf16.detach().float().cpu().numpy().astype(np.float64) if isinstance(y_bf16, torch.Tensor) \
        else np.asarray(y_bf16, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    lo, hi = _bf16_round(y_ref - bound), _bf16_round(y_ref + bound)
    bad = (got < lo) | (got > hi)
    if bad.any():
        i = np.unravel_index(int(np.argmax(bad)), bad.shape)
        raise AssertionError("%s: %d of %d bf16 outputs outside [RN(y - B), RN(y + B)]; first at %s: got %r, oracle "
                             "%r, bound %r" % (what, int(bad.sum()), bad.size, i, got[i], y_ref[i], bound[i]))
    exact = (got == _bf16_round(y_ref))
    log("%s: %d of %d bf16 outputs equal RN_bf16(oracle), the rest its neighbour within the bound"
        % (what, int(exact.sum()), exact.size))


def tile_sample(n: int, tile: int, rng, extra=()) -> np.ndarray:
    """One random index in every tile of `tile` consecutive indices of [0, n)
    (the last, possibly ragged, tile included), plus its last index and any
    extra ones."""
    picks = [int(rng.integers(t, min(t + tile, n))) for t in range(0, n, tile)]
    return np.unique(np.array(picks + [n - 1] + list(extra), np.int64))


# ---------------------------------------------------------------------------
# The GEMM layout of packed operands, restated from include/macaq.h: rows
# padded to a multiple of 32, K to a multiple of 256, padding all zero; blocks
# of 32 rows x 256 elements ordered (row group, k block); inside a block, chunk
# c = 2h + j (32 elements) of row r has its 16 code bytes at
# h*1024 + (32j + r)*16 and its scale at (32j + r)*4 + h.
# ---------------------------------------------------------------------------

def padded(rows: int, K: int):
    return -(-rows // 32) * 32, -(-K // 256) * 256


def gemm_layout_to_row_major(codes, scales, rows: int, K: int, check_padding: bool = True):
    """Row-major (codes [rows, K/2], scales [rows, K/32]) of a GEMM-layout operand."""
    RP, KP = padded(rows, K)
    KB = KP // 256
    c = np.asarray(codes).reshape(-1)
    s = np.asarray(scales).reshape(-1)
    assert c.size == RP * KP // 2 and s.size == RP * KP // 32, (c.size, s.size, RP, KP)
    # codes: (g, kb, h, j, r, b) -> (g, r, kb, h, j, b); scales: (g, kb, j, r, h) -> (g, r, kb, h, j)
    cf = c.reshape(RP // 32, KB, 4, 2, 32, 16).transpose(0, 4, 1, 2, 3, 5).reshape(RP, KP // 2)
    sf = s.reshape(RP // 32, KB, 2, 32, 4).transpose(0, 3, 1, 4, 2).reshape(RP, KP // 32)
    if check_padding:
        assert not cf[rows:].any() and not cf[:, K // 2:].any(), "code padding is not zero"
        assert not sf[rows:].any() and not sf[:, K // 32:].any(), "scale padding is not zero"
    return np.ascontiguousarray(cf[:rows, :K // 2]), np.ascontiguousarray(sf[:rows, :K // 32])


def row_major_to_gemm_layout(codes, scales):
    """Inverse of gemm_layout_to_row_major (numpy, zero padding)."""
    codes = np.asarray(codes, np.uint8)
    scales = np.asarray(scales, np.uint8)
    rows, K = codes.shape[0], codes.shape[1] * 2
    RP, KP = padded(rows, K)
    KB = KP // 256
    cf = np.zeros((RP, KP // 2), np.uint8)
    sf = np.zeros((RP, KP // 32), np.uint8)
    cf[:rows, :K // 2] = codes
    sf[:rows, :K // 32] = scales
    c = cf.reshape(RP // 32, 32, KB, 4, 2, 16).transpose(0, 2, 3, 4, 1, 5).reshape(-1)
    s = sf.reshape(RP // 32, 32, KB, 4, 2).transpose(0, 2, 4, 1, 3).reshape(-1)
    return np.ascontiguousarray(c), np.ascontiguousarray(s)


def packed_to_row_major(p, check_padding: bool = True):
    """(codes, scales) row-major numpy arrays of a binding.Packed operand."""
    return gemm_layout_to_row_major(p.codes.cpu().numpy(), p.scales.cpu().numpy(), p.rows, p.K, check_padding)
