"""CPU oracle for the MACaQ online W4A4 linear layer.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` are the only callers. The product package
never imports this module, and this module never imports the product package.

This file only marshals numpy arrays into the plain C implementation in
``macaq_oracle.c`` (built with gcc, ``-ffp-contract=off``); every step of the
arithmetic lives there, with its sources:

* "MACaQ: Fast, Model Agnostic Calibrated Quantization for Low-Precision
  Weights and Activations" (paper card, Abstract) -- per-channel scale and
  block-Hadamard online on the activations, inverse absorbed into the same
  layer's weights, MXFP4 W4A4, round-to-nearest weights.
* OCP Microscaling Formats v1.0 -- E2M1 elements, one E8M0 scale per 32.

* The MoE block (routing, gathered gate/up, SiLU * up, the down projection's
  own transform and MXFP4, down, weighted combine): "MACaQ - Huawei
  open-sources a 4-bit quantizer ..." (What it is) covers MoE models;
  "Huawei's MACaQ-R beats Unsloth's ..." ("Changed tensors") names the
  experts' gate, up and down projections. The gated FFN form is a reading.

* Flip-Refinement (Hessian of the transformed calibration rows, greedy
  single-code moves with the block scales kept): "MACaQ ..." (paper card,
  Abstract); "Huawei's MACaQ-R beats Unsloth's ..." (Why that's still
  interesting; What we found when we compared the files). Objective, move
  order and stopping rule are readings.

Parity status per function (what pins it, see ``tests/test_oracle_pins.py``,
``tests/test_oracle_moe_pins.py``, ``tests/test_oracle_refine_pins.py``):
calibrate, multipliers, transform_rows, quant_rows, dequant_rows, gemm_codes,
linear, linear_grouped, moe_route, silu_mul, moe_combine, moe_block, hessian
and flip_refine are all pinned by closed forms, hand-worked values,
independent restatements and brute force; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "macaq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmacaq_oracle.so")
_lib = None

_u8p = ctypes.POINTER(ctypes.c_uint8)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64 = ctypes.c_int64
_int = ctypes.c_int


def build() -> str:
    """Compile the oracle with gcc (IEEE fp32, no contraction into FMA)."""
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread",
           "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    vp = ctypes.c_void_p
    lib.oracle_calibrate.argtypes = [vp, _int, _i64, _i64, _i64, _f32p]
    lib.oracle_multipliers.argtypes = [_f32p, _i64, _int, _f32p, _f32p]
    lib.oracle_transform_rows.argtypes = [vp, _int, _i64, _i64, _i64, _f32p, _int, _f32p]
    lib.oracle_quant_rows.argtypes = [vp, _int, _i64, _i64, _i64, _f32p, _int, _u8p, _u8p]
    lib.oracle_dequant_rows.argtypes = [_u8p, _u8p, _i64, _i64, _f64p]
    lib.oracle_gemm_codes.argtypes = [_u8p, _u8p, _i64, _u8p, _u8p, _i64, _i64, _f64p, _int]
    lib.oracle_linear.argtypes = [vp, _i64, _i64, _i64, _f32p, _int, _u8p, _u8p, _i64, _f64p, _int]
    lib.oracle_linear_grouped.argtypes = [vp, _i32p, _int, _i64, _i64, _f32p, _int, _u8p, _u8p, _i64,
                                          _f64p, _int]
    lib.oracle_moe_route.argtypes = [_i32p, _i64, _int, _int, _i32p, _i32p, _i32p]
    lib.oracle_silu_mul.argtypes = [_f64p, _i64, _i64, _f32p]
    lib.oracle_moe_combine.argtypes = [_f32p, _i64, _i32p, _f32p, _i64, _int, _f64p]
    lib.oracle_moe_block.argtypes = [vp, _i64, _i64, _i32p, _f32p, _int, _int, _f32p, _u8p, _u8p, _f32p, _u8p,
                                     _u8p, _i64, _int, _u8p, _u8p, _u8p, _f64p, _int]
    lib.oracle_hessian.argtypes = [vp, _i64, _i64, _i64, _f32p, _int, _f64p]
    lib.oracle_calibrate_pow.argtypes = [vp, _int, _i64, _i64, _i64, _int, _f32p]
    lib.oracle_calibrate_pow.restype = _int
    lib.oracle_flip_refine.argtypes = [vp, _int, _i64, _i64, _i64, _f32p, _int, _f64p, _int, _u8p, _u8p, _i32p]
    for f in (lib.oracle_calibrate, lib.oracle_multipliers, lib.oracle_transform_rows, lib.oracle_quant_rows,
              lib.oracle_dequant_rows, lib.oracle_gemm_codes, lib.oracle_linear, lib.oracle_linear_grouped,
              lib.oracle_moe_route, lib.oracle_silu_mul, lib.oracle_moe_combine, lib.oracle_moe_block,
              lib.oracle_hessian, lib.oracle_flip_refine):
        f.restype = _int
    _lib = lib
    return lib


def _ptr(a: np.ndarray, t):
    return a.ctypes.data_as(t)


def _opt_f32(a):
    if a is None:
        return None, _f32p()
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a, _ptr(a, _f32p)


def _elems(x: np.ndarray):
    """(contiguous array, dtype id): uint16 holds bf16 bits (0), float32 is 1."""
    if x.dtype == np.uint16:
        return np.ascontiguousarray(x), 0
    if x.dtype == np.float32:
        return np.ascontiguousarray(x), 1
    raise TypeError("oracle inputs are bf16 bits (uint16) or float32, got %s" % x.dtype)


def _check(rc: int, name: str):
    if rc != 0:
        raise ValueError("%s rejected its arguments (code %d)" % (name, rc))


def default_threads() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def calibrate(xcal: np.ndarray) -> np.ndarray:
    """s[k] = sqrt(max_r |xcal[r, k]|) as fp32 (1 for an all-zero channel)."""
    lib = _load()
    x, dt = _elems(xcal)
    R, K = x.shape
    s = np.empty(K, np.float32)
    _check(lib.oracle_calibrate(x.ctypes.data, dt, R, K, K, _ptr(s, _f32p)), "calibrate")
    return s


def calibrate_pow(xcal: np.ndarray, quarters: int) -> np.ndarray:
    """s[k] = (max_r |xcal[r, k]|)^(quarters / 4), quarters in {0, 1, 2, 4}."""
    lib = _load()
    x, dt = _elems(xcal)
    R, K = x.shape
    s = np.empty(K, np.float32)
    _check(lib.oracle_calibrate_pow(x.ctypes.data, dt, R, K, K, quarters, _ptr(s, _f32p)), "calibrate_pow")
    return s


def multipliers(s: np.ndarray, b: int):
    """(a, r): activation multiplier c_b / s and weight multiplier c_b * s."""
    lib = _load()
    s = np.ascontiguousarray(s, dtype=np.float32)
    K = s.shape[0]
    a = np.empty(K, np.float32)
    r = np.empty(K, np.float32)
    _check(lib.oracle_multipliers(_ptr(s, _f32p), K, b, _ptr(a, _f32p), _ptr(r, _f32p)), "multipliers")
    return a, r


def transform_rows(x: np.ndarray, m, b: int) -> np.ndarray:
    """fp32 rows of S_b (m * x) (no multiply when m is None, no Hadamard when b == 0)."""
    lib = _load()
    x, dt = _elems(x)
    M, K = x.shape
    m_keep, mp = _opt_f32(m)
    t = np.empty((M, K), np.float32)
    _check(lib.oracle_transform_rows(x.ctypes.data, dt, M, K, K, mp, b, _ptr(t, _f32p)), "transform_rows")
    return t


def quant_rows(x: np.ndarray, m, b: int):
    """(codes uint8 [M, K/2], scales uint8 [M, K/32]) of MXFP4(S_b (m * x))."""
    lib = _load()
    x, dt = _elems(x)
    M, K = x.shape
    m_keep, mp = _opt_f32(m)
    codes = np.empty((M, K // 2), np.uint8)
    scales = np.empty((M, K // 32), np.uint8)
    _check(lib.oracle_quant_rows(x.ctypes.data, dt, M, K, K, mp, b, _ptr(codes, _u8p), _ptr(scales, _u8p)),
           "quant_rows")
    return codes, scales


def prepare_weights(w: np.ndarray, r, b: int):
    """W' = MXFP4(W D^-1 H^T) row by row: the same row quantizer with r."""
    return quant_rows(w, r, b)


def dequant_rows(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    lib = _load()
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    M, K2 = codes.shape
    out = np.empty((M, 2 * K2), np.float64)
    _check(lib.oracle_dequant_rows(_ptr(codes, _u8p), _ptr(scales, _u8p), M, 2 * K2, _ptr(out, _f64p)),
           "dequant_rows")
    return out


def gemm_codes(a_codes, a_scales, w_codes, w_scales, threads: int | None = None) -> np.ndarray:
    """fp64 y[m, n] = sum_k dq(A[m, k]) dq(W'[n, k])."""
    lib = _load()
    ac = np.ascontiguousarray(a_codes, np.uint8)
    as_ = np.ascontiguousarray(a_scales, np.uint8)
    wc = np.ascontiguousarray(w_codes, np.uint8)
    ws = np.ascontiguousarray(w_scales, np.uint8)
    M, N, K = ac.shape[0], wc.shape[0], 2 * ac.shape[1]
    y = np.empty((M, N), np.float64)
    _check(lib.oracle_gemm_codes(_ptr(ac, _u8p), _ptr(as_, _u8p), M, _ptr(wc, _u8p), _ptr(ws, _u8p), N, K,
                                 _ptr(y, _f64p), threads or default_threads()), "gemm_codes")
    return y


def linear(x: np.ndarray, a, b: int, w_codes, w_scales, threads: int | None = None) -> np.ndarray:
    """fp64 y = W' Q(H D x) for bf16 rows x (uint16 bits)."""
    lib = _load()
    x = np.ascontiguousarray(x, np.uint16)
    M, K = x.shape
    a_keep, ap = _opt_f32(a)
    wc = np.ascontiguousarray(w_codes, np.uint8)
    ws = np.ascontiguousarray(w_scales, np.uint8)
    N = wc.shape[0]
    y = np.empty((M, N), np.float64)
    _check(lib.oracle_linear(x.ctypes.data, M, K, K, ap, b, _ptr(wc, _u8p), _ptr(ws, _u8p), N, _ptr(y, _f64p),
                             threads or default_threads()), "linear")
    return y


def linear_grouped(x: np.ndarray, offsets: np.ndarray, a, b: int, w_codes, w_scales,
                   threads: int | None = None) -> np.ndarray:
    """Per expert e, rows [off[e], off[e+1]) of x through a[e] and W'_e."""
    lib = _load()
    x = np.ascontiguousarray(x, np.uint16)
    T, K = x.shape
    off = np.ascontiguousarray(offsets, np.int32)
    E = off.shape[0] - 1
    a_keep, ap = _opt_f32(a)
    wc = np.ascontiguousarray(w_codes, np.uint8)
    ws = np.ascontiguousarray(w_scales, np.uint8)
    N = wc.shape[1]
    y = np.zeros((T, N), np.float64)
    _check(lib.oracle_linear_grouped(x.ctypes.data, _ptr(off, _i32p), E, T, K, ap, b, _ptr(wc, _u8p),
                                     _ptr(ws, _u8p), N, _ptr(y, _f64p), threads or default_threads()),
           "linear_grouped")
    return y


def moe_route(ids: np.ndarray, E: int):
    """(offsets [E+1], row_token [T*k], pos [T*k]) of the stable sort of the
    (token, slot) entries by expert; ids [T, k] int32."""
    lib = _load()
    ids = np.ascontiguousarray(ids, np.int32)
    T, k = ids.shape
    off = np.empty(E + 1, np.int32)
    row_token = np.full(T * k, -1, np.int32)
    pos = np.empty(T * k, np.int32)
    _check(lib.oracle_moe_route(_ptr(ids, _i32p), T, k, E, _ptr(off, _i32p), _ptr(row_token, _i32p),
                                _ptr(pos, _i32p)), "moe_route")
    return off, row_token, pos


def silu_mul(gu: np.ndarray) -> np.ndarray:
    """h [R, F] fp32 = SiLU(gate) * up from stacked gate/up outputs [R, 2F]
    (blocks of 32 gate columns, then the matching 32 up columns)."""
    lib = _load()
    gu = np.ascontiguousarray(gu, np.float64)
    R, F2 = gu.shape
    h = np.empty((R, F2 // 2), np.float32)
    _check(lib.oracle_silu_mul(_ptr(gu, _f64p), R, F2 // 2, _ptr(h, _f32p)), "silu_mul")
    return h


def moe_combine(rows: np.ndarray, pos: np.ndarray, w: np.ndarray) -> np.ndarray:
    """y [T, H] fp64 = sum_j w[t, j] * rows[pos[t, j]] (pos < 0 skipped)."""
    lib = _load()
    rows = np.ascontiguousarray(rows, np.float32)
    pos = np.ascontiguousarray(pos, np.int32)
    w = np.ascontiguousarray(w, np.float32)
    T, k = w.shape
    H = rows.shape[1]
    y = np.empty((T, H), np.float64)
    _check(lib.oracle_moe_combine(_ptr(rows, _f32p), H, _ptr(pos, _i32p), _ptr(w, _f32p), T, k, _ptr(y, _f64p)),
           "moe_combine")
    return y


def moe_block(x: np.ndarray, ids: np.ndarray, w: np.ndarray, E: int, a_gu, wgu_codes, wgu_scales, a_dn,
              wdn_codes, wdn_scales, b: int, want: np.ndarray | None = None, threads: int | None = None):
    """(y [T, H] fp64, dn_codes [T*k, F/2], dn_scales [T*k, F/32]) of the MoE
    block for bf16 tokens x [T, H] (uint16 bits), top-k ids and weights
    [T, k]; stacked gate/up weights [E, 2F, H/2] + [E, 2F, H/32], down
    weights [E, H, F/2] + [E, H, F/32]. `want` (bool [T]) restricts the work
    to some tokens; the other rows of y and of the down inputs stay zero."""
    lib = _load()
    x = np.ascontiguousarray(x, np.uint16)
    T, H = x.shape
    ids = np.ascontiguousarray(ids, np.int32)
    w = np.ascontiguousarray(w, np.float32)
    k = ids.shape[1]
    gc = np.ascontiguousarray(wgu_codes, np.uint8)
    gs = np.ascontiguousarray(wgu_scales, np.uint8)
    dc = np.ascontiguousarray(wdn_codes, np.uint8)
    ds = np.ascontiguousarray(wdn_scales, np.uint8)
    F = 2 * dc.shape[2]
    agu_keep, agp = _opt_f32(a_gu)
    adn_keep, adp = _opt_f32(a_dn)
    if want is None:
        wp = _u8p()
    else:
        want = np.ascontiguousarray(want, np.uint8)
        wp = _ptr(want, _u8p)
    y = np.zeros((T, H), np.float64)
    hc = np.zeros((T * k, F // 2), np.uint8)
    hs = np.zeros((T * k, F // 32), np.uint8)
    _check(lib.oracle_moe_block(x.ctypes.data, T, H, _ptr(ids, _i32p), _ptr(w, _f32p), k, E, agp, _ptr(gc, _u8p),
                                _ptr(gs, _u8p), adp, _ptr(dc, _u8p), _ptr(ds, _u8p), F, b, wp, _ptr(hc, _u8p),
                                _ptr(hs, _u8p), _ptr(y, _f64p), threads or default_threads()), "moe_block")
    return y, hc, hs


def hessian(xcal: np.ndarray, a, b: int) -> np.ndarray:
    """H [K, K] (fp64) = X~^T X~ of bf16 calibration rows (uint16 bits)
    through multiplier a and the block-Hadamard of size b."""
    lib = _load()
    x = np.ascontiguousarray(xcal, np.uint16)
    R, K = x.shape
    a_keep, ap = _opt_f32(a)
    H = np.empty((K, K), np.float64)
    _check(lib.oracle_hessian(x.ctypes.data, R, K, K, ap, b, _ptr(H, _f64p)), "hessian")
    return H


def flip_refine(w: np.ndarray, r, b: int, H: np.ndarray, max_flips: int, codes: np.ndarray, scales: np.ndarray):
    """(refined codes [N, K/2], flips per row) of prepared weights (row-major
    codes and scales, scales kept) for weight rows w (bf16 bits or fp32)."""
    lib = _load()
    w, dt = _elems(w)
    N, K = w.shape
    r_keep, rp = _opt_f32(r)
    H = np.ascontiguousarray(H, np.float64)
    out = np.array(codes, np.uint8, copy=True, order="C")
    sc = np.ascontiguousarray(scales, np.uint8)
    flips = np.zeros(N, np.int32)
    _check(lib.oracle_flip_refine(w.ctypes.data, dt, N, K, K, rp, b, _ptr(H, _f64p), max_flips, _ptr(out, _u8p),
                                  _ptr(sc, _u8p), _ptr(flips, _i32p)), "flip_refine")
    return out, flips
