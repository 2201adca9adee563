"""ctypes binding of ``libmacaq.so`` (C ABI in ``include/macaq.h``).

Argument marshalling only: torch supplies device memory and the current
stream; every step of the computation runs in the library's HIP kernels.
There is no fallback: if the library is missing or the device is not gfx950
the calls raise.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import NamedTuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libmacaq.so")
_lib = None
_lock = threading.Lock()

MACAQ_BF16 = 0
MACAQ_F32 = 1
MACAQ_ROW_MAJOR = 0
MACAQ_GEMM_LAYOUT = 1
_STATUS_NAMES = {0: "MACAQ_OK", 1: "MACAQ_EINVAL", 2: "MACAQ_EALIGN", 3: "MACAQ_EWORKSPACE",
                 4: "MACAQ_EUNSUPPORTED", 5: "MACAQ_EHIP"}

# name -> (restype, argtypes), in the order of include/macaq.h
_vp, _i64, _i32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
_SIGNATURES = {
    "macaq_packed_codes_bytes": (_sz, [_i64, _i64]),
    "macaq_packed_scales_bytes": (_sz, [_i64, _i64]),
    "macaq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "macaq_last_error": (ctypes.c_char_p, []),
    "macaq_calibrate": (ctypes.c_int, [_vp, _i64, _i64, _i64, _vp, _vp]),
    "macaq_calibrate_pow": (ctypes.c_int, [_vp, _i64, _i64, _i64, _i32, _vp, _vp]),
    "macaq_debug_override_arch": (None, [ctypes.c_char_p]),
    "macaq_debug_limit_workgroups": (None, [_i32]),
    "macaq_debug_mfma_probe": (ctypes.c_int, [_vp, _i32, _i32, _vp, _vp]),
    "macaq_debug_read_probe": (ctypes.c_int, [_vp, _i64, _i32, _vp, _vp]),
    "macaq_make_multipliers": (ctypes.c_int, [_vp, _i64, _i32, _vp, _vp]),
    "macaq_make_multipliers_device": (ctypes.c_int, [_vp, _i64, _i32, _vp, _vp, _vp]),
    "macaq_prepare_weights": (ctypes.c_int, [_vp, ctypes.c_int, _i64, _i64, _i64, _vp, _i32, ctypes.c_int, _vp, _vp,
                                             _vp]),
    "macaq_quant_act": (ctypes.c_int, [_vp, _i64, _i64, _i64, _vp, _i32, ctypes.c_int, _vp, _vp, _vp]),
    "macaq_linear_workspace_size": (_sz, [_i64, _i64, _i64]),
    "macaq_linear": (ctypes.c_int, [_vp, _i64, _i64, _i64, _vp, _i32, _vp, _vp, _i64, _vp, ctypes.c_int, _i64,
                                    _vp, _sz, _vp]),
    "macaq_linear_noalloc": (ctypes.c_int, [_vp, _i64, _i64, _i64, _vp, _i32, _vp, _vp, _i64, _vp, ctypes.c_int,
                                            _i64, _vp]),
    "macaq_gemm_workspace_size": (_sz, [_i64, _i64, _i64]),
    "macaq_gemm": (ctypes.c_int, [_vp, _vp, _i64, _i64, _vp, _vp, _i64, _vp, ctypes.c_int, _i64, _vp, _sz, _vp]),
    "macaq_linear_grouped_workspace_size": (_sz, [_i64, _i32, _i64, _i64]),
    "macaq_linear_grouped": (ctypes.c_int, [_vp, _vp, _i32, _i64, _i64, _vp, _i32, _vp, _vp, _i64, _vp,
                                            ctypes.c_int, _vp, _sz, _vp]),
    "macaq_moe_workspace_size": (_sz, [_i64, _i32, _i32, _i64, _i64]),
    "macaq_moe_route_workspace_size": (_sz, [_i64, _i32, _i32]),
    "macaq_moe_route": (ctypes.c_int, [_vp, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp]),
    "macaq_moe_gate_up": (ctypes.c_int, [_vp, _i64, _i64, _i64, _i32, _vp, _vp, _i32, _vp, _i32, _vp, _vp, _i64,
                                         _vp, _vp, _vp, _vp, _sz, _vp]),
    "macaq_moe_down_combine": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i32, _i32, _vp, _vp, _i64, _i64, _vp,
                                              ctypes.c_int, _i64, _vp, _sz, _vp]),
    "macaq_moe_block": (ctypes.c_int, [_vp, _i64, _i64, _i64, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                       _i64, _i32, _vp, ctypes.c_int, _i64, _vp, _sz, _vp]),
    "macaq_hessian_workspace_size": (_sz, [_i64, _i64]),
    "macaq_hessian": (ctypes.c_int, [_vp, _i64, _i64, _i64, _vp, _i32, _vp, _vp, _sz, _vp]),
    "macaq_flip_refine_workspace_size": (_sz, [_i64, _i64]),
    "macaq_flip_refine": (ctypes.c_int, [_vp, ctypes.c_int, _i64, _i64, _i64, _vp, _i32, _vp, _i32, _vp, _vp, _vp,
                                         _vp, _sz, _vp]),
}


class Packed(NamedTuple):
    """An MXFP4 operand in the GEMM layout: `rows` x `K` elements (padded to 32
    rows and a multiple of 256 in K inside the buffers). codes / scales are
    uint8 tensors of packed_codes_bytes / packed_scales_bytes bytes (with a
    leading expert dimension for grouped weights)."""
    codes: torch.Tensor
    scales: torch.Tensor
    rows: int
    K: int


class MacaqError(RuntimeError):
    def __init__(self, func: str, status: int, detail: str):
        self.status = status
        super().__init__("%s failed: %s (%s): %s" % (func, _STATUS_NAMES.get(status, status),
                                                    _status_string(status), detail))


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libmacaq.so. It is (re)built first when it is missing or was built
    from other sources than those in csrc/ and include/ now (the digest that
    build.py records beside it), so the library that runs is always the one
    the sources describe."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        from . import build as _build
        alt = os.environ.get("MACAQ_LIBRARY")
        if alt:
            # another build of the same sources (the sanitized host build of
            # the CPU tests); loaded as it is
            lib = ctypes.CDLL(alt)
            for name, (res, args) in _SIGNATURES.items():
                f = getattr(lib, name)
                f.restype = res
                f.argtypes = args
            _lib = lib
            return lib
        if not _build.is_current():
            print("macaq: libmacaq.so is missing or older than its sources; building it", flush=True)
            _build.build()
            if not _build.is_current():
                raise RuntimeError("macaq: the built library does not match its sources")
        lib = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            f = getattr(lib, name)
            f.restype = res
            f.argtypes = args
        _lib = lib
        return lib


def override_arch(arch: str | None):
    """Make the library's device check see `arch` instead of the device
    (None restores the real query): the test hook of macaq.h."""
    load_library().macaq_debug_override_arch(None if arch is None else arch.encode())


def limit_workgroups(n: int):
    """Cap every persistent GEMM launch at n workgroups (n <= 0: the planned
    grid): the stress hook of macaq.h, for tests; results must not change."""
    load_library().macaq_debug_limit_workgroups(int(n))


MFMA_PROBE_OPERAND_BYTES = 24576


def mfma_probe(operands: torch.Tensor, workgroups: int, iters: int, out: torch.Tensor) -> torch.Tensor:
    """Back-to-back scaled-FP4 MFMAs on register operands (the measurement
    probe of macaq.h); operands: device uint8 of at least 24576 bytes, out:
    device fp32 of workgroups * 256."""
    _need_cuda(operands, out)
    assert operands.numel() * operands.element_size() >= MFMA_PROBE_OPERAND_BYTES
    assert out.dtype == torch.float32 and out.numel() >= workgroups * 256
    _check(load_library().macaq_debug_mfma_probe(_ptr(operands), workgroups, iters, _ptr(out), _stream(out)),
           "macaq_debug_mfma_probe")
    return out


def read_probe(src: torch.Tensor, workgroups: int, out: torch.Tensor) -> torch.Tensor:
    """A plain read of src (device, contiguous) by the measurement probe of
    macaq.h; out: device int32 of workgroups * 256."""
    _need_cuda(src, out)
    assert src.is_contiguous() and out.dtype == torch.int32 and out.numel() >= workgroups * 256
    _check(load_library().macaq_debug_read_probe(_ptr(src), src.numel() * src.element_size(), workgroups, _ptr(out),
                                                 _stream(src)), "macaq_debug_read_probe")
    return out


def _status_string(status: int) -> str:
    lib = load_library()
    return lib.macaq_status_string(status).decode()


def _check(status: int, func: str):
    if status != 0:
        lib = load_library()
        raise MacaqError(func, status, lib.macaq_last_error().decode())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("macaq: tensors must be on the GPU")


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return MACAQ_BF16
    if dt == torch.float32:
        return MACAQ_F32
    raise ValueError("macaq: dtype %s is not bf16 or fp32" % dt)


def calibrate(xcal: torch.Tensor, quarters: int = 2) -> torch.Tensor:
    """Per-channel scale s[k] = (max_r |xcal[r, k]|)^(quarters / 4) of bf16
    calibration rows (quarters 2, the default: the square root)."""
    _need_cuda(xcal)
    assert xcal.dtype == torch.bfloat16 and xcal.dim() == 2 and xcal.stride(1) == 1
    R, K = xcal.shape
    s = torch.empty(K, dtype=torch.float32, device=xcal.device)
    if quarters == 2:
        _check(load_library().macaq_calibrate(_ptr(xcal), R, K, xcal.stride(0), _ptr(s), _stream(xcal)),
               "macaq_calibrate")
    else:
        _check(load_library().macaq_calibrate_pow(_ptr(xcal), R, K, xcal.stride(0), quarters, _ptr(s),
                                                  _stream(xcal)), "macaq_calibrate_pow")
    return s


def make_multipliers(s: torch.Tensor, b: int):
    """(a, r): activation multiplier c_b / s and weight multiplier c_b * s of
    a device scale s (macaq_make_multipliers_device, on s's stream)."""
    _need_cuda(s)
    s = s.contiguous()
    a = torch.empty_like(s)
    r = torch.empty_like(s)
    _check(load_library().macaq_make_multipliers_device(_ptr(s), s.numel(), b, _ptr(a), _ptr(r), _stream(s)),
           "macaq_make_multipliers_device")
    return a, r


def make_multipliers_host(s, b: int):
    """(a, r) of a host scale s (numpy fp32 or a CPU tensor) through the
    library's host-only macaq_make_multipliers; returns numpy fp32 arrays."""
    import numpy as np
    if isinstance(s, torch.Tensor):
        if s.is_cuda:
            raise ValueError("macaq: make_multipliers_host takes a host scale")
        s = s.numpy()
    s = np.ascontiguousarray(s, dtype=np.float32)
    a = np.empty_like(s)
    r = np.empty_like(s)
    _check(load_library().macaq_make_multipliers(s.ctypes.data, s.size, b, a.ctypes.data, r.ctypes.data),
           "macaq_make_multipliers")
    return a, r


def packed_codes_bytes(rows: int, K: int) -> int:
    return int(load_library().macaq_packed_codes_bytes(rows, K))


def packed_scales_bytes(rows: int, K: int) -> int:
    return int(load_library().macaq_packed_scales_bytes(rows, K))


def prepare_weights(w: torch.Tensor, r: torch.Tensor | None, b: int, out: Packed | None = None,
                    layout: str = "gemm"):
    """W' = MXFP4(W D^-1 H^T). layout "gemm" (default): a Packed operand in
    the GEMM layout; layout "row": (codes [N, K/2], scales [N, K/32])."""
    _need_cuda(w, r)
    assert w.dim() == 2 and w.stride(1) == 1
    N, K = w.shape
    if layout == "row":
        codes = torch.empty(N, K // 2, dtype=torch.uint8, device=w.device)
        scales = torch.empty(N, K // 32, dtype=torch.uint8, device=w.device)
        _check(load_library().macaq_prepare_weights(_ptr(w), _dtype_code(w.dtype), N, K, w.stride(0), _ptr(r), b,
                                                    MACAQ_ROW_MAJOR, _ptr(codes), _ptr(scales), _stream(w)),
               "macaq_prepare_weights")
        return codes, scales
    if layout != "gemm":
        raise ValueError("layout is 'row' or 'gemm'")
    if out is None:
        out = Packed(torch.empty(packed_codes_bytes(N, K), dtype=torch.uint8, device=w.device),
                     torch.empty(packed_scales_bytes(N, K), dtype=torch.uint8, device=w.device), N, K)
    _check(load_library().macaq_prepare_weights(_ptr(w), _dtype_code(w.dtype), N, K, w.stride(0), _ptr(r), b,
                                                MACAQ_GEMM_LAYOUT, _ptr(out.codes), _ptr(out.scales), _stream(w)),
           "macaq_prepare_weights")
    return out


def quant_act(x: torch.Tensor, a: torch.Tensor | None, b: int, layout: str = "row", codes: torch.Tensor | None = None,
              scales: torch.Tensor | None = None):
    """MXFP4(H D x) of bf16 rows. layout "row": (codes [M, K/2], scales [M, K/32]);
    layout "gemm": a Packed operand in the GEMM layout."""
    _need_cuda(x, a, codes, scales)
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1
    M, K = x.shape
    gemm = layout == "gemm"
    if not gemm and layout != "row":
        raise ValueError("layout is 'row' or 'gemm'")
    if codes is None:
        codes = (torch.empty(packed_codes_bytes(M, K), dtype=torch.uint8, device=x.device) if gemm
                 else torch.empty(M, K // 2, dtype=torch.uint8, device=x.device))
    if scales is None:
        scales = (torch.empty(packed_scales_bytes(M, K), dtype=torch.uint8, device=x.device) if gemm
                  else torch.empty(M, K // 32, dtype=torch.uint8, device=x.device))
    _check(load_library().macaq_quant_act(_ptr(x), M, K, x.stride(0), _ptr(a), b,
                                          MACAQ_GEMM_LAYOUT if gemm else MACAQ_ROW_MAJOR, _ptr(codes), _ptr(scales),
                                          _stream(x)), "macaq_quant_act")
    return Packed(codes, scales, M, K) if gemm else (codes, scales)


def linear_workspace_size(M: int, K: int, N: int) -> int:
    return int(load_library().macaq_linear_workspace_size(M, K, N))


def gemm_workspace_size(M: int, K: int, N: int) -> int:
    return int(load_library().macaq_gemm_workspace_size(M, K, N))


def linear_grouped_workspace_size(T: int, E: int, K: int, N: int) -> int:
    return int(load_library().macaq_linear_grouped_workspace_size(T, E, K, N))


def _workspace(nbytes: int, device, given: torch.Tensor | None):
    if given is not None:
        return given
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def linear(x: torch.Tensor, a: torch.Tensor | None, b: int, w: Packed, out_dtype: torch.dtype = torch.bfloat16,
           out: torch.Tensor | None = None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """y = W' MXFP4(H D x) for bf16 rows x [M, K]; returns [M, N] of out_dtype."""
    _need_cuda(x, a, w.codes, w.scales)
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1
    M, K = x.shape
    assert K == w.K, "activation K %d does not match the weights' %d" % (K, w.K)
    N = w.rows
    y = out if out is not None else torch.empty(M, N, dtype=out_dtype, device=x.device)
    ws = _workspace(linear_workspace_size(M, K, N), x.device, workspace)
    _check(load_library().macaq_linear(_ptr(x), M, K, x.stride(0), _ptr(a), b, _ptr(w.codes), _ptr(w.scales), N,
                                       _ptr(y), _dtype_code(y.dtype), y.stride(0), _ptr(ws), ws.numel(), _stream(x)),
           "macaq_linear")
    return y


NOALLOC_SCRATCH_BYTES = 128 << 20


def linear_noalloc(x: torch.Tensor, a: torch.Tensor | None, b: int, w: Packed, out: torch.Tensor) -> torch.Tensor:
    """linear() through macaq_linear_noalloc: no workspace, the library's own
    scratch (128 MiB per GPU); out [M, N] (bf16 or fp32) must be given."""
    _need_cuda(x, a, w.codes, w.scales, out)
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1
    M, K = x.shape
    assert K == w.K, "activation K %d does not match the weights' %d" % (K, w.K)
    _check(load_library().macaq_linear_noalloc(_ptr(x), M, K, x.stride(0), _ptr(a), b, _ptr(w.codes), _ptr(w.scales),
                                               w.rows, _ptr(out), _dtype_code(out.dtype), out.stride(0), _stream(x)),
           "macaq_linear_noalloc")
    return out


def linear_plain_gemm(a: Packed, w: Packed, out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None,
                      workspace: torch.Tensor | None = None) -> torch.Tensor:
    """The GEMM alone on MXFP4 operands in the GEMM layout: y = dq(A) dq(W')^T."""
    _need_cuda(a.codes, a.scales, w.codes, w.scales)
    assert a.K == w.K
    M, K, N = a.rows, a.K, w.rows
    y = out if out is not None else torch.empty(M, N, dtype=out_dtype, device=a.codes.device)
    ws = _workspace(gemm_workspace_size(M, K, N), a.codes.device, workspace)
    _check(load_library().macaq_gemm(_ptr(a.codes), _ptr(a.scales), M, K, _ptr(w.codes), _ptr(w.scales), N, _ptr(y),
                                     _dtype_code(y.dtype), y.stride(0), _ptr(ws), ws.numel(),
                                     _stream(a.codes)), "macaq_gemm")
    return y


def linear_grouped(x: torch.Tensor, offsets: torch.Tensor, a: torch.Tensor | None, b: int, w: Packed,
                   out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None,
                   workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Per expert e: rows [off[e], off[e+1]) of x through a[e] and W'_e; w holds
    the E experts' prepared weights stacked along dimension 0."""
    _need_cuda(x, offsets, a, w.codes, w.scales)
    assert x.dtype == torch.bfloat16 and x.is_contiguous() and offsets.dtype == torch.int32
    T, K = x.shape
    E = offsets.numel() - 1
    N = w.rows
    assert w.codes.shape[0] == E and w.codes[0].numel() == packed_codes_bytes(N, K)
    y = out if out is not None else torch.empty(T, N, dtype=out_dtype, device=x.device)
    ws = _workspace(linear_grouped_workspace_size(T, E, K, N), x.device, workspace)
    _check(load_library().macaq_linear_grouped(_ptr(x), _ptr(offsets), E, T, K, _ptr(a), b, _ptr(w.codes),
                                               _ptr(w.scales), N, _ptr(y), _dtype_code(y.dtype), _ptr(ws),
                                               ws.numel(), _stream(x)), "macaq_linear_grouped")
    return y


def empty_grouped_weights(E: int, N: int, K: int, device) -> Packed:
    """Storage for E experts' prepared weights (fill with prepare_weights(out=expert(w, e)))."""
    return Packed(torch.empty(E, packed_codes_bytes(N, K), dtype=torch.uint8, device=device),
                  torch.empty(E, packed_scales_bytes(N, K), dtype=torch.uint8, device=device), N, K)


def expert(w: Packed, e: int) -> Packed:
    return Packed(w.codes[e], w.scales[e], w.rows, w.K)


class Layer:
    """A prepared layer: the activation multiplier a and W' codes/scales from
    the same calibration scale s and Hadamard block b."""

    def __init__(self, a, r, b, w: Packed, s=None):
        self.a, self.r, self.b, self.w, self.s = a, r, b, w, s

    def __call__(self, x, out_dtype=torch.bfloat16, out=None, workspace=None):
        return linear(x, self.a, self.b, self.w, out_dtype, out, workspace)


def prepare_layer(w: torch.Tensor, xcal: torch.Tensor | None, b: int) -> Layer:
    """Calibrate s on xcal, fold c_b into a and r, and prepare W'. With
    xcal None and b == 0 the layer is plain MXFP4 (no transform)."""
    if xcal is None:
        if b != 0:
            raise ValueError("a Hadamard block without a calibration scale is not a MACaQ layer")
        return Layer(None, None, 0, prepare_weights(w, None, 0))
    s = calibrate(xcal)
    a, r = make_multipliers(s, b)
    return Layer(a, r, b, prepare_weights(w, r, b), s)


# ---- MoE block around the grouped layer -----------------------------------

def stack_gate_up(w_gate: torch.Tensor, w_up: torch.Tensor) -> torch.Tensor:
    """[.., F, H] gate and up weights -> [.., 2F, H] with alternating blocks of
    32 rows (gate channels 32c .. 32c+31, then the matching up channels), the
    layout the MoE gate/up GEMM's epilogue expects."""
    assert w_gate.shape == w_up.shape and w_gate.shape[-2] % 32 == 0
    F, H = w_gate.shape[-2:]
    lead = w_gate.shape[:-2]
    g = w_gate.reshape(*lead, F // 32, 1, 32, H)
    u = w_up.reshape(*lead, F // 32, 1, 32, H)
    return torch.cat([g, u], dim=-3).reshape(*lead, 2 * F, H).contiguous()


def moe_workspace_size(T: int, k: int, E: int, H: int, F: int) -> int:
    return int(load_library().macaq_moe_workspace_size(T, k, E, H, F))


def moe_route_workspace_size(T: int, k: int, E: int) -> int:
    return int(load_library().macaq_moe_route_workspace_size(T, k, E))


def moe_route(ids: torch.Tensor, E: int, workspace: torch.Tensor | None = None):
    """(offsets [E+1], row_token [T*k], pos [T*k]) of the stable sort of the
    top-k entries ids [T, k] (int32) by expert."""
    _need_cuda(ids)
    assert ids.dtype == torch.int32 and ids.dim() == 2 and ids.is_contiguous()
    T, k = ids.shape
    dev = ids.device
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    row_token = torch.empty(max(T * k, 1), dtype=torch.int32, device=dev)
    pos = torch.empty(max(T * k, 1), dtype=torch.int32, device=dev)
    ws = _workspace(moe_route_workspace_size(T, k, E), dev, workspace)
    _check(load_library().macaq_moe_route(_ptr(ids), T, k, E, _ptr(offsets), _ptr(row_token), _ptr(pos), _ptr(ws),
                                          ws.numel(), _stream(ids)), "macaq_moe_route")
    return offsets, row_token[:T * k], pos[:T * k]


def moe_gate_up(x: torch.Tensor, k: int, row_token: torch.Tensor, offsets: torch.Tensor, a_gu, b: int, wgu: Packed,
                a_dn, out: Packed | None = None, workspace: torch.Tensor | None = None) -> Packed:
    """The down projection's MXFP4 input (GEMM layout, T*k rows x F) of every
    routed row: gathered gate/up through a_gu[e] and the stacked weights, then
    SiLU(gate) * up through a_dn[e] and the block-Hadamard."""
    _need_cuda(x, row_token, offsets, a_gu, a_dn, wgu.codes, wgu.scales)
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1
    T, H = x.shape
    E = offsets.numel() - 1
    F = wgu.rows // 2
    R = T * k
    if out is None:
        out = Packed(torch.empty(packed_codes_bytes(R, F), dtype=torch.uint8, device=x.device),
                     torch.empty(packed_scales_bytes(R, F), dtype=torch.uint8, device=x.device), R, F)
    ws = _workspace(moe_workspace_size(T, k, E, H, F), x.device, workspace)
    _check(load_library().macaq_moe_gate_up(_ptr(x), T, H, x.stride(0), k, _ptr(row_token), _ptr(offsets), E,
                                            _ptr(a_gu), b, _ptr(wgu.codes), _ptr(wgu.scales), F, _ptr(a_dn),
                                            _ptr(out.codes), _ptr(out.scales), _ptr(ws), ws.numel(), _stream(x)),
           "macaq_moe_gate_up")
    return out


def moe_down_combine(dn: Packed, offsets: torch.Tensor, pos: torch.Tensor, w: torch.Tensor, wdn: Packed,
                     out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None,
                     workspace: torch.Tensor | None = None) -> torch.Tensor:
    """y [T, H] = sum_j w[t, j] * bf16(down_e(row pos[t*k + j])) for routing
    weights w [T, k] (fp32)."""
    _need_cuda(dn.codes, offsets, pos, w, wdn.codes)
    assert w.dtype == torch.float32 and w.is_contiguous()
    T, k = w.shape
    E = offsets.numel() - 1
    H, F = wdn.rows, wdn.K
    y = out if out is not None else torch.empty(T, H, dtype=out_dtype, device=w.device)
    ws = _workspace(moe_workspace_size(T, k, E, H, F), w.device, workspace)
    _check(load_library().macaq_moe_down_combine(_ptr(dn.codes), _ptr(dn.scales), _ptr(offsets), _ptr(pos), _ptr(w),
                                                 T, k, E, _ptr(wdn.codes), _ptr(wdn.scales), H, F, _ptr(y),
                                                 _dtype_code(y.dtype), y.stride(0), _ptr(ws), ws.numel(),
                                                 _stream(w)), "macaq_moe_down_combine")
    return y


def moe_block(x: torch.Tensor, ids: torch.Tensor, w: torch.Tensor, a_gu, wgu: Packed, a_dn, wdn: Packed, b: int,
              out_dtype: torch.dtype = torch.bfloat16, out: torch.Tensor | None = None,
              workspace: torch.Tensor | None = None) -> torch.Tensor:
    """The whole MoE block for bf16 tokens x [T, H], top-k ids [T, k] (int32)
    and routing weights w [T, k] (fp32)."""
    _need_cuda(x, ids, w, a_gu, a_dn, wgu.codes, wdn.codes)
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1
    assert ids.dtype == torch.int32 and ids.is_contiguous() and w.dtype == torch.float32 and w.is_contiguous()
    T, H = x.shape
    k = ids.shape[1]
    E = wgu.codes.shape[0]
    F = wgu.rows // 2
    y = out if out is not None else torch.empty(T, H, dtype=out_dtype, device=x.device)
    ws = _workspace(moe_workspace_size(T, k, E, H, F), x.device, workspace)
    _check(load_library().macaq_moe_block(_ptr(x), T, H, x.stride(0), _ptr(ids), _ptr(w), k, E, _ptr(a_gu),
                                          _ptr(wgu.codes), _ptr(wgu.scales), _ptr(a_dn), _ptr(wdn.codes),
                                          _ptr(wdn.scales), F, b, _ptr(y), _dtype_code(y.dtype), y.stride(0),
                                          _ptr(ws), ws.numel(), _stream(x)), "macaq_moe_block")
    return y


class MoELayer:
    """A prepared MoE block: per-expert multipliers a_gu [E, H], a_dn [E, F] and
    the stacked gate/up and down weights of every expert."""

    def __init__(self, a_gu, wgu: Packed, a_dn, wdn: Packed, b: int):
        self.a_gu, self.wgu, self.a_dn, self.wdn, self.b = a_gu, wgu, a_dn, wdn, b

    def __call__(self, x, ids, w, out_dtype=torch.bfloat16, out=None, workspace=None):
        return moe_block(x, ids, w, self.a_gu, self.wgu, self.a_dn, self.wdn, self.b, out_dtype, out, workspace)


def prepare_moe(w_gate: torch.Tensor, w_up: torch.Tensor, w_dn: torch.Tensor, xcal_gu: torch.Tensor | None,
                xcal_dn: torch.Tensor | None, b: int) -> MoELayer:
    """Per expert e: calibrate the gate/up input on xcal_gu[e] and the down
    input on xcal_dn[e], fold c_b into the multipliers, and prepare the
    stacked gate/up [2F, H] and down [H, F] weights. With no calibration rows
    and b == 0 the block is plain MXFP4."""
    E, F, H = w_gate.shape
    dev = w_gate.device
    wgu_rows = stack_gate_up(w_gate, w_up)
    wgu = empty_grouped_weights(E, 2 * F, H, dev)
    wdn = empty_grouped_weights(E, H, F, dev)
    plain = xcal_gu is None
    if plain and b != 0:
        raise ValueError("a Hadamard block without calibration rows is not a MACaQ layer")
    a_gu = None if plain else torch.empty(E, H, dtype=torch.float32, device=dev)
    a_dn = None if plain else torch.empty(E, F, dtype=torch.float32, device=dev)
    for e in range(E):
        if plain:
            prepare_weights(wgu_rows[e], None, 0, out=expert(wgu, e))
            prepare_weights(w_dn[e], None, 0, out=expert(wdn, e))
            continue
        a, r = make_multipliers(calibrate(xcal_gu[e]), b)
        a_gu[e] = a
        prepare_weights(wgu_rows[e], r, b, out=expert(wgu, e))
        a, r = make_multipliers(calibrate(xcal_dn[e]), b)
        a_dn[e] = a
        prepare_weights(w_dn[e], r, b, out=expert(wdn, e))
    return MoELayer(a_gu, wgu, a_dn, wdn, b)


# ---- Flip-Refinement (offline) ---------------------------------------------

def hessian(xcal: torch.Tensor, a: torch.Tensor | None, b: int) -> torch.Tensor:
    """H = X~^T X~ (fp64 [K, K]) of bf16 calibration rows through a and the
    block-Hadamard of size b."""
    _need_cuda(xcal, a)
    assert xcal.dtype == torch.bfloat16 and xcal.dim() == 2 and xcal.stride(1) == 1
    R, K = xcal.shape
    H = torch.empty(K, K, dtype=torch.float64, device=xcal.device)
    ws = _workspace(int(load_library().macaq_hessian_workspace_size(R, K)), xcal.device, None)
    _check(load_library().macaq_hessian(_ptr(xcal), R, K, xcal.stride(0), _ptr(a), b, _ptr(H), _ptr(ws), ws.numel(),
                                        _stream(xcal)), "macaq_hessian")
    return H


def flip_refine(w: torch.Tensor, r: torch.Tensor | None, b: int, H: torch.Tensor, max_flips: int, packed: Packed,
                workspace: torch.Tensor | None = None) -> torch.Tensor:
    """Refine packed (from prepare_weights(w, r, b)) in place; returns the
    number of moves of every row (int32 [N])."""
    _need_cuda(w, r, H, packed.codes, packed.scales)
    assert w.dim() == 2 and w.stride(1) == 1 and H.dtype == torch.float64 and H.is_contiguous()
    N, K = w.shape
    flips = torch.empty(N, dtype=torch.int32, device=w.device)
    ws = _workspace(int(load_library().macaq_flip_refine_workspace_size(N, K)), w.device, workspace)
    _check(load_library().macaq_flip_refine(_ptr(w), _dtype_code(w.dtype), N, K, w.stride(0), _ptr(r), b, _ptr(H),
                                            max_flips, _ptr(packed.codes), _ptr(packed.scales), _ptr(flips),
                                            _ptr(ws), ws.numel(), _stream(w)), "macaq_flip_refine")
    return flips
