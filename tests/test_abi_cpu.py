"""The C-ABI library loads, exports what include/macaq.h declares, and rejects
bad arguments on the host, before touching any device (no GPU needed: only
argument checks run, no kernel is launched and no pointer is dereferenced)."""
import ctypes
import os
import re

import pytest

from mxfp4_w4a4_post_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "macaq.h")

OK, EINVAL, EALIGN, EWORKSPACE, EUNSUPPORTED, EHIP = range(6)
FAKE = 0x10000  # an aligned address that is never dereferenced: every call below fails its host checks first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(macaq_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return binding.load_library()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) == 31, names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(binding._SIGNATURES), "binding signatures out of sync with the header"


def test_status_strings(lib):
    for code in range(6):
        s = lib.macaq_status_string(code).decode()
        assert s and s != "unknown status"
    assert lib.macaq_status_string(99).decode() == "unknown status"


def _last(lib):
    return lib.macaq_last_error().decode()


def test_quant_act_rejects(lib):
    def f(X, M, K, ldx, a, b, codes, scales, stream, layout=0):
        return lib.macaq_quant_act(X, M, K, ldx, a, b, layout, codes, scales, stream)

    assert f(None, 4, 64, 64, None, 32, FAKE, FAKE, None) == EINVAL
    assert f(FAKE, 4, 48, 48, None, 0, FAKE, FAKE, None) == EINVAL  # K % 32
    assert "multiple of 32" in _last(lib)
    assert f(FAKE, 4, 96, 96, None, 64, FAKE, FAKE, None) == EINVAL  # K % b
    assert f(FAKE, 4, 64, 64, None, 16, FAKE, FAKE, None) == EINVAL  # b not allowed
    assert f(FAKE, 4, 64, 32, None, 32, FAKE, FAKE, None) == EINVAL  # ldx < K
    assert f(FAKE, -1, 64, 64, None, 32, FAKE, FAKE, None) == EINVAL
    assert f(FAKE, 4, 64, 64, None, 32, FAKE, FAKE, None, layout=7) == EINVAL
    assert f(FAKE, 1 << 24, 1 << 10, 1 << 10, None, 32, FAKE, FAKE, None, layout=1) == EINVAL  # over 2 GiB packed
    assert f(FAKE + 2, 4, 64, 64, None, 32, FAKE, FAKE, None) == EALIGN
    assert f(FAKE, 4, 64, 68, None, 32, FAKE, FAKE, None) == EALIGN  # ldx not a multiple of 8
    assert f(FAKE, 4, 64, 64, FAKE + 4, 32, FAKE, FAKE, None) == EALIGN
    assert f(None, 0, 64, 64, None, 32, None, None, None) == OK  # empty: nothing to do


def test_prepare_weights_rejects(lib):
    def f(W, dt, N, K, ldw, r, b, codes, scales, layout=1):
        return lib.macaq_prepare_weights(W, dt, N, K, ldw, r, b, layout, codes, scales, None)

    assert f(FAKE, 7, 8, 64, 64, None, 32, FAKE, FAKE) == EINVAL  # dtype
    assert f(FAKE, 1, 8, 64, 66, None, 32, FAKE, FAKE) == EALIGN  # fp32 rows not 16-byte multiples
    assert f(FAKE, 0, 8, 64, 64, None, 32, None, FAKE) == EINVAL
    assert f(FAKE, 0, 8, 64, 64, None, 32, FAKE, FAKE, layout=5) == EINVAL  # bad layout
    assert f(FAKE, 0, 1 << 24, 1 << 10, 1 << 10, None, 32, FAKE, FAKE) == EINVAL  # GEMM layout over 2 GiB
    assert f(FAKE, 0, 0, 64, 64, None, 32, FAKE, FAKE) == OK
    assert f(FAKE, 0, 0, 64, 64, None, 32, FAKE, FAKE, layout=0) == OK


def test_linear_rejects(lib):
    f = lib.macaq_linear
    good = dict(X=FAKE, M=4, K=64, ldx=64, a=None, b=32, wc=FAKE, ws=FAKE, N=16, Y=FAKE, dt=0, ldy=16)

    def call(**kw):
        d = dict(good)
        d.update(kw)
        return f(d["X"], d["M"], d["K"], d["ldx"], d["a"], d["b"], d["wc"], d["ws"], d["N"], d["Y"], d["dt"],
                 d["ldy"], kw.get("wsp", FAKE), kw.get("wsb", 0), None)

    assert call(N=0) == EINVAL
    assert call(ldy=8) == EINVAL
    assert call(dt=3) == EINVAL
    assert call(Y=None) == EINVAL
    assert call(Y=FAKE + 1) == EALIGN  # bf16 output must be 2-byte aligned
    assert call(Y=FAKE + 2, dt=1) == EALIGN  # fp32 output must be 4-byte aligned
    need = lib.macaq_linear_workspace_size(4, 64, 16)
    assert need > 0
    assert call(wsb=need - 1) == EWORKSPACE
    assert call(wsp=FAKE + 16, wsb=need) == EWORKSPACE  # workspace must be 256-byte aligned
    assert call(wsp=None, wsb=need) == EWORKSPACE
    assert call(M=0) == OK


def test_gemm_and_grouped_reject(lib):
    assert lib.macaq_gemm(FAKE, FAKE, 4, 40, FAKE, FAKE, 16, FAKE, 0, 16, FAKE, 0, None) == EINVAL
    assert lib.macaq_gemm(FAKE, FAKE, 4, 64, FAKE + 1, FAKE, 16, FAKE, 0, 16, FAKE, 0, None) == EALIGN
    g = lib.macaq_linear_grouped
    assert g(FAKE, FAKE, 0, 16, 64, None, 0, FAKE, FAKE, 8, FAKE, 0, FAKE, 0, None) == EINVAL  # E < 1
    assert g(FAKE, None, 2, 16, 64, None, 0, FAKE, FAKE, 8, FAKE, 0, FAKE, 0, None) == EINVAL
    assert g(FAKE, FAKE, 2, 16, 64, None, 0, FAKE, FAKE, 8, FAKE, 0, FAKE, 0, None) == EWORKSPACE
    assert g(FAKE, FAKE, 2, 0, 64, None, 0, FAKE, FAKE, 8, FAKE, 0, FAKE, 0, None) == OK


def test_probes_reject(lib):
    m = lib.macaq_debug_mfma_probe
    assert m(None, 256, 10, FAKE, None) == EINVAL
    assert m(FAKE, 0, 10, FAKE, None) == EINVAL
    assert m(FAKE, 70000, 10, FAKE, None) == EINVAL
    assert m(FAKE, 256, 0, FAKE, None) == EINVAL
    assert m(FAKE + 4, 256, 10, FAKE, None) == EALIGN
    r = lib.macaq_debug_read_probe
    assert r(FAKE, 1 << 20, 256, None, None) == EINVAL
    assert r(FAKE, 8, 256, FAKE, None) == EINVAL
    assert r(FAKE, 1 << 20, 0, FAKE, None) == EINVAL
    assert r(FAKE, (1 << 20) + 4, 256, FAKE, None) == EALIGN
    assert r(FAKE + 8, 1 << 20, 256, FAKE, None) == EALIGN


def test_calibrate_and_multipliers_reject(lib):
    assert lib.macaq_calibrate(FAKE, 0, 8, 8, FAKE, None) == EINVAL
    assert lib.macaq_calibrate(FAKE, 4, 8, 4, FAKE, None) == EINVAL
    assert lib.macaq_calibrate(FAKE + 1, 4, 8, 8, FAKE, None) == EALIGN
    d = lib.macaq_make_multipliers_device
    assert d(FAKE, 8, 48, FAKE, FAKE, None) == EINVAL
    assert d(FAKE, 8, 32, None, None, None) == EINVAL
    assert d(FAKE, 0, 32, FAKE, None, None) == EINVAL
    assert d(FAKE + 2, 8, 32, FAKE, None, None) == EALIGN


def _f32(a):
    import numpy as np
    a = np.ascontiguousarray(a, dtype=np.float32)
    return a, a.ctypes.data


def test_make_multipliers_host_matches_oracle(lib, orc):
    """The host-only macaq_make_multipliers (no device, no stream) against
    the oracle, bit for bit, for every Hadamard block, on scales that span
    the fp32 range (subnormal to near overflow) and values whose quotient
    and product round at a tie-adjacent point."""
    import numpy as np
    rng = np.random.default_rng(11)
    s = np.concatenate([
        np.float32(2.0) ** rng.integers(-149, 127, size=300).astype(np.float32),
        (rng.random(300) * 100 + 1e-3).astype(np.float32),
        np.array([1.0, 3.0, np.float32(np.sqrt(2.0)), 1e-40, 3.4e38, 0.1], np.float32),
    ]).astype(np.float32)
    for b in (0, 32, 64, 128):
        a_o, r_o = orc.multipliers(s, b)
        s_, sp = _f32(s)
        a = np.full_like(s, np.nan)
        r = np.full_like(s, np.nan)
        assert lib.macaq_make_multipliers(sp, s.size, b, a.ctypes.data, r.ctypes.data) == OK
        assert np.array_equal(a.view(np.uint32), a_o.view(np.uint32)), b
        assert np.array_equal(r.view(np.uint32), r_o.view(np.uint32)), b
        # either output may be skipped
        a2 = np.zeros_like(s)
        assert lib.macaq_make_multipliers(sp, s.size, b, a2.ctypes.data, None) == OK
        assert np.array_equal(a2.view(np.uint32), a_o.view(np.uint32))


def test_make_multipliers_host_rejects(lib):
    """Bad arguments and non-positive or non-finite scales: a status, and
    nothing written."""
    import numpy as np
    s, sp = _f32([1.0, 2.0, 0.0, 4.0])
    a = np.full(4, 7.0, np.float32)
    assert lib.macaq_make_multipliers(sp, 4, 32, a.ctypes.data, None) == EINVAL  # s[2] == 0
    assert "s[2]" in _last(lib)
    for bad in (-1.0, np.inf, np.nan):
        s2, sp2 = _f32([1.0, bad])
        assert lib.macaq_make_multipliers(sp2, 2, 32, a.ctypes.data, None) == EINVAL
    assert np.all(a == 7.0)
    assert lib.macaq_make_multipliers(sp, 4, 48, a.ctypes.data, None) == EINVAL  # block
    assert lib.macaq_make_multipliers(sp, 0, 32, a.ctypes.data, None) == EINVAL  # K
    assert lib.macaq_make_multipliers(None, 4, 32, a.ctypes.data, None) == EINVAL
    assert lib.macaq_make_multipliers(sp, 4, 32, None, None) == EINVAL
    assert lib.macaq_make_multipliers(sp + 2, 2, 32, a.ctypes.data, None) == EALIGN
    assert np.all(a == 7.0)


def test_binding_host_multipliers(orc):
    import numpy as np
    s = np.array([0.5, 2.0, 9.0, 1e-3], np.float32)
    a, r = binding.make_multipliers_host(s, 64)
    a_o, r_o = orc.multipliers(s, 64)
    assert np.array_equal(a, a_o) and np.array_equal(r, r_o)


def test_unsupported_device_reported_before_any_work(lib):
    """With the device check told it runs on another architecture, every
    enqueuing call returns MACAQ_EUNSUPPORTED after its argument checks, and
    the caller's output stays untouched (host buffers stand in for device
    memory: nothing may be written or launched)."""
    import numpy as np
    y = np.full(4 * 16, 3.0, np.float32)
    codes = np.full(4 * 64 // 2, 0xAB, np.uint8)
    scales = np.full(4 * 64 // 32, 0xCD, np.uint8)
    x = np.zeros((4, 64), np.uint16)
    ws = np.zeros(1 << 16, np.uint8)
    wsp = (ws.ctypes.data + 255) // 256 * 256
    binding.override_arch("gfx942")
    try:
        st = lib.macaq_quant_act(x.ctypes.data, 4, 64, 64, None, 32, 0, codes.ctypes.data, scales.ctypes.data, None)
        assert st == EUNSUPPORTED and "gfx942" in _last(lib)
        st = lib.macaq_prepare_weights(x.ctypes.data, 0, 4, 64, 64, None, 32, 0, codes.ctypes.data,
                                       scales.ctypes.data, None)
        assert st == EUNSUPPORTED
        st = lib.macaq_linear(x.ctypes.data, 4, 64, 64, None, 32, FAKE, FAKE, 16, y.ctypes.data, 1, 16, wsp,
                              len(ws) - 256, None)
        assert st == EUNSUPPORTED
        assert lib.macaq_make_multipliers_device(FAKE, 8, 32, FAKE, FAKE, None) == EUNSUPPORTED
        # argument errors still win over the device check
        assert lib.macaq_linear(x.ctypes.data, 4, 64, 64, None, 32, FAKE, FAKE, 0, y.ctypes.data, 1, 16, wsp,
                                len(ws) - 256, None) == EINVAL
        # the host-only call needs no device
        s, sp = _f32([1.0, 2.0])
        a = np.zeros(2, np.float32)
        assert lib.macaq_make_multipliers(sp, 2, 32, a.ctypes.data, None) == OK
    finally:
        binding.override_arch(None)
    assert np.all(y == 3.0) and np.all(codes == 0xAB) and np.all(scales == 0xCD)


def test_packed_sizes(lib):
    """GEMM layout: rows padded to 32, K to 256; codes K/2 and scales K/32 bytes a row."""
    for rows, K in [(1, 32), (16, 256), (65, 96), (2048, 4096), (8192, 28672)]:
        RP, KP = -(-rows // 32) * 32, -(-K // 256) * 256
        assert lib.macaq_packed_codes_bytes(rows, K) == RP * KP // 2
        assert lib.macaq_packed_scales_bytes(rows, K) == RP * KP // 32
    assert lib.macaq_packed_codes_bytes(0, 64) == 0


def test_workspace_sizes_cover_staging(lib):
    # quantized activations staged in the workspace in the GEMM layout, 256-byte padded
    for M, K, N in [(16, 256, 256), (2048, 4096, 4096), (1, 25600, 5120), (8192, 28672, 8192)]:
        need = lib.macaq_linear_workspace_size(M, K, N)
        assert need >= lib.macaq_packed_codes_bytes(M, K) + lib.macaq_packed_scales_bytes(M, K)
        assert need % 256 == 0
    assert lib.macaq_linear_workspace_size(0, 64, 16) == 0
    T, E, K, N = 32768, 128, 2048, 1536
    assert lib.macaq_linear_grouped_workspace_size(T, E, K, N) >= T * K // 2 + T * K // 32


def test_binding_has_no_cpu_fallback():
    """The product path refuses CPU tensors instead of computing elsewhere."""
    import torch
    with pytest.raises(ValueError):
        binding.quant_act(torch.zeros(4, 64, dtype=torch.bfloat16), None, 0)


def test_moe_calls_reject(lib):
    """Host checks of the MoE block calls (nothing is dereferenced)."""
    ws = 1 << 30
    # route: bad E, k, T*k overflow, NULL, misaligned, short or missing workspace
    assert lib.macaq_moe_route(FAKE, 16, 2, 0, FAKE, FAKE, FAKE, FAKE, ws, None) == EINVAL
    assert lib.macaq_moe_route(FAKE, 16, 2, 5000, FAKE, FAKE, FAKE, FAKE, ws, None) == EINVAL
    assert lib.macaq_moe_route(FAKE, 16, 0, 8, FAKE, FAKE, FAKE, FAKE, ws, None) == EINVAL
    assert lib.macaq_moe_route(FAKE, 1 << 30, 8, 8, FAKE, FAKE, FAKE, FAKE, ws, None) == EINVAL
    assert lib.macaq_moe_route(None, 16, 2, 8, FAKE, FAKE, FAKE, FAKE, ws, None) == EINVAL
    assert lib.macaq_moe_route(FAKE + 2, 16, 2, 8, FAKE, FAKE, FAKE, FAKE, ws, None) == EALIGN
    need = lib.macaq_moe_route_workspace_size(16, 2, 8)
    assert need >= 8 * 4 and lib.macaq_moe_route_workspace_size(16, 2, 0) == 0
    assert lib.macaq_moe_route(FAKE, 16, 2, 8, FAKE, FAKE, FAKE, FAKE, need - 1, None) == EWORKSPACE
    assert lib.macaq_moe_route(FAKE, 16, 2, 8, FAKE, FAKE, FAKE, None, need, None) == EWORKSPACE
    assert lib.macaq_moe_route(FAKE, 16, 2, 8, FAKE, FAKE, FAKE, FAKE + 16, need, None) == EWORKSPACE

    def gate_up(X=FAKE, T=16, H=256, ldx=256, k=2, E=8, a_gu=FAKE, b=32, F=128, a_dn=FAKE, dn=FAKE, wsb=ws,
                wsp=FAKE):
        return lib.macaq_moe_gate_up(X, T, H, ldx, k, FAKE, FAKE, E, a_gu, b, FAKE, FAKE, F, a_dn, dn, FAKE, wsp,
                                     wsb, None)

    assert gate_up(H=48) == EINVAL          # H % 32
    assert gate_up(F=96, b=64) == EINVAL    # F % b
    assert gate_up(b=16) == EINVAL
    assert gate_up(ldx=128) == EINVAL
    assert gate_up(a_gu=None) == EINVAL     # b > 0 needs multipliers
    assert gate_up(X=FAKE + 8) == EALIGN
    assert gate_up(dn=FAKE + 4) == EALIGN
    assert gate_up(wsb=16) == EWORKSPACE
    assert gate_up(wsp=FAKE + 16) == EWORKSPACE
    assert gate_up(T=0) == OK               # nothing to do

    def down(T=16, k=2, E=8, H=256, F=128, Y=FAKE, dt=0, ldy=256, wsb=ws):
        return lib.macaq_moe_down_combine(FAKE, FAKE, FAKE, FAKE, FAKE, T, k, E, FAKE, FAKE, H, F, Y, dt, ldy, FAKE,
                                          wsb, None)

    assert down(ldy=128) == EINVAL
    assert down(dt=3) == EINVAL
    assert down(Y=None) == EINVAL
    assert down(E=0) == EINVAL
    assert down(wsb=0) == EWORKSPACE

    def block(T=16, H=256, ldx=256, k=2, E=8, b=32, F=128, wsb=ws, a_dn=FAKE):
        return lib.macaq_moe_block(FAKE, T, H, ldx, FAKE, FAKE, k, E, FAKE, FAKE, FAKE, a_dn, FAKE, FAKE, F, b, FAKE,
                                   0, H, FAKE, wsb, None)

    assert block(a_dn=None) == EINVAL
    assert block(F=40) == EINVAL
    assert block(wsb=1024) == EWORKSPACE
    assert block(T=0) == OK
    need = lib.macaq_moe_workspace_size(16, 2, 8, 256, 128)
    assert need > 0 and block(wsb=need - 1) == EWORKSPACE
    assert lib.macaq_moe_workspace_size(0, 2, 8, 256, 128) == 0


def test_refine_calls_reject(lib):
    ws = 1 << 30
    H = lib.macaq_hessian
    assert H(FAKE, 0, 64, 64, FAKE, 32, FAKE, FAKE, ws, None) == EINVAL      # R < 1
    assert H(FAKE, 8, 48, 48, FAKE, 32, FAKE, FAKE, ws, None) == EINVAL      # K % 32
    assert H(FAKE, 8, 65536, 65536, FAKE, 32, FAKE, FAKE, ws, None) == EINVAL  # K too large
    assert H(FAKE, 8, 64, 64, None, 32, FAKE, FAKE, ws, None) == EINVAL      # a needed
    assert H(FAKE, 8, 64, 64, FAKE, 32, FAKE + 8, FAKE, ws, None) == EALIGN
    assert H(FAKE, 8, 64, 64, FAKE, 32, FAKE, FAKE, 16, None) == EWORKSPACE
    assert lib.macaq_hessian_workspace_size(8, 64) == 8 * 64 * 4 + (256 - 8 * 64 * 4 % 256) % 256
    F = lib.macaq_flip_refine

    def f(N=8, K=64, ldw=64, dt=0, b=32, cap=4, r=FAKE, W=FAKE, wsb=ws):
        return F(W, dt, N, K, ldw, r, b, FAKE, cap, FAKE, FAKE, None, FAKE, wsb, None)

    assert f(cap=-1) == EINVAL
    assert f(dt=7) == EINVAL
    assert f(r=None) == EINVAL
    assert f(K=96, ldw=96, b=64) == EINVAL
    assert f(W=FAKE + 4) == EALIGN
    assert f(dt=1, ldw=66) == EALIGN
    assert f(wsb=100) == EWORKSPACE
    assert lib.macaq_flip_refine_workspace_size(8, 64) >= 2 * 8 * 64 * 8 + 64 * 8


def test_calibrate_pow_rejects(lib):
    assert lib.macaq_calibrate_pow(FAKE, 4, 64, 64, 3, FAKE, None) == EINVAL
    assert lib.macaq_calibrate_pow(None, 4, 64, 64, 1, FAKE, None) == EINVAL
    assert lib.macaq_calibrate_pow(FAKE, 0, 64, 64, 4, FAKE, None) == EINVAL
    assert lib.macaq_calibrate_pow(FAKE + 1, 4, 64, 64, 0, FAKE, None) == EALIGN
