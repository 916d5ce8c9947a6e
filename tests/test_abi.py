"""The C-ABI library loads, exports every entry point the header declares,
and validates arguments on the host (no device is touched on these paths)."""
import ctypes
import os
import re

import pytest

import gemm_router_fp32_amd as g

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(g.SO_PATH):
        from gemm_router_fp32_amd import build
        build.build()
    return g.lib()


def _declared():
    src = open(os.path.join(ROOT, "include", "q4moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(q4moe_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert len(names) >= 16
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(g.EXPORTS)


def test_version_and_strings(L):
    assert g.q4moe_abi_version() == 1
    assert L.q4moe_status_str(0) == b"ok"
    assert L.q4moe_status_str(4) == b"workspace too small"


A16 = 1 << 20  # a fake 16-byte-aligned device address; never dereferenced


def _router(E=128, H=2688, k=6, wg=A16, b=A16):
    return g.RouterS(wg, b, E, H, k)


def _experts(fmt=1, E=128, H=2688, I=1856, gs=A16):
    return g.ExpertsS(fmt, E, H, I, A16, A16, gs if fmt == 1 else None, A16, A16, gs if fmt == 1 else None)


def _decode(L, r, ex, x=A16, T=1, y=A16, ws=A16, wsb=1 << 30):
    return L.q4moe_w4a16_decode(ctypes.byref(r), ctypes.byref(ex), x, T, y, None, None, ws, wsb, None)


def test_decode_validation(L):
    r, ex = _router(), _experts()
    assert _decode(L, r, ex, x=None) == g.EINVAL
    assert _decode(L, _router(k=0), ex) == g.EINVAL
    assert _decode(L, _router(k=9), ex) == g.EINVAL
    assert _decode(L, _router(wg=None), ex) == g.EINVAL
    assert _decode(L, r, ex, T=0) == g.EINVAL
    assert _decode(L, r, ex, T=65537) == g.EINVAL
    # NVFP4 above 8 tokens takes the grouped path: hidden and inter multiples of 64
    assert _decode(L, r, _experts(I=1856 + 32), T=9) == g.EUNSUPPORTED
    assert b"multiples of 64" in L.q4moe_last_error()
    # the grouped entry point: the same rule at any token count
    assert L.q4moe_w4a16_grouped(ctypes.byref(r), ctypes.byref(_experts(I=1856 + 32)), A16, 1, A16, None, None,
                                 A16, 1 << 30, None) == g.EUNSUPPORTED
    assert L.q4moe_w4a16_grouped(ctypes.byref(r), ctypes.byref(ex), A16, 0, A16, None, None, A16, 1 << 30,
                                 None) == g.EINVAL
    gneed = L.q4moe_w4a16_grouped_ws_bytes(ctypes.byref(r), ctypes.byref(ex), 2)
    assert gneed > L.q4moe_w4a16_decode_ws_bytes(ctypes.byref(r), ctypes.byref(ex), 2)
    assert L.q4moe_w4a16_grouped(ctypes.byref(r), ctypes.byref(ex), A16, 2, A16, None, None, A16, gneed - 1,
                                 None) == g.EWORKSPACE
    assert _decode(L, r, _experts(I=1850)) == g.EINVAL
    assert _decode(L, r, _experts(fmt=7)) == g.EINVAL
    assert _decode(L, r, _experts(gs=None)) == g.EINVAL
    assert _decode(L, _router(H=2600), _experts(H=2600)) == g.EINVAL
    assert b"hidden" in L.q4moe_last_error()
    assert _decode(L, r, ex, x=A16 + 2) == g.EALIGN
    assert _decode(L, r, ex, ws=A16 + 8) == g.EALIGN
    need = L.q4moe_w4a16_decode_ws_bytes(ctypes.byref(r), ctypes.byref(ex), 1)
    assert need > 0
    assert _decode(L, r, ex, wsb=need - 1) == g.EWORKSPACE


def test_int4_needs_group_64(L):
    # every call here fails validation, so nothing reaches a device
    r = _router(H=2688)
    assert _decode(L, r, _experts(fmt=2, I=1856 + 32)) == g.EINVAL  # 1888 % 64 != 0
    ex = g.ExpertsS(2, 128, 2688, 1856, A16, A16, A16, A16, A16, None)  # int4 takes no gscale
    assert _decode(L, r, ex) == g.EINVAL


def test_no_device_is_a_clean_status(L):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a device is present")
    r, ex = _router(), _experts()
    assert _decode(L, r, ex) == g.EDEVICE
    assert b"device" in L.q4moe_last_error().lower()


def test_dequant_and_gemv_validation(L):
    m = g.QMatS(1, 128, 2688, A16, A16, A16)
    assert L.q4moe_dequant_ref(ctypes.byref(m), None, None) == g.EINVAL
    assert L.q4moe_dequant_ref(ctypes.byref(g.QMatS(1, 128, 40, A16, A16, A16)), A16, None) == g.EINVAL
    assert L.q4moe_dequant_ref(ctypes.byref(g.QMatS(2, 128, 2688, A16, A16, A16)), A16, None) == g.EINVAL
    assert L.q4moe_dequant_ref(ctypes.byref(g.QMatS(1, 128, 2688, A16, A16 + 1, A16)), A16, None) == g.EALIGN
    need = L.q4moe_w4a16_gemv_ws_bytes(ctypes.byref(m), 4)
    assert L.q4moe_w4a16_gemv(ctypes.byref(m), A16, 5, A16, None, A16, need, None) == g.EINVAL
    assert L.q4moe_w4a16_gemv(ctypes.byref(m), A16, 4, A16, None, A16, need - 1, None) == g.EWORKSPACE
    mi = g.QMatS(2, 128, 2688, A16, A16, None)
    assert L.q4moe_w4a16_gemv(ctypes.byref(mi), A16, 1, A16, None, A16, need, None) == g.EUNSUPPORTED


def test_router_validation(L):
    r = _router()
    assert L.q4moe_router_topk(ctypes.byref(r), A16, 0, A16, A16, None, A16, 1 << 20, None) == g.EINVAL
    assert L.q4moe_router_topk(ctypes.byref(_router(E=300)), A16, 1, A16, A16, None, A16, 1 << 20, None) == g.EINVAL
    assert L.q4moe_router_topk(ctypes.byref(r), A16, 1, A16 + 2, A16, None, A16, 1 << 20, None) == g.EALIGN
    assert L.q4moe_router_topk(ctypes.byref(r), A16, 1, A16, A16, None, A16, 8, None) == g.EWORKSPACE


def _shared(H=2688, S=3712, up=A16, dn=A16, sc=(2.0 ** -8, 2.0 ** -6, 2.0 ** -8, 2.0 ** -5)):
    return g.SharedFp8S(H, S, up, dn, *sc)


def _decode_sh(L, r, ex, sh, T=1, x=A16, ws=A16, wsb=1 << 30):
    shp = None if sh is None else ctypes.byref(sh)
    return L.q4moe_w4a16_decode_shared(ctypes.byref(r), ctypes.byref(ex), shp, x, T, A16, None, None, ws, wsb, None)


def test_decode_shared_validation(L):
    # every call here fails validation, so nothing reaches a device
    r, ex = _router(), _experts()
    assert _decode_sh(L, r, ex, None) == g.EINVAL
    assert _decode_sh(L, r, ex, _shared(H=2560)) == g.EINVAL
    assert _decode_sh(L, r, ex, _shared(S=3700)) == g.EINVAL
    assert _decode_sh(L, r, ex, _shared(S=8192)) == g.EINVAL
    assert _decode_sh(L, r, ex, _shared(up=None)) == g.EINVAL
    assert _decode_sh(L, r, ex, _shared(dn=A16 + 8)) == g.EALIGN
    assert _decode_sh(L, r, ex, _shared(sc=(1.0, 0.0, 1.0, 1.0))) == g.EINVAL
    assert _decode_sh(L, r, ex, _shared(sc=(1.0, 1.0, float("inf"), 1.0))) == g.EINVAL
    # more than 4 tokens (or int4 routed experts): the grouped GEMMs, hidden and inter multiples of 64
    assert _decode_sh(L, r, _experts(I=1856 + 32), _shared(), T=5) == g.EUNSUPPORTED
    need5 = L.q4moe_w4a16_decode_shared_ws_bytes(ctypes.byref(r), ctypes.byref(ex), ctypes.byref(_shared()), 5)
    assert _decode_sh(L, r, ex, _shared(), T=5, wsb=need5 - 1) == g.EWORKSPACE
    need_i4 = L.q4moe_w4a16_decode_shared_ws_bytes(ctypes.byref(r), ctypes.byref(_experts(fmt=2)),
                                                   ctypes.byref(_shared()), 1)
    assert _decode_sh(L, r, _experts(fmt=2), _shared(), wsb=need_i4 - 1) == g.EWORKSPACE
    sh = _shared()
    need = L.q4moe_w4a16_decode_shared_ws_bytes(ctypes.byref(r), ctypes.byref(ex), ctypes.byref(sh), 1)
    plain = L.q4moe_w4a16_decode_ws_bytes(ctypes.byref(r), ctypes.byref(ex), 1)
    assert need > plain
    assert _decode_sh(L, r, ex, sh, wsb=need - 1) == g.EWORKSPACE
    t = g.SharedTaps()
    assert L.q4moe_w4a16_decode_shared_taps(ctypes.byref(r), ctypes.byref(ex), ctypes.byref(sh), 1,
                                            ctypes.byref(t)) == g.OK
    assert 0 < t.xq < t.sh_h32 < t.sh_hq < need and t.y32 < need
    # 2-4 tokens: per-token taps and the shared output buffer
    need4 = L.q4moe_w4a16_decode_shared_ws_bytes(ctypes.byref(r), ctypes.byref(ex), ctypes.byref(sh), 4)
    assert L.q4moe_w4a16_decode_shared_taps(ctypes.byref(r), ctypes.byref(ex), ctypes.byref(sh), 4,
                                            ctypes.byref(t)) == g.OK
    assert t.sh_h32 - t.xq >= 4 * 2688 and t.sh_hq - t.sh_h32 >= 4 * 3712 * 4
    assert t.sh_hq + 4 * 3712 + 4 * 2688 * 4 <= need4
    assert _decode_sh(L, r, ex, sh, T=4, wsb=need4 - 1) == g.EWORKSPACE


def test_w4a4_decode_validation(L):
    r, ex = _router(), _experts()

    def call(ex_, T=1, wsb=1 << 30):
        return L.q4moe_w4a4_decode(ctypes.byref(r), ctypes.byref(ex_), A16, T, A16, None, None, A16, wsb, None)

    assert call(ex, T=9) == g.EUNSUPPORTED
    assert call(_experts(fmt=2)) == g.EUNSUPPORTED
    assert call(ex, T=0) == g.EINVAL
    need = L.q4moe_w4a4_decode_ws_bytes(ctypes.byref(r), ctypes.byref(ex), 1)
    assert need > L.q4moe_w4a16_decode_ws_bytes(ctypes.byref(r), ctypes.byref(ex), 1)
    assert call(ex, wsb=need - 1) == g.EWORKSPACE
    t = g.W4A4TokenTaps()
    assert L.q4moe_w4a4_decode_taps(ctypes.byref(r), ctypes.byref(ex), 1, ctypes.byref(t)) == g.OK
    assert t.xq_codes < t.xq_scales < t.hq_codes < t.hq_scales < need


def test_w4a4_decode_shared_validation(L):
    r, ex, sh = _router(), _experts(), _shared()
    def call(ex_, sh_, T=1, wsb=1 << 30):
        shp = None if sh_ is None else ctypes.byref(sh_)
        return L.q4moe_w4a4_decode_shared(ctypes.byref(r), ctypes.byref(ex_), shp, A16, T, A16, None, None, A16, wsb,
                                          None)
    assert call(ex, None) == g.EINVAL
    assert call(ex, sh, T=5) == g.EUNSUPPORTED
    assert call(_experts(fmt=2), sh) == g.EUNSUPPORTED
    assert call(ex, _shared(S=100)) == g.EINVAL
    need = L.q4moe_w4a4_decode_shared_ws_bytes(ctypes.byref(r), ctypes.byref(ex), ctypes.byref(sh), 1)
    assert need > L.q4moe_w4a4_decode_ws_bytes(ctypes.byref(r), ctypes.byref(ex), 1)
    assert call(ex, sh, wsb=need - 1) == g.EWORKSPACE


def test_quantize_weights_validation(L):
    need = L.q4moe_quantize_weights_ws_bytes(64, 2688)
    assert need > 0

    def call(rows=64, cols=2688, mode=0, w=A16, codes=A16, wsb=need):
        return L.q4moe_quantize_weights(w, rows, cols, mode, codes, A16, A16, A16, wsb, None)

    assert call(cols=40) == g.EINVAL
    assert call(rows=0) == g.EINVAL
    assert call(mode=2) == g.EINVAL
    assert call(w=None) == g.EINVAL
    assert call(w=A16 + 8) == g.EALIGN
    assert call(codes=A16 + 4) == g.EALIGN
    assert call(wsb=need - 1) == g.EWORKSPACE


def test_fp8_gemv_validation(L):
    # every call here fails validation, so nothing reaches a device
    def mat(rows=1024, cols=2688, codes=A16, ws=2.0 ** -8, is_=2.0 ** -6):
        return g.Fp8MatS(rows, cols, codes, ws, is_)

    need = L.q4moe_fp8_gemv_ws_bytes(ctypes.byref(mat()), 4)

    def call(m, T=1, x=A16, wsb=need, logits=A16):
        return L.q4moe_fp8_gemv(ctypes.byref(m), x, T, logits, None, A16, wsb, None)

    assert need > L.q4moe_fp8_gemv_ws_bytes(ctypes.byref(mat()), 1)
    assert call(mat(cols=2600)) == g.EINVAL
    assert call(mat(cols=8192)) == g.EINVAL
    assert call(mat(), T=5) == g.EINVAL
    assert call(mat(is_=0.0)) == g.EINVAL
    assert call(mat(ws=float("nan"))) == g.EINVAL
    assert call(mat(codes=None)) == g.EINVAL
    assert call(mat(codes=A16 + 4)) == g.EALIGN
    assert call(mat(), x=A16 + 2) == g.EALIGN
    assert call(mat(), T=4, wsb=need - 1) == g.EWORKSPACE
    assert call(mat(rows=1 << 21, cols=4096)) == g.EUNSUPPORTED
    off = ctypes.c_size_t(0)
    assert L.q4moe_fp8_gemv_taps(ctypes.byref(mat()), 4, ctypes.byref(off)) == g.OK
    assert 0 < off.value and off.value + 4 * 2688 <= need


def test_decode_shared_q4_validation(L):
    # the 4-bit shared expert is a bank of one expert; every call here fails
    # validation, so nothing reaches a device
    r, ex = _router(), _experts()

    def sh4(fmt=2, E=1, H=2688, S=3712, gs=A16):
        return g.ExpertsS(fmt, E, H, S, A16, A16, gs if fmt == 1 else None, A16, A16, gs if fmt == 1 else None)

    def call(ex_, sh_, T=1, wsb=1 << 30):
        shp = None if sh_ is None else ctypes.byref(sh_)
        return L.q4moe_w4a16_decode_shared_q4(ctypes.byref(r), ctypes.byref(ex_), shp, A16, T, A16, None, None, A16,
                                              wsb, None)

    assert call(ex, None) == g.EINVAL
    assert call(ex, sh4(E=2)) == g.EINVAL
    assert call(ex, sh4(H=2560)) == g.EINVAL
    assert call(ex, sh4(S=3700)) == g.EINVAL
    assert call(ex, sh4(fmt=7)) == g.EINVAL
    assert call(ex, g.ExpertsS(2, 1, 2688, 3712, A16, A16, A16, A16, A16, None)) == g.EINVAL  # int4 takes no gscale
    need = L.q4moe_w4a16_decode_shared_q4_ws_bytes(ctypes.byref(r), ctypes.byref(ex), ctypes.byref(sh4()), 1)
    assert need > L.q4moe_w4a16_decode_ws_bytes(ctypes.byref(r), ctypes.byref(ex), 1)
    assert call(ex, sh4(), wsb=need - 1) == g.EWORKSPACE
    t = g.SharedTaps()
    assert L.q4moe_w4a16_decode_shared_q4_taps(ctypes.byref(r), ctypes.byref(ex), ctypes.byref(sh4()), 4,
                                               ctypes.byref(t)) == g.OK
    assert t.xq == 0 and t.sh_hq == 0 and 0 < t.sh_h32 and 0 < t.y32


def test_decode_stack_validation(L):
    r, ex = _router(), _experts()
    rs = (g.RouterS * 2)(r, r)
    es = (g.ExpertsS * 2)(ex, ex)
    xs = (ctypes.c_void_p * 2)(A16, A16)
    ys = (ctypes.c_void_p * 2)(A16, A16)
    need = L.q4moe_w4a16_decode_stack_ws_bytes(ctypes.byref(r), ctypes.byref(ex))
    assert need == L.q4moe_w4a16_decode_ws_bytes(ctypes.byref(r), ctypes.byref(ex), 1)

    def call(rs=rs, es=es, n=2, xs=xs, ys=ys, chain=0, wsb=need):
        cast = lambda a: None if a is None else ctypes.cast(a, ctypes.c_void_p)
        return L.q4moe_w4a16_decode_stack(cast(rs), cast(es), n, cast(xs), cast(ys), chain, None, None, A16, wsb,
                                          None)

    assert call(n=0) == g.EINVAL
    assert call(rs=None) == g.EINVAL
    assert call(ys=None) == g.EINVAL
    assert call(es=(g.ExpertsS * 2)(ex, _experts(I=1856 + 32))) == g.EINVAL  # shapes differ
    assert b"differs" in L.q4moe_last_error()
    assert call(xs=(ctypes.c_void_p * 2)(A16, None)) == g.EINVAL  # x of layer 1 outside a chain
    assert call(xs=(ctypes.c_void_p * 2)(A16, A16 + 2)) == g.EALIGN
    assert call(wsb=need - 16) == g.EWORKSPACE
