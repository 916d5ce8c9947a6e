"""Python binding of the q4moe CPU oracle (liboracle.so, plain C, fp64).

TEST INFRASTRUCTURE ONLY.  The tests, the package smoke check and the
benchmark's CPU-baseline leg are the only callers; the library under test
never imports this module and this module never imports the library.
Definitions and their sources are documented in q4moe_oracle.h.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_LIB = None

NVFP4, INT4_G64 = 1, 2


def build():
    src = os.path.join(_HERE, "q4moe_oracle.c")
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", src,
           "-o", _SO + ".tmp", "-lm"]
    subprocess.check_call(cmd)
    os.replace(_SO + ".tmp", _SO)


class _Bank(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("E", ctypes.c_int32), ("H", ctypes.c_int32),
                ("I", ctypes.c_int32),
                ("up_codes", ctypes.c_void_p), ("up_scales", ctypes.c_void_p),
                ("up_g", ctypes.c_void_p),
                ("down_codes", ctypes.c_void_p), ("down_scales", ctypes.c_void_p),
                ("down_g", ctypes.c_void_p)]


class _Shared(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("S", ctypes.c_int32),
                ("up_codes", ctypes.c_void_p), ("down_codes", ctypes.c_void_p),
                ("up_wscale", ctypes.c_float), ("up_iscale", ctypes.c_float),
                ("down_wscale", ctypes.c_float), ("down_iscale", ctypes.c_float)]


def lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        p, i32, d, f = ctypes.c_void_p, ctypes.c_int32, ctypes.c_double, ctypes.c_float
        u32 = ctypes.c_uint32
        for name in ("q4o_e2m1", "q4o_e4m3fn", "q4o_int4", "q4o_bf16"):
            getattr(L, name).restype = d
            getattr(L, name).argtypes = [u32]
        L.q4o_e4m3fn_from.restype = u32
        L.q4o_e4m3fn_from.argtypes = [f]
        L.q4o_bf16_from.restype = u32
        L.q4o_bf16_from.argtypes = [d]
        L.q4o_threads.restype = i32
        L.q4o_set_threads.argtypes = [i32]
        L.q4o_dequant.argtypes = [i32, i32, i32, p, p, f, p]
        L.q4o_router.argtypes = [i32, i32, i32, i32, p, p, p, p, p, p, p, p]
        L.q4o_moe_w4a16.argtypes = [ctypes.POINTER(_Bank), i32, i32, p, p, p, p, p]
        L.q4o_quant_nvfp4.argtypes = [i32, i32, p, p, p]
        L.q4o_moe_w4a4.argtypes = [ctypes.POINTER(_Bank), i32, i32, p, p, p, p, p, p, p, p, p, p]
        L.q4o_w4a4_down_combine.argtypes = [ctypes.POINTER(_Bank), i32, i32, p, p, p, p, p]
        L.q4o_w4a4_up.argtypes = [ctypes.POINTER(_Bank), i32, i32, p, p, p, p]
        L.q4o_gemv_nvfp4.argtypes = [i32, i32, p, p, f, i32, p, p, p, p]
        L.q4o_fp8_code.restype = u32
        L.q4o_fp8_code.argtypes = [f, f]
        L.q4o_fp8_quant.argtypes = [i32, p, f, p]
        L.q4o_fp8_gemv.argtypes = [i32, i32, p, p, f, f, p]
        L.q4o_shared_fp8.argtypes = [ctypes.POINTER(_Shared), p, p, p, p, p, p]
        L.q4o_quant_weights_nvfp4.argtypes = [i32, i32, p, i32, p, p, p]
        L.q4o_wq_gscale.restype = f
        L.q4o_wq_gscale.argtypes = [ctypes.c_int64, p]
        L.q4o_wq_block.restype = u32
        L.q4o_wq_block.argtypes = [p, f, ctypes.c_int, p]
        L.q4o_wq_codes_excess.restype = d
        L.q4o_wq_codes_excess.argtypes = [p, f, u32, p]
        L.q4o_wq_codes_excess_blocks.argtypes = [ctypes.c_int64, p, f, p, p, p]
        _LIB = L
    return _LIB


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


# --- element formats -------------------------------------------------------

def e2m1(code):
    return lib().q4o_e2m1(int(code))


def e4m3fn(byte):
    return lib().q4o_e4m3fn(int(byte))


def int4(code):
    return lib().q4o_int4(int(code))


def bf16(bits):
    return lib().q4o_bf16(int(bits))


def e4m3fn_from(v):
    return int(lib().q4o_e4m3fn_from(float(v)))


def bf16_from(v):
    return int(lib().q4o_bf16_from(float(v)))


def bf16_round(a):
    """Nearest-even bf16 bit patterns of an fp64 array (oracle outputs chained onward)."""
    a = np.asarray(a, dtype=np.float64)
    return np.array([bf16_from(v) for v in a.ravel()], dtype=np.uint16).reshape(a.shape)


def threads():
    return int(lib().q4o_threads())


def set_threads(n):
    lib().q4o_set_threads(int(n))


# --- matrices ----------------------------------------------------------------

def dequant(fmt, codes, scales, g=1.0):
    """fp32 [rows, cols] values of a quantized matrix (logical layout)."""
    codes = _c(codes, np.uint8)
    rows, cols = codes.shape[0], codes.shape[1] * 2
    scales = _c(scales, np.uint8 if fmt == NVFP4 else np.uint16)
    out = np.empty((rows, cols), np.float32)
    lib().q4o_dequant(fmt, rows, cols, _p(codes), _p(scales), float(g), _p(out))
    return out


class Bank:
    """Expert bank (expert-major numpy arrays, logical layout) for the oracle."""

    def __init__(self, fmt, up_codes, up_scales, down_codes, down_scales, up_g=None, down_g=None):
        self.fmt = fmt
        sdt = np.uint8 if fmt == NVFP4 else np.uint16
        self.up_codes = _c(up_codes, np.uint8)
        self.up_scales = _c(up_scales, sdt)
        self.down_codes = _c(down_codes, np.uint8)
        self.down_scales = _c(down_scales, sdt)
        E, I, H2 = self.up_codes.shape
        self.E, self.I, self.H = E, I, H2 * 2
        self.up_g = _c(np.ones(E) if up_g is None else up_g, np.float32)
        self.down_g = _c(np.ones(E) if down_g is None else down_g, np.float32)
        self.s = _Bank(fmt, E, self.H, I, _p(self.up_codes), _p(self.up_scales), _p(self.up_g),
                       _p(self.down_codes), _p(self.down_scales), _p(self.down_g))

    @classmethod
    def from_dict(cls, fmt, d):
        return cls(fmt, d["up_codes"], d["up_scales"], d["down_codes"], d["down_scales"],
                   d.get("up_gscale"), d.get("down_gscale"))


def router(wg, bias, x, k):
    """Router for bf16 tokens x [T, H]; returns dict of logits, scores, ids, w, gap."""
    wg = _c(wg, np.float32)
    bias = _c(bias, np.float32)
    x = _c(np.atleast_2d(x), np.uint16)
    E, H = wg.shape
    T = x.shape[0]
    out = dict(logits=np.empty((T, E)), scores=np.empty((T, E)),
               ids=np.empty((T, k), np.int32), w=np.empty((T, k)), gap=np.empty(T))
    lib().q4o_router(E, H, T, k, _p(wg), _p(bias), _p(x), _p(out["logits"]), _p(out["scores"]),
                     _p(out["ids"]), _p(out["w"]), _p(out["gap"]))
    return out


def moe_w4a16(bank, x, ids, w):
    """Unrounded y [T, H] and the up outputs u [T, k, I] of the W4A16 decode."""
    x = _c(np.atleast_2d(x), np.uint16)
    ids = _c(ids, np.int32)
    w = _c(w, np.float64)
    T, k = ids.shape
    y = np.empty((T, bank.H))
    u = np.empty((T, k, bank.I))
    lib().q4o_moe_w4a16(ctypes.byref(bank.s), T, k, _p(x), _p(ids), _p(w), _p(u), _p(y))
    return y, u


def quant_nvfp4(v):
    """NVFP4 activation quantizer on fp32 rows: codes [rows, cols/2], scales [rows, cols/16]."""
    v = _c(np.atleast_2d(v), np.float32)
    rows, cols = v.shape
    codes = np.zeros((rows, cols // 2), np.uint8)
    scales = np.zeros((rows, cols // 16), np.uint8)
    lib().q4o_quant_nvfp4(rows, cols, _p(v), _p(codes), _p(scales))
    return codes, scales


def moe_w4a4(bank, x, ids, w):
    x = _c(np.atleast_2d(x), np.uint16)
    ids = _c(ids, np.int32)
    w = _c(w, np.float64)
    T, k = ids.shape
    H, I = bank.H, bank.I
    o = dict(xq_codes=np.zeros((T, H // 2), np.uint8), xq_scales=np.zeros((T, H // 16), np.uint8),
             u=np.empty((T, k, I)), h32=np.empty((T, k, I), np.float32),
             hq_codes=np.zeros((T, k, I // 2), np.uint8), hq_scales=np.zeros((T, k, I // 16), np.uint8),
             y=np.empty((T, H)))
    lib().q4o_moe_w4a4(ctypes.byref(bank.s), T, k, _p(x), _p(ids), _p(w), _p(o["xq_codes"]),
                       _p(o["xq_scales"]), _p(o["u"]), _p(o["h32"]), _p(o["hq_codes"]),
                       _p(o["hq_scales"]), _p(o["y"]))
    return o


def w4a4_down_combine(bank, ids, w, hq_codes, hq_scales):
    ids = _c(ids, np.int32)
    w = _c(w, np.float64)
    T, k = ids.shape
    hq_codes = _c(hq_codes, np.uint8).reshape(T * k, bank.I // 2)
    hq_scales = _c(hq_scales, np.uint8).reshape(T * k, bank.I // 16)
    y = np.empty((T, bank.H))
    lib().q4o_w4a4_down_combine(ctypes.byref(bank.s), T, k, _p(ids), _p(w), _p(hq_codes),
                                _p(hq_scales), _p(y))
    return y


def w4a4_up(bank, ids, xq_codes, xq_scales):
    ids = _c(ids, np.int32)
    T, k = ids.shape
    xq_codes = _c(xq_codes, np.uint8)
    xq_scales = _c(xq_scales, np.uint8)
    u = np.empty((T, k, bank.I))
    lib().q4o_w4a4_up(ctypes.byref(bank.s), T, k, _p(ids), _p(xq_codes), _p(xq_scales), _p(u))
    return u


def gemv_nvfp4(codes, scales, g, x):
    """fp64 logits [T, rows], argmax [T] (lowest index among maxima), gap [T]."""
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    x = _c(np.atleast_2d(x), np.uint16)
    rows, cols = codes.shape[0], codes.shape[1] * 2
    T = x.shape[0]
    logits = np.empty((T, rows))
    am = np.empty(T, np.int32)
    gap = np.empty(T)
    lib().q4o_gemv_nvfp4(rows, cols, _p(codes), _p(scales), float(g), T, _p(x), _p(logits),
                         _p(am), _p(gap))
    return logits, am, gap


# --- shared expert, FP8 per-tensor W8A8 ------------------------------------

def fp8_code(v, s):
    """E4M3FN code of fl32(v / s): nearest-even, saturating at 448."""
    return lib().q4o_fp8_code(float(v), float(s))


def fp8_quant(v, s):
    v = _c(v, np.float32).reshape(-1)
    out = np.zeros(v.size, np.uint8)
    lib().q4o_fp8_quant(v.size, _p(v), float(s), _p(out))
    return out


def fp8_gemv(w, a, s_w, s_in):
    """(sum_c e4m3(w[r, c]) e4m3(a[c])) * s_w * s_in for codes w [rows, cols], a [cols]."""
    w = _c(w, np.uint8)
    a = _c(a, np.uint8).reshape(-1)
    rows, cols = w.shape
    assert a.size == cols
    out = np.zeros(rows, np.float64)
    lib().q4o_fp8_gemv(rows, cols, _p(w), _p(a), float(s_w), float(s_in), _p(out))
    return out


def shared_fp8(sh, x):
    """One token through the shared expert.  sh: dict with up_codes [S, H],
    down_codes [H, S] (uint8 E4M3FN) and the four fp32 scales; x: bf16 bits
    [H].  Returns dict xq, u, h32, hq, z."""
    up = _c(sh["up_codes"], np.uint8)
    dn = _c(sh["down_codes"], np.uint8)
    S, H = up.shape
    assert dn.shape == (H, S)
    x = _c(x, np.uint16).reshape(-1)
    assert x.size == H
    d = _Shared(H, S, _p(up).value, _p(dn).value, float(sh["up_wscale"]), float(sh["up_iscale"]),
                float(sh["down_wscale"]), float(sh["down_iscale"]))
    xq = np.zeros(H, np.uint8)
    u = np.zeros(S, np.float64)
    h32 = np.zeros(S, np.float32)
    hq = np.zeros(S, np.uint8)
    z = np.zeros(H, np.float64)
    lib().q4o_shared_fp8(ctypes.byref(d), _p(x), _p(xq), _p(u), _p(h32), _p(hq), _p(z))
    return {"xq": xq, "u": u, "h32": h32, "hq": hq, "z": z}


# --- NVFP4 weight quantizer --------------------------------------------------

def quant_weights_nvfp4(w_bits, mse=False):
    """bf16 bits [rows, cols] -> (codes [rows, cols/2], scales [rows, cols/16], g)."""
    w = _c(np.atleast_2d(w_bits), np.uint16)
    rows, cols = w.shape
    codes = np.zeros((rows, cols // 2), np.uint8)
    scales = np.zeros((rows, cols // 16), np.uint8)
    g = np.zeros(1, np.float32)
    lib().q4o_quant_weights_nvfp4(rows, cols, _p(w), int(bool(mse)), _p(codes), _p(scales), _p(g))
    return codes, scales, np.float32(g[0])


def wq_block(w16_bits, g, mse=False):
    """One block of 16: (scale byte, 8 code bytes)."""
    w = _c(w16_bits, np.uint16).reshape(16)
    c = np.zeros(8, np.uint8)
    b = lib().q4o_wq_block(_p(w), float(g), int(bool(mse)), _p(c))
    return b, c


def wq_codes_excess(w_bits, g, scales):
    """For bf16 weights [rows, cols] and given block scale bytes [rows, cols/16]:
    the codes those bytes give (the quantizer's code rule), and per block how
    much the exact squared error exceeds the block's exact MSE minimum."""
    w = _c(np.atleast_2d(w_bits), np.uint16)
    rows, cols = w.shape
    sc = _c(scales, np.uint8).reshape(-1)
    assert sc.size == rows * cols // 16
    codes = np.zeros(rows * cols // 2, np.uint8)
    excess = np.zeros(sc.size)
    lib().q4o_wq_codes_excess_blocks(sc.size, _p(w), float(g), _p(sc), _p(codes), _p(excess))
    return codes.reshape(rows, cols // 2), excess.reshape(rows, cols // 16)
