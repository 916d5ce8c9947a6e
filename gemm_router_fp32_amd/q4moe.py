"""ctypes binding of libq4moe.so: the entry points of include/q4moe.h under
the same names.  Argument marshalling only: descriptors are filled from
torch tensors (device memory) and the current HIP stream is passed through.
There is no fallback: a missing library raises."""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
SO_PATH = os.path.join(_HERE, "libq4moe.so")

OK, EINVAL, EALIGN, EUNSUPPORTED, EWORKSPACE, EDEVICE = range(6)
NVFP4, INT4_G64 = 1, 2

_i32, _p, _sz = ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t


class QMatS(ctypes.Structure):
    _fields_ = [("fmt", _i32), ("rows", _i32), ("cols", _i32),
                ("codes", _p), ("scales", _p), ("gscale", _p)]


class ExpertsS(ctypes.Structure):
    _fields_ = [("fmt", _i32), ("n_experts", _i32), ("hidden", _i32), ("inter", _i32),
                ("up_codes", _p), ("up_scales", _p), ("up_gscale", _p),
                ("down_codes", _p), ("down_scales", _p), ("down_gscale", _p)]


class RouterS(ctypes.Structure):
    _fields_ = [("w_g", _p), ("bias", _p), ("n_experts", _i32), ("hidden", _i32), ("top_k", _i32)]


class DecodeTaps(ctypes.Structure):
    _fields_ = [("y32", _sz), ("h", _sz)]


class W4A4Taps(ctypes.Structure):
    _fields_ = [("perm", _sz), ("expert_offsets", _sz), ("xq_codes", _sz), ("xq_scales", _sz),
                ("h32", _sz), ("hq_codes", _sz), ("hq_scales", _sz), ("y32", _sz)]


class SharedFp8S(ctypes.Structure):
    _fields_ = [("hidden", _i32), ("inter", _i32), ("up_codes", _p), ("down_codes", _p),
                ("up_wscale", ctypes.c_float), ("up_iscale", ctypes.c_float),
                ("down_wscale", ctypes.c_float), ("down_iscale", ctypes.c_float)]


class Fp8MatS(ctypes.Structure):
    _fields_ = [("rows", _i32), ("cols", _i32), ("codes", _p), ("wscale", ctypes.c_float),
                ("iscale", ctypes.c_float)]


class SharedTaps(ctypes.Structure):
    _fields_ = [("y32", _sz), ("h", _sz), ("xq", _sz), ("sh_h32", _sz), ("sh_hq", _sz)]


class W4A4TokenTaps(ctypes.Structure):
    _fields_ = [("y32", _sz), ("h32", _sz), ("xq_codes", _sz), ("xq_scales", _sz), ("hq_codes", _sz),
                ("hq_scales", _sz)]


class W4A4SharedTaps(ctypes.Structure):
    _fields_ = [("y32", _sz), ("h32", _sz), ("xq_codes", _sz), ("xq_scales", _sz), ("hq_codes", _sz),
                ("hq_scales", _sz), ("sh_xq", _sz), ("sh_h32", _sz), ("sh_hq", _sz)]


class Q4moeError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{msg} (status {status})")
        self.status = status


_LIB = None

# name -> (restype, argtypes)
_SIGS = {
    "q4moe_router_topk_ws_bytes": (_sz, [_p, _i32]),
    "q4moe_router_topk": (_i32, [_p, _p, _i32, _p, _p, _p, _p, _sz, _p]),
    "q4moe_dequant_ref": (_i32, [_p, _p, _p]),
    "q4moe_w4a16_decode_ws_bytes": (_sz, [_p, _p, _i32]),
    "q4moe_w4a16_decode": (_i32, [_p, _p, _p, _i32, _p, _p, _p, _p, _sz, _p]),
    "q4moe_w4a16_decode_taps": (_i32, [_p, _p, _i32, _p]),
    "q4moe_w4a16_decode_noalloc": (_i32, [_p, _p, _p, _i32, _p, _p, _p, _p]),
    "q4moe_w4a16_decode_stack_ws_bytes": (_sz, [_p, _p]),
    "q4moe_w4a16_decode_stack": (_i32, [_p, _p, _i32, _p, _p, _i32, _p, _p, _p, _sz, _p]),
    "q4moe_w4a16_grouped_ws_bytes": (_sz, [_p, _p, _i32]),
    "q4moe_w4a16_grouped": (_i32, [_p, _p, _p, _i32, _p, _p, _p, _p, _sz, _p]),
    "q4moe_w4a4_decode_ws_bytes": (_sz, [_p, _p, _i32]),
    "q4moe_w4a4_decode": (_i32, [_p, _p, _p, _i32, _p, _p, _p, _p, _sz, _p]),
    "q4moe_w4a4_decode_taps": (_i32, [_p, _p, _i32, _p]),
    "q4moe_w4a4_moe_ws_bytes": (_sz, [_p, _p, _i32]),
    "q4moe_w4a4_moe": (_i32, [_p, _p, _p, _i32, _p, _p, _p, _p, _sz, _p]),
    "q4moe_quantize_weights_ws_bytes": (_sz, [_i32, _i32]),
    "q4moe_quantize_weights": (_i32, [_p, _i32, _i32, _i32, _p, _p, _p, _p, _sz, _p]),
    "q4moe_w4a4_decode_shared_ws_bytes": (_sz, [_p, _p, _p, _i32]),
    "q4moe_w4a4_decode_shared": (_i32, [_p, _p, _p, _p, _i32, _p, _p, _p, _p, _sz, _p]),
    "q4moe_w4a4_decode_shared_taps": (_i32, [_p, _p, _p, _i32, _p]),
    "q4moe_w4a16_decode_shared_ws_bytes": (_sz, [_p, _p, _p, _i32]),
    "q4moe_w4a16_decode_shared": (_i32, [_p, _p, _p, _p, _i32, _p, _p, _p, _p, _sz, _p]),
    "q4moe_w4a16_decode_shared_taps": (_i32, [_p, _p, _p, _i32, _p]),
    "q4moe_w4a16_decode_shared_q4_ws_bytes": (_sz, [_p, _p, _p, _i32]),
    "q4moe_w4a16_decode_shared_q4": (_i32, [_p, _p, _p, _p, _i32, _p, _p, _p, _p, _sz, _p]),
    "q4moe_w4a16_decode_shared_q4_taps": (_i32, [_p, _p, _p, _i32, _p]),
    "q4moe_w4a4_grouped_ws_bytes": (_sz, [_p, _p, _i32]),
    "q4moe_w4a4_grouped": (_i32, [_p, _p, _p, _i32, _p, _p, _p, _p, _sz, _p]),
    "q4moe_w4a4_grouped_taps": (_i32, [_p, _p, _i32, _p]),
    "q4moe_w4a16_gemv_ws_bytes": (_sz, [_p, _i32]),
    "q4moe_w4a16_gemv": (_i32, [_p, _p, _i32, _p, _p, _p, _sz, _p]),
    "q4moe_fp8_gemv_ws_bytes": (_sz, [_p, _i32]),
    "q4moe_fp8_gemv": (_i32, [_p, _p, _i32, _p, _p, _p, _sz, _p]),
    "q4moe_fp8_gemv_taps": (_i32, [_p, _i32, ctypes.POINTER(_sz)]),
    "q4moe_ws_init": (_i32, [_p, _sz, _p]),
    "q4moe_ws_check": (_i32, [_p, _sz, _p, _p]),
    "q4moe_status_str": (ctypes.c_char_p, [_i32]),
    "q4moe_last_error": (ctypes.c_char_p, []),
    "q4moe_abi_version": (_i32, []),
}
EXPORTS = tuple(_SIGS)


def lib():
    """The loaded libq4moe.so; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(SO_PATH):
            raise RuntimeError(f"libq4moe.so not found at {SO_PATH}: build it first "
                               "(python gemm_router_fp32_amd/build.py or __graft_entry__.build())")
        L = ctypes.CDLL(SO_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _LIB = L
    return _LIB


def _check(st):
    if st != OK:
        L = lib()
        raise Q4moeError(st, f"{L.q4moe_status_str(st).decode()}: {L.q4moe_last_error().decode()}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is not None:
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


# --- descriptors (hold references to the tensors they point into) ----------

class Router:
    def __init__(self, w_g, bias, top_k):
        self.w_g, self.bias = w_g, bias
        E, H = w_g.shape
        self.s = RouterS(w_g.data_ptr(), bias.data_ptr(), E, H, top_k)
        self.n_experts, self.hidden, self.top_k = E, H, top_k


class Experts:
    def __init__(self, fmt, up_codes, up_scales, down_codes, down_scales, up_gscale=None, down_gscale=None):
        self.t = (up_codes, up_scales, down_codes, down_scales, up_gscale, down_gscale)
        E, I, H2 = up_codes.shape
        self.fmt, self.n_experts, self.hidden, self.inter = fmt, E, H2 * 2, I
        self.s = ExpertsS(fmt, E, H2 * 2, I, up_codes.data_ptr(), up_scales.data_ptr(),
                          None if up_gscale is None else up_gscale.data_ptr(),
                          down_codes.data_ptr(), down_scales.data_ptr(),
                          None if down_gscale is None else down_gscale.data_ptr())


class SharedFp8:
    """FP8 per-tensor W8A8 shared expert: up_codes [inter, hidden] and
    down_codes [hidden, inter] uint8 E4M3FN tensors, four fp32 scales."""
    def __init__(self, up_codes, down_codes, up_wscale, up_iscale, down_wscale, down_iscale):
        self.t = (up_codes, down_codes)
        I, H = up_codes.shape
        self.hidden, self.inter = H, I
        self.s = SharedFp8S(H, I, up_codes.data_ptr(), down_codes.data_ptr(), float(up_wscale),
                            float(up_iscale), float(down_wscale), float(down_iscale))


class QMat:
    def __init__(self, fmt, codes, scales, gscale=None):
        self.t = (codes, scales, gscale)
        rows, c2 = codes.shape
        self.fmt, self.rows, self.cols = fmt, rows, c2 * 2
        self.s = QMatS(fmt, rows, c2 * 2, codes.data_ptr(), scales.data_ptr(),
                       None if gscale is None else gscale.data_ptr())


class Fp8Mat:
    """FP8 per-tensor W8A8 matrix: codes [rows, cols] uint8 E4M3FN tensor,
    fp32 weight scale and static input scale."""
    def __init__(self, codes, wscale, iscale):
        self.t = (codes,)
        self.rows, self.cols = codes.shape
        self.s = Fp8MatS(self.rows, self.cols, codes.data_ptr(), float(wscale), float(iscale))


def workspace(nbytes, device="cuda"):
    """A zero-filled, 16-byte-aligned workspace tensor of at least nbytes."""
    n = max(16, (int(nbytes) + 15) // 16 * 16)
    return torch.zeros(n, dtype=torch.uint8, device=device)


# --- entry points ----------------------------------------------------------

def q4moe_router_topk_ws_bytes(router, n_tok):
    return lib().q4moe_router_topk_ws_bytes(ctypes.byref(router.s), n_tok)


def q4moe_router_topk(router, x, ids, w, logits=None, ws=None, stream=None):
    n_tok = x.shape[0]
    if ws is None:
        ws = workspace(q4moe_router_topk_ws_bytes(router, n_tok), x.device)
    _check(lib().q4moe_router_topk(ctypes.byref(router.s), _ptr(x), n_tok, _ptr(ids), _ptr(w), _ptr(logits),
                                   _ptr(ws), ws.numel(), _stream(stream)))


def q4moe_dequant_ref(qmat, out, stream=None):
    _check(lib().q4moe_dequant_ref(ctypes.byref(qmat.s), _ptr(out), _stream(stream)))


def q4moe_w4a16_decode_ws_bytes(router, experts, n_tok):
    return lib().q4moe_w4a16_decode_ws_bytes(ctypes.byref(router.s), ctypes.byref(experts.s), n_tok)


def q4moe_w4a16_decode_taps(router, experts, n_tok):
    t = DecodeTaps()
    _check(lib().q4moe_w4a16_decode_taps(ctypes.byref(router.s), ctypes.byref(experts.s), n_tok, ctypes.byref(t)))
    return t


def q4moe_w4a16_decode(router, experts, x, y, ids=None, w=None, ws=None, stream=None):
    n_tok = x.shape[0]
    if ws is None:
        ws = workspace(q4moe_w4a16_decode_ws_bytes(router, experts, n_tok), x.device)
    _check(lib().q4moe_w4a16_decode(ctypes.byref(router.s), ctypes.byref(experts.s), _ptr(x), n_tok, _ptr(y),
                                    _ptr(ids), _ptr(w), _ptr(ws), ws.numel(), _stream(stream)))
    return ws


def q4moe_w4a16_decode_stack_ws_bytes(router, experts):
    return lib().q4moe_w4a16_decode_stack_ws_bytes(ctypes.byref(router.s), ctypes.byref(experts.s))


def _ptr_array(ts):
    arr = (ctypes.c_void_p * len(ts))(*[None if t is None else t.data_ptr() for t in ts])
    return arr, ctypes.cast(arr, ctypes.c_void_p)


def q4moe_w4a16_decode_stack(routers, experts, xs, ys, chain=False, ids=None, w=None, ws=None, stream=None):
    """len(routers) single-token layers in order (x of layer l > 0 is layer l - 1's y when chain)."""
    n = len(routers)
    rs = (RouterS * n)(*[r.s for r in routers])
    es = (ExpertsS * n)(*[e.s for e in experts])
    xa, xp = _ptr_array(xs)
    ya, yp = _ptr_array(ys)
    ia, ip = _ptr_array(ids) if ids is not None else (None, None)
    wa, wp = _ptr_array(w) if w is not None else (None, None)
    if ws is None:
        ws = workspace(q4moe_w4a16_decode_stack_ws_bytes(routers[0], experts[0]), ys[0].device)
    _check(lib().q4moe_w4a16_decode_stack(ctypes.cast(rs, ctypes.c_void_p), ctypes.cast(es, ctypes.c_void_p), n,
                                          xp, yp, 1 if chain else 0, ip, wp, _ptr(ws), ws.numel(),
                                          _stream(stream)))
    return ws


def q4moe_w4a16_grouped_ws_bytes(router, experts, n_tok):
    return lib().q4moe_w4a16_grouped_ws_bytes(ctypes.byref(router.s), ctypes.byref(experts.s), n_tok)


def q4moe_w4a16_grouped(router, experts, x, y, ids=None, w=None, ws=None, stream=None):
    n_tok = x.shape[0]
    if ws is None:
        ws = workspace(q4moe_w4a16_grouped_ws_bytes(router, experts, n_tok), x.device)
    _check(lib().q4moe_w4a16_grouped(ctypes.byref(router.s), ctypes.byref(experts.s), _ptr(x), n_tok, _ptr(y),
                                     _ptr(ids), _ptr(w), _ptr(ws), ws.numel(), _stream(stream)))
    return ws


def q4moe_w4a16_decode_noalloc(router, experts, x, y, ids=None, w=None, stream=None):
    """q4moe_w4a16_decode on the library's static per-GPU scratch (no workspace)."""
    _check(lib().q4moe_w4a16_decode_noalloc(ctypes.byref(router.s), ctypes.byref(experts.s), _ptr(x), x.shape[0],
                                            _ptr(y), _ptr(ids), _ptr(w), _stream(stream)))


def q4moe_w4a4_decode_ws_bytes(router, experts, n_tok):
    return lib().q4moe_w4a4_decode_ws_bytes(ctypes.byref(router.s), ctypes.byref(experts.s), n_tok)


def q4moe_w4a4_decode_taps(router, experts, n_tok):
    t = W4A4TokenTaps()
    _check(lib().q4moe_w4a4_decode_taps(ctypes.byref(router.s), ctypes.byref(experts.s), n_tok, ctypes.byref(t)))
    return t


def q4moe_w4a4_decode(router, experts, x, y, ids=None, w=None, ws=None, stream=None):
    n_tok = x.shape[0]
    if ws is None:
        ws = workspace(q4moe_w4a4_decode_ws_bytes(router, experts, n_tok), x.device)
    _check(lib().q4moe_w4a4_decode(ctypes.byref(router.s), ctypes.byref(experts.s), _ptr(x), n_tok, _ptr(y),
                                   _ptr(ids), _ptr(w), _ptr(ws), ws.numel(), _stream(stream)))
    return ws


def q4moe_w4a4_moe_ws_bytes(router, experts, n_tok):
    return lib().q4moe_w4a4_moe_ws_bytes(ctypes.byref(router.s), ctypes.byref(experts.s), n_tok)


def q4moe_w4a4_moe(router, experts, x, y, ids, w, ws=None, stream=None):
    n_tok = x.shape[0]
    if ws is None:
        ws = workspace(q4moe_w4a4_moe_ws_bytes(router, experts, n_tok), x.device)
    _check(lib().q4moe_w4a4_moe(ctypes.byref(router.s), ctypes.byref(experts.s), _ptr(x), n_tok, _ptr(y), _ptr(ids),
                                _ptr(w), _ptr(ws), ws.numel(), _stream(stream)))
    return ws


WQ_MAX, WQ_MSE = 0, 1


def q4moe_quantize_weights_ws_bytes(rows, cols):
    return lib().q4moe_quantize_weights_ws_bytes(rows, cols)


def q4moe_quantize_weights(w, codes, scales, gscale, mode=WQ_MAX, ws=None, stream=None):
    """w: bf16 bits [rows, cols] (int16 tensor); codes uint8 [rows, cols/2];
    scales uint8 [rows, cols/16]; gscale float32 [1]."""
    rows, cols = w.shape
    if ws is None:
        ws = workspace(q4moe_quantize_weights_ws_bytes(rows, cols), w.device)
    _check(lib().q4moe_quantize_weights(_ptr(w), rows, cols, mode, _ptr(codes), _ptr(scales), _ptr(gscale),
                                        _ptr(ws), ws.numel(), _stream(stream)))
    return ws


def q4moe_w4a4_decode_shared_ws_bytes(router, experts, shared, n_tok):
    return lib().q4moe_w4a4_decode_shared_ws_bytes(ctypes.byref(router.s), ctypes.byref(experts.s),
                                                   ctypes.byref(shared.s), n_tok)


def q4moe_w4a4_decode_shared_taps(router, experts, shared, n_tok):
    t = W4A4SharedTaps()
    _check(lib().q4moe_w4a4_decode_shared_taps(ctypes.byref(router.s), ctypes.byref(experts.s),
                                               ctypes.byref(shared.s), n_tok, ctypes.byref(t)))
    return t


def q4moe_w4a4_decode_shared(router, experts, shared, x, y, ids=None, w=None, ws=None, stream=None):
    n_tok = x.shape[0]
    if ws is None:
        ws = workspace(q4moe_w4a4_decode_shared_ws_bytes(router, experts, shared, n_tok), x.device)
    _check(lib().q4moe_w4a4_decode_shared(ctypes.byref(router.s), ctypes.byref(experts.s), ctypes.byref(shared.s),
                                          _ptr(x), n_tok, _ptr(y), _ptr(ids), _ptr(w), _ptr(ws), ws.numel(),
                                          _stream(stream)))
    return ws


def q4moe_w4a16_decode_shared_ws_bytes(router, experts, shared, n_tok):
    return lib().q4moe_w4a16_decode_shared_ws_bytes(ctypes.byref(router.s), ctypes.byref(experts.s),
                                                    ctypes.byref(shared.s), n_tok)


def q4moe_w4a16_decode_shared_taps(router, experts, shared, n_tok):
    t = SharedTaps()
    _check(lib().q4moe_w4a16_decode_shared_taps(ctypes.byref(router.s), ctypes.byref(experts.s),
                                                ctypes.byref(shared.s), n_tok, ctypes.byref(t)))
    return t


def q4moe_w4a16_decode_shared(router, experts, shared, x, y, ids=None, w=None, ws=None, stream=None):
    n_tok = x.shape[0]
    if ws is None:
        ws = workspace(q4moe_w4a16_decode_shared_ws_bytes(router, experts, shared, n_tok), x.device)
    _check(lib().q4moe_w4a16_decode_shared(ctypes.byref(router.s), ctypes.byref(experts.s), ctypes.byref(shared.s),
                                           _ptr(x), n_tok, _ptr(y), _ptr(ids), _ptr(w), _ptr(ws), ws.numel(),
                                           _stream(stream)))
    return ws


def q4moe_w4a16_decode_shared_q4_ws_bytes(router, experts, shared, n_tok):
    return lib().q4moe_w4a16_decode_shared_q4_ws_bytes(ctypes.byref(router.s), ctypes.byref(experts.s),
                                                       ctypes.byref(shared.s), n_tok)


def q4moe_w4a16_decode_shared_q4_taps(router, experts, shared, n_tok):
    t = SharedTaps()
    _check(lib().q4moe_w4a16_decode_shared_q4_taps(ctypes.byref(router.s), ctypes.byref(experts.s),
                                                   ctypes.byref(shared.s), n_tok, ctypes.byref(t)))
    return t


def q4moe_w4a16_decode_shared_q4(router, experts, shared, x, y, ids=None, w=None, ws=None, stream=None):
    """q4moe_w4a16_decode plus a 4-bit shared expert (an Experts bank of one expert)."""
    n_tok = x.shape[0]
    if ws is None:
        ws = workspace(q4moe_w4a16_decode_shared_q4_ws_bytes(router, experts, shared, n_tok), x.device)
    _check(lib().q4moe_w4a16_decode_shared_q4(ctypes.byref(router.s), ctypes.byref(experts.s),
                                              ctypes.byref(shared.s), _ptr(x), n_tok, _ptr(y), _ptr(ids), _ptr(w),
                                              _ptr(ws), ws.numel(), _stream(stream)))
    return ws


def q4moe_w4a4_grouped_ws_bytes(router, experts, n_tok):
    return lib().q4moe_w4a4_grouped_ws_bytes(ctypes.byref(router.s), ctypes.byref(experts.s), n_tok)


def q4moe_w4a4_grouped_taps(router, experts, n_tok):
    t = W4A4Taps()
    _check(lib().q4moe_w4a4_grouped_taps(ctypes.byref(router.s), ctypes.byref(experts.s), n_tok, ctypes.byref(t)))
    return t


def q4moe_w4a4_grouped(router, experts, x, y, ids, w, ws=None, stream=None):
    n_tok = x.shape[0]
    if ws is None:
        ws = workspace(q4moe_w4a4_grouped_ws_bytes(router, experts, n_tok), x.device)
    _check(lib().q4moe_w4a4_grouped(ctypes.byref(router.s), ctypes.byref(experts.s), _ptr(x), n_tok, _ptr(y),
                                    _ptr(ids), _ptr(w), _ptr(ws), ws.numel(), _stream(stream)))
    return ws


def q4moe_w4a16_gemv_ws_bytes(qmat, n_tok):
    return lib().q4moe_w4a16_gemv_ws_bytes(ctypes.byref(qmat.s), n_tok)


def q4moe_w4a16_gemv(qmat, x, logits, argmax=None, ws=None, stream=None):
    n_tok = x.shape[0]
    if ws is None:
        ws = workspace(q4moe_w4a16_gemv_ws_bytes(qmat, n_tok), x.device)
    _check(lib().q4moe_w4a16_gemv(ctypes.byref(qmat.s), _ptr(x), n_tok, _ptr(logits), _ptr(argmax), _ptr(ws),
                                  ws.numel(), _stream(stream)))
    return ws


def q4moe_fp8_gemv_ws_bytes(mat, n_tok):
    return lib().q4moe_fp8_gemv_ws_bytes(ctypes.byref(mat.s), n_tok)


def q4moe_fp8_gemv_taps(mat, n_tok):
    """Byte offset of the activation codes [n_tok][cols] in the workspace."""
    off = _sz(0)
    _check(lib().q4moe_fp8_gemv_taps(ctypes.byref(mat.s), n_tok, ctypes.byref(off)))
    return off.value


def q4moe_fp8_gemv(mat, x, logits, argmax=None, ws=None, stream=None):
    n_tok = x.shape[0]
    if ws is None:
        ws = workspace(q4moe_fp8_gemv_ws_bytes(mat, n_tok), x.device)
    _check(lib().q4moe_fp8_gemv(ctypes.byref(mat.s), _ptr(x), n_tok, _ptr(logits), _ptr(argmax), _ptr(ws),
                                ws.numel(), _stream(stream)))
    return ws


def q4moe_ws_init(ws, stream=None):
    _check(lib().q4moe_ws_init(_ptr(ws), ws.numel(), _stream(stream)))


def q4moe_ws_check(ws, stream=None):
    flags = ctypes.c_uint32(0)
    _check(lib().q4moe_ws_check(_ptr(ws), ws.numel(), _stream(stream), ctypes.byref(flags)))
    return flags.value


def q4moe_abi_version():
    return lib().q4moe_abi_version()
