"""Seeded synthetic inputs for the routed-MoE decode workloads.

This module is shared by the oracle-side and the GPU-side tests and by the
benchmark.  It holds no step of the quantized-MoE computation: it only turns
counter-based SplitMix64 draws (see synth.c) into the stored input tensors,
with the shapes and value distributions of the workloads:

* activations x: bf16, N(0, 1), one independent stream per token row and per
  regeneration attempt;
* router: fp32 W_g ~ N(0, sigma_g^2) and fp32 bias ~ U(-0.01, 0.01);
* NVFP4 matrices: uniform random nibble codes (all 16, including -0) and
  E4M3FN block scales uniform over the seven powers of two 2^-4 .. 2^2;
* int4 group-64 matrices: uniform nibble codes (two's complement -8..7) and
  bf16 group scales |N(0, 0.01^2)| + 1e-3;
* FP8 shared expert: E4M3FN weight bytes uniform over FP8_WEIGHT_BYTES and
  fixed power-of-two per-tensor scales (FP8_SHARED_SCALES); the FP8 lm_head
  of the drafter the same way (FP8_LM_SCALES).

Expert weights are the logical row-major layout: element (r, 2j) is the low
nibble of byte r*cols/2 + j, scale (r, b) is entry r*(cols/block) + b.
"""
import ctypes
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "libsynth.so")
_LIB = None

# Stream identifiers (the third element of a key tuple).
S_X, S_WG, S_BIAS, S_UP_CODES, S_UP_SCALES, S_DN_CODES, S_DN_SCALES, S_LM_CODES, S_LM_SCALES = range(1, 10)
S_SH_UP, S_SH_DN = 10, 11
S_LM_FP8 = 12
# Workload families (the first element of a key tuple).  One-token and
# four-token NVFP4 decode and the 23-layer NVFP4 stack share a family, so
# layer 0 of the stack is the one-layer workload.
FAM_NVFP4, FAM_INT4, FAM_W4A4 = 0, 1, 2

# E4M3FN bytes of 2^k for k = -4..2 (exponent field k+7, mantissa 0).
NVFP4_SCALE_BYTES = np.array([(k + 7) << 3 for k in range(-4, 3)], dtype=np.uint8)

# Every finite E4M3FN byte (both signs, subnormals, zeros and 448): all but
# the two NaN encodings S.1111.111.  An alternative block-scale table for
# edge-case parity runs.
E4M3_FINITE_BYTES = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], dtype=np.uint8)

# FP8 shared-expert weight bytes: both signs, exponent fields 1..10, every
# mantissa (magnitudes 2^-6 .. 15), so no NaN and no subnormal.
FP8_WEIGHT_BYTES = np.array([(sg << 7) | (e << 3) | m for sg in (0, 1) for e in range(1, 11) for m in range(8)],
                            dtype=np.uint8)
# Per-tensor scales of the synthetic shared expert (the static input scales
# keep x / s and h / s inside the E4M3FN range for these distributions).
FP8_SHARED_SCALES = {"up_wscale": 2.0 ** -8, "up_iscale": 2.0 ** -6,
                     "down_wscale": 2.0 ** -8, "down_iscale": 2.0 ** -5}

NTHREADS = max(1, min(16, os.cpu_count() or 1))
_CHUNK = 1 << 20


def build():
    cmd = ["gcc", "-O2", "-fPIC", "-shared", "-std=c11", os.path.join(_HERE, "synth.c"),
           "-o", _SO + ".tmp", "-lm"]
    subprocess.check_call(cmd)
    os.replace(_SO + ".tmp", _SO)


def lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        u64, p = ctypes.c_uint64, ctypes.c_void_p
        L.synth_key.restype = u64
        L.synth_key.argtypes = [u64] * 6
        L.synth_draw.restype = u64
        L.synth_draw.argtypes = [u64, u64]
        L.synth_bytes.argtypes = [u64, u64, u64, p]
        L.synth_choice_bytes.argtypes = [u64, u64, u64, p, ctypes.c_uint32, p]
        L.synth_bf16_normal.argtypes = [u64, u64, u64, ctypes.c_double, ctypes.c_double, ctypes.c_int, p]
        L.synth_f32_normal.argtypes = [u64, u64, u64, ctypes.c_double, ctypes.c_double, p]
        L.synth_f32_uniform.argtypes = [u64, u64, u64, ctypes.c_double, ctypes.c_double, p]
        L.synth_f64_normal.argtypes = [u64, u64, u64, p]
        _LIB = L
    return _LIB


def key(seed, fam, layer, stream, index=0, attempt=0):
    return lib().synth_key(seed, fam, layer, stream, index, attempt)


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _fill(fn, out, *args, pool=None):
    """Fill the flat array `out` by chunks: fn(key-args..., start, count, ..., ptr)."""
    n = out.size
    item = out.itemsize
    base = out.ctypes.data
    jobs = [(s, min(_CHUNK, n - s)) for s in range(0, n, _CHUNK)]

    def run(job):
        s, c = job
        fn(s, c, ctypes.c_void_p(base + s * item))

    if pool is None or len(jobs) == 1:
        for j in jobs:
            run(j)
    else:
        list(pool.map(run, jobs))
    return out


def _out(out, n, dtype):
    if out is None:
        return np.empty(n, dtype=dtype)
    assert out.dtype == dtype and out.size == n and out.flags.c_contiguous
    return out.reshape(-1)


def bytes_(k, n, pool=None, out=None):
    out = _out(out, n, np.uint8)
    return _fill(lambda s, c, p: lib().synth_bytes(k, s, c, p), out, pool=pool)


def choice_bytes(k, n, table, pool=None, out=None):
    table = np.ascontiguousarray(table, dtype=np.uint8)
    out = _out(out, n, np.uint8)
    return _fill(lambda s, c, p: lib().synth_choice_bytes(k, s, c, _ptr(table), table.size, p), out, pool=pool)


def bf16_normal(k, n, mu=0.0, sigma=1.0, fold=False, pool=None, out=None):
    out = _out(out, n, np.uint16)
    return _fill(lambda s, c, p: lib().synth_bf16_normal(k, s, c, mu, sigma, int(fold), p), out, pool=pool)


def f32_normal(k, n, mu=0.0, sigma=1.0, pool=None, out=None):
    out = _out(out, n, np.float32)
    return _fill(lambda s, c, p: lib().synth_f32_normal(k, s, c, mu, sigma, p), out, pool=pool)


def f32_uniform(k, n, lo, hi, pool=None, out=None):
    out = _out(out, n, np.float32)
    return _fill(lambda s, c, p: lib().synth_f32_uniform(k, s, c, lo, hi, p), out, pool=pool)


def f64_normal(k, n):
    out = np.empty(n, dtype=np.float64)
    lib().synth_f64_normal(k, 0, n, _ptr(out))
    return out


# ---------------------------------------------------------------------------
# Workload tensors
# ---------------------------------------------------------------------------

def x_rows(seed, fam, layer, H, attempts):
    """bf16 bits [T, H]; row t is stream (fam, layer, X, t, attempts[t])."""
    rows = [bf16_normal(key(seed, fam, layer, S_X, t, a), H) for t, a in enumerate(attempts)]
    return np.stack(rows).reshape(len(attempts), H)


def router(seed, fam, layer, E, H, sigma_g=0.02):
    """fp32 W_g [E, H] ~ N(0, sigma_g^2) and fp32 bias [E] ~ U(-0.01, 0.01)."""
    wg = f32_normal(key(seed, fam, layer, S_WG), E * H, 0.0, sigma_g).reshape(E, H)
    b = f32_uniform(key(seed, fam, layer, S_BIAS), E, -0.01, 0.01)
    return wg, b


def nvfp4_matrix(seed, fam, layer, s_codes, s_scales, index, rows, cols, pool=None,
                 out_codes=None, out_scales=None, scale_bytes=NVFP4_SCALE_BYTES):
    codes = bytes_(key(seed, fam, layer, s_codes, index), rows * cols // 2, pool, out_codes)
    scales = choice_bytes(key(seed, fam, layer, s_scales, index), rows * cols // 16,
                          scale_bytes, pool, out_scales)
    return codes.reshape(rows, cols // 2), scales.reshape(rows, cols // 16)


def int4_matrix(seed, fam, layer, s_codes, s_scales, index, rows, cols, pool=None,
                out_codes=None, out_scales=None):
    codes = bytes_(key(seed, fam, layer, s_codes, index), rows * cols // 2, pool, out_codes)
    scales = bf16_normal(key(seed, fam, layer, s_scales, index), rows * cols // 64,
                         1e-3, 0.01, True, pool, out_scales)
    return codes.reshape(rows, cols // 2), scales.reshape(rows, cols // 64)


def bank_arrays(E, H, I, fmt, alloc=np.zeros):
    """Empty expert-bank arrays (expert-major, logical layout)."""
    sdt = np.uint8 if fmt == "nvfp4" else np.uint16
    blk = 16 if fmt == "nvfp4" else 64
    return {
        "up_codes": alloc((E, I, H // 2), np.uint8),
        "up_scales": alloc((E, I, H // blk), sdt),
        "down_codes": alloc((E, H, I // 2), np.uint8),
        "down_scales": alloc((E, H, I // blk), sdt),
        "up_gscale": np.zeros(E, np.float32),
        "down_gscale": np.zeros(E, np.float32),
    }


def expert_bank(seed, fam, layer, E, H, I, fmt, experts=None, gscale=1.0 / 64, out=None,
                scale_bytes=NVFP4_SCALE_BYTES):
    """Expert bank as a dict of expert-major numpy arrays.

    fmt: "nvfp4" or "int4".  `experts` restricts generation to a subset of
    expert indices (the other entries are left as they are), which lets a
    consumer regenerate only the experts a token selected.  `out` reuses the
    arrays of an earlier bank of the same shape.  NVFP4 per-tensor scales are
    `gscale`, block scales drawn uniformly from `scale_bytes`; int4 tensors
    carry none (stored as 1.0).
    """
    if fmt == "nvfp4":
        def mat(*a):
            return nvfp4_matrix(*a, scale_bytes=scale_bytes)
    else:
        mat = int4_matrix
    bank = bank_arrays(E, H, I, fmt) if out is None else out
    bank["up_gscale"][:] = gscale if fmt == "nvfp4" else 1.0
    bank["down_gscale"][:] = gscale if fmt == "nvfp4" else 1.0
    ids = range(E) if experts is None else sorted(set(int(e) for e in experts))

    def one(e):
        mat(seed, fam, layer, S_UP_CODES, S_UP_SCALES, e, I, H, None,
            bank["up_codes"][e], bank["up_scales"][e])
        mat(seed, fam, layer, S_DN_CODES, S_DN_SCALES, e, H, I, None,
            bank["down_codes"][e], bank["down_scales"][e])

    with ThreadPoolExecutor(NTHREADS) as pool:
        list(pool.map(one, ids))
    return bank


def lm_head(seed, fam, layer, V, H, gscale=1.0 / 64, scale_bytes=NVFP4_SCALE_BYTES):
    """NVFP4 lm_head [V, H]: codes, scales, per-tensor fp32 scale."""
    with ThreadPoolExecutor(NTHREADS) as pool:
        codes, scales = nvfp4_matrix(seed, fam, layer, S_LM_CODES, S_LM_SCALES, 0, V, H, pool,
                                     scale_bytes=scale_bytes)
    return codes, scales, np.float32(gscale)


# Per-tensor scales of the synthetic FP8 lm_head (the input scale keeps
# x / s inside the E4M3FN range for N(0, 1) activations).
FP8_LM_SCALES = {"wscale": 2.0 ** -8, "iscale": 2.0 ** -6}


def lm_head_fp8(seed, fam, layer, V, H):
    """FP8 lm_head [V, H]: E4M3FN codes uniform over FP8_WEIGHT_BYTES and the
    fp32 weight and input scales."""
    with ThreadPoolExecutor(NTHREADS) as pool:
        codes = choice_bytes(key(seed, fam, layer, S_LM_FP8), V * H, FP8_WEIGHT_BYTES, pool)
    return codes.reshape(V, H), np.float32(FP8_LM_SCALES["wscale"]), np.float32(FP8_LM_SCALES["iscale"])


def shared_fp8(seed, fam, layer, H, S):
    """FP8 shared expert: up_codes [S, H], down_codes [H, S] (E4M3FN bytes)
    and its four per-tensor scales, as a dict."""
    with ThreadPoolExecutor(NTHREADS) as pool:
        up = choice_bytes(key(seed, fam, layer, S_SH_UP), S * H, FP8_WEIGHT_BYTES, pool)
        dn = choice_bytes(key(seed, fam, layer, S_SH_DN), H * S, FP8_WEIGHT_BYTES, pool)
    sh = {"up_codes": up.reshape(S, H), "down_codes": dn.reshape(H, S)}
    sh.update({k: np.float32(v) for k, v in FP8_SHARED_SCALES.items()})
    return sh
