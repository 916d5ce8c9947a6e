"""Independent references used to pin the oracle (numpy / torch CPU only).

Nothing here shares code with the oracle or with the HIP library: element
values come from the OCP E2M1 table in tests/golden and from torch's own
float8_e4m3fn and bfloat16 decoders; matrix products are numpy's.
"""
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load_e2m1():
    vals = np.zeros(16)
    for line in open(os.path.join(GOLDEN, "e2m1_ocp.txt")):
        if line.startswith("#") or not line.strip():
            continue
        c, v = line.split()
        vals[int(c)] = float(v)
    return vals


OCP_E2M1 = _load_e2m1()
E4M3_TORCH = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def bf16_bits_to_f64(bits):
    b = np.asarray(bits, dtype=np.uint16)
    return torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()


def unpack(codes):
    """uint8 [rows, cols/2] -> uint8 nibbles [rows, cols]; element 2j = low nibble."""
    c = np.asarray(codes, dtype=np.uint8)
    out = np.empty(c.shape[:-1] + (c.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = c & 15
    out[..., 1::2] = c >> 4
    return out


def pack(nib):
    n = np.asarray(nib, dtype=np.uint8)
    return (n[..., 0::2] | (n[..., 1::2] << 4)).astype(np.uint8)


def dense_nvfp4(codes, scales, g=1.0):
    """fp32-valued (held in fp64) dense matrix of an NVFP4 matrix."""
    v = OCP_E2M1[unpack(codes)]
    s = np.repeat(E4M3_TORCH[np.asarray(scales, dtype=np.uint8)], 16, axis=-1)
    return (v * s * np.float64(np.float32(g))).astype(np.float32).astype(np.float64)


def dense_int4(codes, scales):
    n = unpack(codes).astype(np.int8)
    iv = np.where(n >= 8, n.astype(np.int16) - 16, n).astype(np.float64)
    s = np.repeat(bf16_bits_to_f64(scales), 64, axis=-1)
    return (iv * s).astype(np.float32).astype(np.float64)


def e4m3_rne_torch(d):
    """E4M3FN byte nearest (RNE) to fp32 values d >= 0, saturating at 448."""
    d = np.minimum(np.asarray(d, dtype=np.float32), np.float32(448.0))
    return torch.from_numpy(d).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


GRID = OCP_E2M1[:8]


def brute_quant(v):
    """NVFP4 activation quantizer by brute force: nearest grid point by distance."""
    v = np.asarray(v, dtype=np.float32)
    rows, cols = v.shape
    blocks = v.reshape(rows, cols // 16, 16)
    amax = np.abs(blocks).max(axis=-1)
    sb = e4m3_rne_torch(amax / np.float32(6.0))
    s = E4M3_TORCH[sb][..., None]
    # beyond 6*s the nearest grid point is 6*s; clamping at 8*s keeps fp64
    # differences exact for inputs far above the scale
    mag = np.minimum(np.abs(blocks.astype(np.float64)), 8.0 * s)
    dist = np.abs(mag[..., None] - GRID * s[..., None])  # [rows, nb, 16, 8]
    best = np.argmin(dist, axis=-1)
    # ties: argmin picks the lower index; move to the even index when tied
    dmin = np.take_along_axis(dist, best[..., None], -1)[..., 0]
    nxt = np.minimum(best + 1, 7)
    dn = np.take_along_axis(dist, nxt[..., None], -1)[..., 0]
    tie = (nxt != best) & (dn == dmin) & (best % 2 == 1)
    best = np.where(tie, nxt, best)
    best = np.where(s == 0.0, 0, best)
    code = best.astype(np.uint8) | (np.signbit(blocks).astype(np.uint8) << 3)
    return pack(code.reshape(rows, cols)), sb.reshape(rows, cols // 16)


# ---------------------------------------------------------------------------
# Output gate for bf16 results against unrounded fp64 oracle values:
#   |y - yhat| <= ulp_bf16(yhat)/2 + 2e-3 * max(|yhat|, 1e-2 * max|yhat|)
# (one bf16 rounding of the exact value plus 2e-3 relative error with a
# floor at 1 % of the largest output, where relative error is meaningless)
# ---------------------------------------------------------------------------

def half_ulp_bf16(v):
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, np.ldexp(1.0, (e - 8).astype(np.int64)), 2.0 ** -134)


def gate_out(y_bf16_bits, yhat, rel=2e-3):
    """Return (ok, worst ratio of error to the allowed bound)."""
    y = bf16_bits_to_f64(y_bf16_bits).astype(np.float64)
    yhat = np.asarray(yhat, dtype=np.float64)
    floor = 1e-2 * np.abs(yhat).max(axis=-1, keepdims=True)
    bound = half_ulp_bf16(yhat) + rel * np.maximum(np.abs(yhat), floor)
    ratio = np.abs(y - yhat) / bound
    return bool(np.all(ratio <= 1.0)), float(ratio.max())


def gate_f32(y32, yhat, rel=2e-3):
    yhat = np.asarray(yhat, dtype=np.float64)
    floor = 1e-2 * np.abs(yhat).max(axis=-1, keepdims=True)
    ratio = np.abs(np.asarray(y32, np.float64) - yhat) / (rel * np.maximum(np.abs(yhat), floor))
    return bool(np.all(ratio <= 1.0)), float(ratio.max())


def bf16_rne_of_f32(a):
    """Nearest-even bf16 bits of fp32 values (exact: integer arithmetic)."""
    u = np.asarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def unfloored_errors(y_bf16_bits, yhat):
    """Errors the floored gate does not show: the largest relative error
    |y - yhat| / |yhat| over nonzero yhat, the same after taking off half a
    bf16 ulp of yhat (the output rounding), and the normwise error
    ||y - yhat||_2 / ||yhat||_2."""
    y = bf16_bits_to_f64(y_bf16_bits).astype(np.float64)
    yhat = np.asarray(yhat, dtype=np.float64)
    nz = yhat != 0
    err = np.abs(y - yhat)
    rel = float((err[nz] / np.abs(yhat[nz])).max()) if nz.any() else 0.0
    rel_r = float((np.maximum(err - half_ulp_bf16(yhat), 0.0)[nz] / np.abs(yhat[nz])).max()) if nz.any() else 0.0
    norm = float(np.linalg.norm(y - yhat) / max(np.linalg.norm(yhat), 1e-300))
    return rel, rel_r, norm
