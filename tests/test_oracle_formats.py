"""Oracle element formats and weight dequantization, pinned to the OCP
tables (tests/golden), torch's own fp8/bf16 decoders and exhaustive sweeps."""
import math

import numpy as np
import pytest
import torch

import oracle
from q4moe_testutil import (E4M3_TORCH, GOLDEN, OCP_E2M1, bf16_bits_to_f64, dense_int4,
                            dense_nvfp4, e4m3_rne_torch, pack)


def _same(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return bool(np.all((a == b) & (np.signbit(a) == np.signbit(b)) | (np.isnan(a) & np.isnan(b))))


def test_e2m1_matches_ocp_table():
    got = np.array([oracle.e2m1(c) for c in range(16)])
    assert _same(got, OCP_E2M1)


def test_e4m3fn_all_bytes_match_torch():
    got = np.array([oracle.e4m3fn(b) for b in range(256)])
    assert _same(got, E4M3_TORCH)


def test_e4m3fn_landmarks_golden():
    for line in open(f"{GOLDEN}/e4m3_spot.txt"):
        if line.startswith("#") or not line.strip():
            continue
        b, v = line.split()
        got = oracle.e4m3fn(int(b, 16))
        if v == "nan":
            assert math.isnan(got)
        else:
            assert got == float(v) and math.copysign(1, got) == math.copysign(1, float(v)), (b, got)


def test_int4_all_codes_two_complement():
    got = [oracle.int4(c) for c in range(16)]
    ref = [int(np.int8(np.uint8(c << 4).view(np.int8)) >> 4) for c in range(16)]
    assert got == ref == [0, 1, 2, 3, 4, 5, 6, 7, -8, -7, -6, -5, -4, -3, -2, -1]


def test_bf16_all_patterns_match_torch():
    bits = np.arange(65536, dtype=np.uint32)
    got = np.array([oracle.bf16(int(b)) for b in bits[::7]])
    assert _same(got, bf16_bits_to_f64(bits[::7].astype(np.uint16)))


def test_nibble_order_low_first():
    # byte 0x21: element 0 = code 1 (0.5), element 1 = code 2 (1.0)
    codes = np.array([[0x21] * 8], np.uint8)
    scales = np.array([[0x38]], np.uint8)
    d = oracle.dequant(oracle.NVFP4, codes, scales, 1.0)
    assert d[0, 0] == 0.5 and d[0, 1] == 1.0


@pytest.mark.parametrize("g", [1.0, 1.0 / 64, 0.3, 2.0 ** -135, 3.0e38])
def test_dequant_nvfp4_exhaustive(g):
    # row r: scale byte r, 16 columns: codes 0..15
    codes = np.tile(pack(np.arange(16, dtype=np.uint8)), (256, 1))
    scales = np.arange(256, dtype=np.uint8).reshape(256, 1)
    got = oracle.dequant(oracle.NVFP4, codes, scales, g)
    ref = dense_nvfp4(codes, scales, g)
    assert _same(got, ref)


def test_dequant_nvfp4_scale_byte_plus8_doubles():
    codes = np.tile(pack(np.arange(16, dtype=np.uint8)), (256, 1))
    scales = np.arange(256, dtype=np.uint8).reshape(256, 1)
    d = oracle.dequant(oracle.NVFP4, codes, scales, 1.0)
    for b in list(range(0x08, 0x77)) + list(range(0x88, 0xF7)):
        assert _same(d[b + 8], 2.0 * d[b]), hex(b)


def test_dequant_int4_exhaustive():
    # 16 codes against every bf16 scale pattern (64 columns per group)
    sb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    sb = sb[np.isfinite(bf16_bits_to_f64(sb))][::5]
    codes = np.tile(pack(np.tile(np.arange(16, dtype=np.uint8), 4)), (sb.size, 1))
    got = oracle.dequant(oracle.INT4_G64, codes, sb.reshape(-1, 1), 1.0)
    assert _same(got, dense_int4(codes, sb.reshape(-1, 1)))


def test_e4m3fn_rounding_matches_torch():
    vals = [E4M3_TORCH[b] for b in range(0x7F)]
    mids = [(vals[i] + vals[i + 1]) / 2 for i in range(len(vals) - 1)]
    pts = np.array(vals + mids, dtype=np.float32)
    near = np.concatenate([pts, np.nextafter(pts, np.float32(0)), np.nextafter(pts, np.float32(1e9))])
    rng = np.random.default_rng(5)
    rand = np.concatenate([rng.uniform(0, 448, 20000), np.exp(rng.uniform(-14, 6, 20000))]).astype(np.float32)
    allv = np.concatenate([near, rand]).astype(np.float32)
    got = np.array([oracle.e4m3fn_from(v) for v in allv], np.uint8)
    assert np.array_equal(got, e4m3_rne_torch(allv))
    for big in [448.0, 463.9, 464.0, 500.0, 1e30]:
        assert oracle.e4m3fn_from(big) == 0x7E


def test_bf16_from_is_nearest_even():
    rng = np.random.default_rng(3)
    vals = np.concatenate([rng.standard_normal(3000) * 50, np.exp(rng.uniform(-80, 80, 3000)),
                           -np.exp(rng.uniform(-80, 80, 3000))])
    # exact midpoints between neighbouring bf16 values (ties)
    base = bf16_bits_to_f64(np.arange(0x3F00, 0x3F40, dtype=np.uint16))
    vals = np.concatenate([vals, (base[:-1] + base[1:]) / 2])
    for v in vals:
        b = oracle.bf16_from(v)
        nb = np.array([b - 1, b, b + 1], dtype=np.int64) & 0xFFFF
        cand = bf16_bits_to_f64(nb.astype(np.uint16))
        d = np.abs(cand - v)
        assert d[1] <= d[0] and d[1] <= d[2], v
        if d[1] == d[0] or d[1] == d[2]:
            assert b % 2 == 0, v
