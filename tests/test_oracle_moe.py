"""Oracle routed-MoE decode (W4A16), W4A4 chunk and lm_head GEMV, pinned by
a hand-derived tiny layer (tests/golden/tiny_expert.txt), brute-force dense
numpy products, exact special cases and power-of-two metamorphic relations."""
import numpy as np
import pytest

import oracle
import synth
from q4moe_testutil import GOLDEN, bf16_bits_to_f64, brute_quant, dense_int4, dense_nvfp4, pack, unpack

H = I = 16
E = 8


def _tiny_bank():
    """The layer of tiny_expert.txt (codes set element by element)."""
    up = np.zeros((E, I, H), np.uint8)
    dn = np.zeros((E, H, I), np.uint8)
    for r in range(16):
        up[3, r, (r + 1) % 16] = 2   # +1.0
        up[3, r, r] = 9              # -0.5
        dn[3, r, (r + 3) % 16] = 4   # +2.0
        up[5, r, r] = 2              # +1.0
        dn[5, r, 15 - r] = 10        # -1.0
    sc_up = np.full((E, I, H // 16), 0x38, np.uint8)
    sc_dn = np.full((E, H, I // 16), 0x38, np.uint8)
    return oracle.Bank(oracle.NVFP4, pack(up), sc_up, pack(dn), sc_dn, np.ones(E), np.ones(E))


def _tiny_router():
    wg = np.zeros((E, H), np.float32)
    b = np.full(E, -0.01, np.float32)
    b[3], b[5] = 0.01, 0.005
    x = np.array([[oracle.bf16_from((i + 1) / 2) for i in range(16)]], np.uint16)
    return wg, b, x


def _golden_tiny():
    rows = [l.split() for l in open(f"{GOLDEN}/tiny_expert.txt") if l.strip() and not l.startswith("#")]
    return np.array([float(r[1]) for r in rows]), np.array([float(r[2]) for r in rows])


@pytest.mark.parametrize("k", [1, 2])
def test_tiny_layer_hand_derived(k):
    bank = _tiny_bank()
    wg, b, x = _tiny_router()
    r = oracle.router(wg, b, x, k)
    assert list(r["ids"][0]) == [3, 5][:k]
    y3, y5 = _golden_tiny()
    y, u = oracle.moe_w4a16(bank, x, r["ids"], r["w"])
    expect = y3 if k == 1 else 0.5 * y3 + 0.5 * y5
    np.testing.assert_array_equal(y[0], expect)
    np.testing.assert_array_equal(u[0, 0], [(r_ + 3) / 4 for r_ in range(15)] + [-3.5])


def test_all_negative_up_gives_positive_zero():
    bank = _tiny_bank()
    up = unpack(bank.up_codes)
    up[3] = np.where(np.arange(16)[None, :] >= 0, 10, 0)  # every up weight -1.0
    bank = oracle.Bank(oracle.NVFP4, pack(up), bank.up_scales, bank.down_codes, bank.down_scales)
    wg, b, x = _tiny_router()
    y, u = oracle.moe_w4a16(bank, x, np.array([[3]]), np.array([[1.0]]))
    assert np.all(u[0, 0] < 0)
    assert np.all(y == 0.0) and not np.any(np.signbit(y))


def _small_layer(fmt, seed=3, E_=16, H_=256, I_=192, T=3, k=6):
    fam = synth.FAM_NVFP4 if fmt == "nvfp4" else synth.FAM_INT4
    bank = synth.expert_bank(seed, fam, 0, E_, H_, I_, fmt)
    wg, b = synth.router(seed, fam, 0, E_, H_)
    x = synth.x_rows(seed, fam, 0, H_, [0] * T)
    ob = oracle.Bank.from_dict(oracle.NVFP4 if fmt == "nvfp4" else oracle.INT4_G64, bank)
    r = oracle.router(wg, b, x, k)
    return bank, ob, x, r


def _dense(bank, fmt, e, which):
    c, s = bank[f"{which}_codes"][e], bank[f"{which}_scales"][e]
    if fmt == "nvfp4":
        return dense_nvfp4(c, s, bank[f"{which}_gscale"][e])
    return dense_int4(c, s)


@pytest.mark.parametrize("fmt", ["nvfp4", "int4"])
def test_decode_matches_dense_brute_force(fmt):
    bank, ob, x, r = _small_layer(fmt)
    y, u = oracle.moe_w4a16(ob, x, r["ids"], r["w"])
    xf = bf16_bits_to_f64(x)
    for t in range(x.shape[0]):
        yref = np.zeros(bank["down_codes"].shape[2] * 2 if False else y.shape[1])
        for i, e in enumerate(r["ids"][t]):
            ue = _dense(bank, fmt, e, "up") @ xf[t]
            # bf16 x times fp32 weights: every product and partial sum is exact in fp64
            np.testing.assert_array_equal(u[t, i], ue)
            h = np.maximum(ue, 0.0) ** 2
            yref += r["w"][t, i] * (_dense(bank, fmt, e, "down") @ h)
        np.testing.assert_allclose(y[t], yref, rtol=1e-12, atol=1e-12 * np.abs(yref).max())


def test_decode_power_of_two_scalings():
    bank, ob, x, r = _small_layer("nvfp4", T=2)
    y0, _ = oracle.moe_w4a16(ob, x, r["ids"], r["w"])
    b2 = dict(bank)
    b2["up_gscale"] = bank["up_gscale"] * 2
    y1, _ = oracle.moe_w4a16(oracle.Bank.from_dict(oracle.NVFP4, b2), x, r["ids"], r["w"])
    np.testing.assert_array_equal(y1, 4 * y0)
    b3 = dict(bank)
    b3["down_gscale"] = bank["down_gscale"] * 2
    y2, _ = oracle.moe_w4a16(oracle.Bank.from_dict(oracle.NVFP4, b3), x, r["ids"], r["w"])
    np.testing.assert_array_equal(y2, 2 * y0)


def test_w4a4_matches_brute_force():
    bank, ob, x, r = _small_layer("nvfp4", T=4)
    o = oracle.moe_w4a4(ob, x, r["ids"], r["w"])
    xq_c, xq_s = brute_quant(bf16_bits_to_f64(x).astype(np.float32))
    assert np.array_equal(o["xq_codes"], xq_c) and np.array_equal(o["xq_scales"], xq_s)
    xd = dense_nvfp4(xq_c, xq_s, 1.0)
    T, k = r["ids"].shape
    y = np.zeros((T, ob.H))
    for t in range(T):
        for i, e in enumerate(r["ids"][t]):
            u = _dense(bank, "nvfp4", e, "up") @ xd[t]
            np.testing.assert_array_equal(o["u"][t, i], u)
            h32 = (np.maximum(u, 0) ** 2).astype(np.float32)
            np.testing.assert_array_equal(o["h32"][t, i], h32)
            hc, hs = brute_quant(h32[None, :])
            assert np.array_equal(o["hq_codes"][t, i], hc[0]) and np.array_equal(o["hq_scales"][t, i], hs[0])
            y[t] += r["w"][t, i] * (_dense(bank, "nvfp4", e, "down") @ dense_nvfp4(hc, hs, 1.0)[0])
    np.testing.assert_allclose(o["y"], y, rtol=1e-12, atol=1e-12 * np.abs(y).max())
    # the stage-wise entry points reproduce the chained result
    np.testing.assert_array_equal(oracle.w4a4_up(ob, r["ids"], o["xq_codes"], o["xq_scales"]), o["u"])
    np.testing.assert_array_equal(oracle.w4a4_down_combine(ob, r["ids"], r["w"], o["hq_codes"], o["hq_scales"]), o["y"])


def test_w4a4_equals_w4a16_when_quantization_is_exact():
    # Inputs on the E2M1 grid with block amax 6 (x) make Q(x) = x; expert 3 of
    # the tiny layer then gives u in {(r+3)/4} which is not exact, so use an
    # up matrix that maps x to u in {0, 3, 6} (h in {0, 9, 36}, amax 36 per block).
    up = np.zeros((E, I, H), np.uint8)
    dn = np.zeros((E, H, I), np.uint8)
    for r_ in range(16):
        up[2, r_, r_] = 2                    # u_r = x_r
        dn[2, r_, (5 * r_ + 1) % 16] = 11    # -1.5
    sc = np.full((E, 16, 1), 0x38, np.uint8)
    bank = oracle.Bank(oracle.NVFP4, pack(up), sc, pack(dn), sc)
    xv = [6, 3, 0, -1, 6, 3, 3, 0, -6, 0, 6, 3, 0, 0, 3, 6]
    x = np.array([[oracle.bf16_from(v) for v in xv]], np.uint16)
    ids, w = np.array([[2]], np.int32), np.array([[1.0]])
    o = oracle.moe_w4a4(bank, x, ids, w)
    y16, _ = oracle.moe_w4a16(bank, x, ids, w)
    np.testing.assert_array_equal(o["y"], y16)
    assert o["hq_scales"][0, 0, 0] == 0x4C  # 36/6 = 6 = 1.5 * 2^2 -> E4M3 exponent 9, mantissa 4


def test_gemv_brute_force_and_argmax_ties():
    codes, scales = synth.nvfp4_matrix(5, 0, 0, synth.S_LM_CODES, synth.S_LM_SCALES, 0, 300, 256)
    x = synth.x_rows(5, 0, 0, 256, [0, 0, 1, 2])
    x[1] = x[0]
    logits, am, gap = oracle.gemv_nvfp4(codes, scales, 1 / 64, x)
    ref = bf16_bits_to_f64(x) @ dense_nvfp4(codes, scales, 1 / 64).T
    np.testing.assert_array_equal(logits, ref)
    assert list(am) == [int(np.argmax(ref[t])) for t in range(4)]
    # duplicate the winning row below it: the lower index must win
    w = int(am[0])
    c2, s2 = codes.copy(), scales.copy()
    c2[w // 2], s2[w // 2] = codes[w], scales[w]
    c2[w], s2[w] = codes[w], scales[w]
    _, am2, gap2 = oracle.gemv_nvfp4(c2, s2, 1 / 64, x[:1])
    assert am2[0] == min(w, w // 2) and gap2[0] == 0.0
