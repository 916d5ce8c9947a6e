"""Oracle NVFP4 weight quantizer (max-based and MSE per-block scale search),
pinned outside itself: an exact round trip of weights built on the grid,
a brute-force fp64 search over every scale byte, MSE never worse than the
max-based choice, and the E2M1 rounding bound of the dequantized weights."""
import numpy as np

import oracle
import synth

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
MIDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def _e4m3(b):
    return np.array([oracle.e4m3fn(int(x)) for x in np.atleast_1d(b)])


def _bf16_bits(v):
    u = np.asarray(v, np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exact in bf16"
    return (u >> 16).astype(np.uint16)


def _dequant(codes, scales, g):
    return oracle.dequant(oracle.NVFP4, codes, scales, float(g)).astype(np.float64)


def test_round_trip_on_grid_both_modes():
    # weights e2m1 * e4m3(b) * g with a largest code 6 in every block, and
    # one block at scale byte 0x7E so that the tensor's g is reproduced
    rng = np.random.default_rng(3)
    rows, cols, g = 8, 64, 2.0 ** -12
    nb = rows * cols // 16
    bytes_ = rng.integers(0x20, 0x60, nb)
    bytes_[5] = 0x7E
    mags = rng.integers(0, 8, (nb, 16))
    mags[:, rng.integers(0, 16)] = 7
    signs = rng.integers(0, 2, (nb, 16))
    vals = E2M1[mags] * _e4m3(bytes_)[:, None] * g * np.where(signs == 1, -1.0, 1.0)
    w = _bf16_bits(vals.reshape(rows, cols))
    for mse in (False, True):
        codes, scales, gq = oracle.quant_weights_nvfp4(w, mse=mse)
        assert gq == np.float32(g)
        assert np.array_equal(scales.reshape(-1), bytes_.astype(np.uint8))
        np.testing.assert_array_equal(_dequant(codes, scales, gq), vals.reshape(rows, cols))


def _fp64_errors(block, g):
    """fp64 squared error of every scale byte 1..126 (nearest E2M1 of the
    exact quotient, ties to the even code)."""
    mag = np.abs(block)
    out = np.empty(127)
    out[0] = np.inf
    for b in range(1, 127):
        eff = np.float64(np.float32(oracle.e4m3fn(b) * np.float32(g)))
        q = mag / eff
        idx = (q[:, None] > MIDS[None, :]).sum(1)
        tie = np.isin(q, MIDS)
        # a tie at mid j (between codes j and j+1) goes to the even code
        j = np.searchsorted(MIDS, q)
        idx = np.where(tie, np.where(j % 2 == 1, j + 1, j), idx)
        out[b] = np.sum((mag - E2M1[idx] * eff) ** 2)
    return out


def test_mse_matches_brute_force_search():
    w = synth.bf16_normal(synth.key(11, 4, 0, 12), 40 * 16).reshape(40, 16)
    wf = (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    codes, scales, g = oracle.quant_weights_nvfp4(w, mse=True)
    _, smax, _ = oracle.quant_weights_nvfp4(w, mse=False)
    for i in range(40):
        err = _fp64_errors(wf[i], g)
        chosen = err[scales[i, 0]]
        assert chosen <= err.min() * (1 + 1e-5) + 1e-30, (i, scales[i, 0], int(np.argmin(err)))
        assert chosen <= err[smax[i, 0]] * (1 + 1e-5) + 1e-30


def test_mse_never_worse_and_error_bound():
    w = synth.bf16_normal(synth.key(12, 4, 0, 12), 96 * 128).reshape(96, 128)
    wf = (w.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    cm, sm, g = oracle.quant_weights_nvfp4(w, mse=False)
    cs, ss, g2 = oracle.quant_weights_nvfp4(w, mse=True)
    assert g == g2 == np.float32(np.abs(wf).max() / 2688.0)
    em = ((_dequant(cm, sm, g) - wf) ** 2).reshape(-1, 16).sum(1)
    es = ((_dequant(cs, ss, g) - wf) ** 2).reshape(-1, 16).sum(1)
    assert np.all(es <= em * (1 + 1e-5) + 1e-30)
    assert es.sum() < em.sum()
    # max-based: every element within half the widest grid gap (1.0) of
    # eff = fl32(e4m3 * g), up to the dequantization's own fp32 rounding
    eff = np.repeat(_e4m3(sm.reshape(-1)).astype(np.float32) * np.float32(g), 16).reshape(w.shape)
    assert np.all(np.abs(_dequant(cm, sm, g) - wf) <= eff.astype(np.float64) * (1 + 2.0 ** -20))


def test_zero_blocks_and_signs():
    w = np.zeros((2, 32), np.uint16)
    w[1, 16:] = _bf16_bits(np.arange(-8, 8) * 0.375)
    w[0, 3] = 0x8000  # -0
    for mse in (False, True):
        codes, scales, g = oracle.quant_weights_nvfp4(w, mse=mse)
        assert scales[0, 0] == 0 and scales[0, 1] == 0 and scales[1, 0] == 0
        assert (codes[0, 1] >> 4) == 8  # -0 keeps its sign bit
        d = _dequant(codes, scales, g)
        assert np.all(np.sign(d[1, 16:]) * np.sign(np.arange(-8, 8)) >= 0)
