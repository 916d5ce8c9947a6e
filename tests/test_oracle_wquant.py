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


def _exact_errors(block_bits, g):
    """Exact squared error (a Fraction) of every scale byte 1..126: codes are
    the E2M1 magnitude nearest the exact quotient |w| / eff, ties to the even
    code, saturating at 6, with eff = fl32(e4m3(b) * g).  Plain rational
    arithmetic, independent of how the oracle evaluates its objective."""
    from fractions import Fraction
    mags = [abs(Fraction(float(v))) for v in (block_bits.astype(np.uint32) << 16).view(np.float32)]
    grid = [Fraction(v) for v in E2M1]
    out = [None]
    for b in range(1, 127):
        eff = Fraction(float(np.float32(np.float32(oracle.e4m3fn(b)) * np.float32(g))))
        err = Fraction(0)
        for m in mags:
            if eff == 0:
                q = Fraction(0)
            else:
                t = m / eff
                # nearest grid point; on an exact midpoint the even code (index)
                i = min(range(8), key=lambda j: (abs(t - grid[j]), j % 2))
                q = grid[i] * eff
            err += (m - q) ** 2
        out.append(err)
    return out


def _lowest_argmin(errs):
    best = min(errs[1:])
    return next(b for b in range(1, 127) if errs[b] == best)


def test_mse_matches_exact_brute_force_search():
    w = synth.bf16_normal(synth.key(11, 4, 0, 12), 24 * 16).reshape(24, 16)
    codes, scales, g = oracle.quant_weights_nvfp4(w, mse=True)
    _, smax, _ = oracle.quant_weights_nvfp4(w, mse=False)
    for i in range(24):
        err = _exact_errors(w[i], g)
        assert scales[i, 0] == _lowest_argmin(err), (i, int(scales[i, 0]), _lowest_argmin(err))
        assert err[scales[i, 0]] <= err[smax[i, 0]]


def test_mse_single_value_block_closed_form():
    # a block holding one value v = 6 * e4m3(b0) * g (all others zero) has
    # error 0 exactly at the bytes whose scale puts v on the grid; the lowest
    # such byte is b0 itself (a smaller scale saturates at 6 below v), so
    # the MSE search returns b0, with code 6 for v
    g = np.float32(2.0 ** -10)
    for b0 in (0x09, 0x21, 0x33, 0x4A, 0x66):
        v = 6.0 * oracle.e4m3fn(b0) * float(g)
        blk = np.zeros(16, np.float32)
        blk[5] = v
        bits = _bf16_bits(blk)
        b, c = oracle.wq_block(bits, g, mse=True)
        assert b == b0, (hex(b0), hex(b))
        assert (c[2] >> 4) == 7 and np.all(np.delete(c, 2) == 0) and (c[2] & 15) == 0


def test_mse_planted_equal_errors_take_the_lowest_byte():
    # two values 1 and 2 (times 2^-6) are exact on the grid for several
    # scales with the same zero error; the lowest such byte must win
    g = np.float32(1.0)
    blk = np.zeros(16, np.float32)
    blk[0], blk[1] = 2.0 ** -6, 2.0 ** -5
    b, _ = oracle.wq_block(_bf16_bits(blk), g, mse=True)
    err = _exact_errors(_bf16_bits(blk), g)
    zero = [c for c in range(1, 127) if err[c] == 0]
    assert len(zero) > 1 and b == zero[0]


def test_codes_excess_agrees_with_exact_search():
    from fractions import Fraction
    w = synth.bf16_normal(synth.key(13, 4, 0, 12), 6 * 16).reshape(6, 16)
    _, _, g = oracle.quant_weights_nvfp4(w, mse=True)
    mags = np.abs((w.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    for i in range(6):
        err = _exact_errors(w[i], g)
        best = min(err[1:])
        for b in (1, 0x30, 0x40, 0x55, 0x7E, _lowest_argmin(err)):
            codes, ex = oracle.wq_codes_excess(w[i:i + 1], g, np.array([[b]], np.uint8))
            assert ex[0, 0] == float(err[b] - best)
            # the returned codes are the grid points e2m1 * eff(b) the error
            # was taken at (the quantizer's grid), signs those of w
            eff = Fraction(float(np.float32(np.float32(oracle.e4m3fn(b)) * g)))
            nib = np.empty(16, np.uint8)
            nib[0::2], nib[1::2] = codes[0] & 15, codes[0] >> 4
            q = [Fraction(E2M1[n & 7]) * eff for n in nib]
            assert sum((Fraction(float(m)) - qq) ** 2 for m, qq in zip(mags[i], q)) == err[b]
            wneg = (w[i] >> 15).astype(bool)
            assert np.all(((nib >> 3) == 1) == wneg)
