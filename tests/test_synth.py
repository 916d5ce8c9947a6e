"""The seeded input generators: determinism, counter-slice consistency and
the value distributions of the workloads."""
import ctypes

import numpy as np

import synth
from q4moe_testutil import bf16_bits_to_f64, unpack


def test_deterministic_and_sliceable():
    k = synth.key(1, 0, 0, synth.S_UP_CODES, 4)
    a = synth.bytes_(k, 1000)
    assert np.array_equal(a, synth.bytes_(k, 1000))
    out = np.empty(37, np.uint8)
    synth.lib().synth_bytes(k, 123, 37, out.ctypes.data_as(ctypes.c_void_p))
    assert np.array_equal(out, a[123:160])
    assert synth.key(1, 0, 0, synth.S_UP_CODES, 4) != synth.key(1, 0, 0, synth.S_UP_CODES, 5)
    assert synth.key(1, 0, 0, synth.S_X, 0, 0) != synth.key(1, 0, 0, synth.S_X, 0, 1)


def test_distributions():
    codes, scales = synth.nvfp4_matrix(2, 0, 0, synth.S_UP_CODES, synth.S_UP_SCALES, 0, 512, 2688)
    counts = np.bincount(unpack(codes).ravel(), minlength=16)
    assert counts.min() > 0.95 * counts.mean() and counts.max() < 1.05 * counts.mean()
    sc = np.bincount(scales.ravel(), minlength=256)
    assert set(np.nonzero(sc)[0]) == {0x18, 0x20, 0x28, 0x30, 0x38, 0x40, 0x48}
    x = bf16_bits_to_f64(synth.x_rows(2, 0, 0, 2688, [0, 0, 0, 0]))
    assert abs(x.mean()) < 0.05 and abs(x.std() - 1) < 0.05
    wg, b = synth.router(2, 0, 0, 128, 2688)
    assert abs(wg.std() - 0.02) < 0.001 and b.min() >= -0.01 and b.max() < 0.01
    _, s4 = synth.int4_matrix(2, 1, 0, synth.S_UP_CODES, synth.S_UP_SCALES, 0, 256, 2688)
    s4 = bf16_bits_to_f64(s4)
    assert s4.min() >= 1e-3 * 0.99 and abs(s4.mean() - (0.01 * np.sqrt(2 / np.pi) + 1e-3)) < 3e-4
