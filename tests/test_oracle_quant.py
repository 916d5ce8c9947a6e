"""Oracle NVFP4 activation quantizer: hand-worked ties (tests/golden),
an exhaustive round trip of all codes x scale bytes, and a brute-force
nearest-point quantizer over every finite bf16 input."""
import numpy as np

import oracle
from q4moe_testutil import GOLDEN, bf16_bits_to_f64, brute_quant, pack, unpack


def _cases():
    for line in open(f"{GOLDEN}/quant_ties.txt"):
        if line.startswith("#") or not line.strip():
            continue
        v, s, c = line.split("|")
        yield (np.array([np.float32(t) for t in v.split()], np.float32),
               int(s, 16), np.array([int(t) for t in c.split()], np.uint8))


def test_quant_hand_worked_cases():
    n = 0
    for v, s, c in _cases():
        codes, scales = oracle.quant_nvfp4(v.reshape(1, 16))
        assert scales[0, 0] == s, (v, scales)
        assert np.array_equal(unpack(codes)[0], c), (v, unpack(codes)[0], c)
        n += 1
    assert n == 7


def test_quant_round_trip_all_codes_and_scales():
    # block b: scale byte b (finite, non-zero), all 16 codes; amax = 6*s so
    # the quantizer re-derives s exactly and every code maps to itself.
    rows = []
    sbytes = [b for b in range(1, 0x7F)]
    for b in sbytes:
        codes = np.tile(pack(np.arange(16, dtype=np.uint8)), (1, 1))
        rows.append(oracle.dequant(oracle.NVFP4, codes, np.array([[b]], np.uint8), 1.0)[0])
    v = np.stack(rows).astype(np.float32)
    codes, scales = oracle.quant_nvfp4(v)
    assert np.array_equal(scales[:, 0], np.array(sbytes, np.uint8))
    assert np.array_equal(unpack(codes), np.tile(np.arange(16, dtype=np.uint8), (len(sbytes), 1)))


def test_quant_matches_brute_force_all_bf16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = bf16_bits_to_f64(bits)
    vals = vals[np.isfinite(vals)].astype(np.float32)
    rng = np.random.default_rng(11)
    rng.shuffle(vals)
    vals = vals[: (vals.size // 16) * 16]
    # blocks of arbitrary bf16 values (wide amax range) ...
    v1 = vals.reshape(-1, 256)
    # ... and blocks with a moderate anchor so small values meet a fixed scale
    anchors = np.float32(6.0) * np.float32(2.0) ** rng.integers(-9, 7, size=vals.size // 16).astype(np.float32)
    small = vals[np.abs(vals) <= 64].astype(np.float32)
    small = small[: (small.size // 15) * 15].reshape(-1, 15)
    m = min(small.shape[0], anchors.size)
    v2 = np.concatenate([anchors[:m, None], small[:m]], axis=1)
    v2 = v2[:, :16].reshape(-1, 16)
    for v in (v1, v2):
        c, s = oracle.quant_nvfp4(v)
        bc, bs = brute_quant(v)
        assert np.array_equal(s, bs)
        assert np.array_equal(c, bc)
