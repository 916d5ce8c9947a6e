"""Oracle FP8 per-tensor W8A8 shared expert, pinned outside itself:
hand-worked activation codes (tests/golden/fp8_act_codes.txt), torch's own
float8_e4m3fn conversion and fp64 matmul on inputs that never saturate,
closed forms (a permutation matrix of one weight value) and the sign
symmetry of the E4M3FN encoding."""
import numpy as np
import torch

import oracle
import synth
from q4moe_testutil import GOLDEN


def _cases():
    for line in open(f"{GOLDEN}/fp8_act_codes.txt"):
        if line.startswith("#") or not line.strip():
            continue
        v, s, rest = line.split("|")
        yield np.float32(float(v)), np.float32(float(s)), int(rest.split("#")[0], 16)


def test_fp8_codes_hand_worked():
    n = 0
    for v, s, b in _cases():
        assert oracle.fp8_code(v, s) == b, (v, s, hex(oracle.fp8_code(v, s)), hex(b))
        n += 1
    assert n == 18


def _torch_fp8_bytes(v32):
    """torch's fp32 -> float8_e4m3fn conversion (nearest-even) as bytes."""
    return torch.from_numpy(np.ascontiguousarray(v32, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _torch_fp8_values(codes):
    return torch.from_numpy(np.ascontiguousarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_fp8_quant_matches_torch_below_saturation():
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.standard_normal(200000) * 50.0, rng.standard_normal(20000) * 1e-3]).astype(np.float32)
    s = np.float32(0.37)
    q = (v / s).astype(np.float32)
    keep = np.abs(q) < 440.0  # torch turns values past the range into NaN; the reading saturates
    assert keep.mean() > 0.99
    got = oracle.fp8_quant(v[keep], s)
    assert np.array_equal(got, _torch_fp8_bytes(q[keep]))


def _torch_shared(sh, x_bits):
    """The shared expert through torch's float8 conversion and fp64 matmul."""
    x = (x_bits.astype(np.uint32) << 16).view(np.float32)
    xq = _torch_fp8_bytes((x / sh["up_iscale"]).astype(np.float32))
    u = (_torch_fp8_values(sh["up_codes"]) @ _torch_fp8_values(xq)) * float(sh["up_wscale"]) * float(sh["up_iscale"])
    h32 = (np.maximum(u, 0.0) ** 2).astype(np.float32)
    hq = _torch_fp8_bytes((h32 / sh["down_iscale"]).astype(np.float32))
    z = (_torch_fp8_values(sh["down_codes"]) @ _torch_fp8_values(hq)) * float(sh["down_wscale"]) * float(sh["down_iscale"])
    return xq, u, h32, hq, z


def test_shared_matches_torch_fp8_and_fp64_matmul():
    for (H, S, layer) in [(64, 96, 0), (2688, 3712, 1)]:
        sh = synth.shared_fp8(7, 3, layer, H, S)
        x = synth.x_rows(7, 3, layer, H, [0])[0]
        r = oracle.shared_fp8(sh, x)
        xq, u, h32, hq, z = _torch_shared(sh, x)
        assert np.array_equal(r["xq"], xq)
        # the oracle's sums are exact; numpy's fp64 matmul rounds
        assert np.allclose(r["u"], u, rtol=1e-12, atol=1e-12 * np.abs(u).max())
        assert np.array_equal(r["h32"], h32) or np.abs(r["h32"] - h32).max() <= 2 ** -20 * h32.max()
        hq_o = oracle.fp8_quant(h32, sh["down_iscale"])  # same h32 -> same codes
        assert np.array_equal(hq_o, hq)
        assert np.allclose(oracle.fp8_gemv(sh["down_codes"], hq, sh["down_wscale"], sh["down_iscale"]), z,
                           rtol=1e-12, atol=1e-12 * np.abs(z).max())


def test_shared_permutation_closed_form():
    # up = P * 2 (one weight byte 0x40 = 2.0 per row at column perm[j]);
    # x exactly on the fp8 grid times the input scale, so xq decodes to
    # x / s_in and u_j = 2 * x[perm[j]] * s_w exactly.  down = -1.0 (0xB8)
    # on the transposed pattern gives z[perm[j]] = -e4m3(hq[j]) * s_w' * s_in'.
    H = S = 48
    rng = np.random.default_rng(11)
    perm = rng.permutation(H)
    grid = np.array([0.5, 1.0, 1.5, 2.0, 3.0, -0.75, -1.25, 6.0], np.float32)
    s_in = np.float32(0.25)
    xv = rng.choice(grid, H).astype(np.float32) * s_in
    x_bits = (xv.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((x_bits.astype(np.uint32) << 16).view(np.float32), xv)
    up = np.zeros((S, H), np.uint8)
    up[np.arange(S), perm] = 0x40
    dn = np.zeros((H, S), np.uint8)
    dn[perm, np.arange(S)] = 0xB8
    sh = {"up_codes": up, "down_codes": dn, "up_wscale": np.float32(0.5), "up_iscale": s_in,
          "down_wscale": np.float32(0.125), "down_iscale": np.float32(1.0)}
    r = oracle.shared_fp8(sh, x_bits)
    assert np.array_equal(r["u"], 2.0 * xv[perm].astype(np.float64) * 0.5)
    h = np.maximum(r["u"], 0) ** 2
    assert np.array_equal(r["h32"], h.astype(np.float32))
    z = np.zeros(H)
    z[perm] = -np.array([oracle.e4m3fn(b) for b in r["hq"]]) * 0.125
    assert np.array_equal(r["z"], z)


def test_shared_sign_symmetry():
    # flipping the sign bit of every down weight negates z exactly; of every
    # up weight, swaps relu's support (u -> -u)
    sh = synth.shared_fp8(9, 3, 2, 128, 192)
    x = synth.x_rows(9, 3, 2, 128, [0])[0]
    r = oracle.shared_fp8(sh, x)
    neg = dict(sh, down_codes=sh["down_codes"] ^ 0x80)
    assert np.array_equal(oracle.shared_fp8(neg, x)["z"], -r["z"])
    neg = dict(sh, up_codes=sh["up_codes"] ^ 0x80)
    assert np.array_equal(oracle.shared_fp8(neg, x)["u"], -r["u"])
