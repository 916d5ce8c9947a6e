"""GPU parity of the FP8 per-tensor W8A8 GEMV + argmax (the MTP drafter's
lm_head) through the C-ABI: the activation codes bit-exact against the
oracle's FP8 quantizer of the same x; logits within the fp32 gate of the
oracle's exact-product fp64 sums on those codes; argmax bit-exact (the
lowest row among equal maxima), with tokens drawn so that fp32 against fp64
cannot swap the top two."""
import numpy as np
import pytest
import torch

import gemm_router_fp32_amd as g
import oracle
import synth
from gpu_util import DEV, dev, host
from inputs import SEED
from q4moe_testutil import bf16_bits_to_f64, gate_f32

pytestmark = pytest.mark.gpu


def _run(codes, ws_, is_, x):
    T = x.shape[0]
    m = g.Fp8Mat(dev(codes), ws_, is_)
    logits = torch.empty((T, codes.shape[0]), dtype=torch.float32, device=DEV)
    am = torch.empty(T, dtype=torch.int32, device=DEV)
    ws = g.q4moe_fp8_gemv(m, dev(x), logits, am)
    torch.cuda.synchronize()
    off = g.q4moe_fp8_gemv_taps(m, T)
    xq = host(ws)[off: off + T * codes.shape[1]].reshape(T, codes.shape[1]).copy()
    return host(logits), host(am), xq


def _oracle(codes, ws_, is_, x):
    xf = bf16_bits_to_f64(x).astype(np.float32)
    xq = np.stack([oracle.fp8_quant(xf[t], is_) for t in range(x.shape[0])])
    lg = np.stack([oracle.fp8_gemv(codes, xq[t], ws_, is_) for t in range(x.shape[0])])
    return xq, lg


def _clear_top(codes, ws_, is_, H, T, seed_layer):
    """x rows whose top-1 logit leads the top-2 by at least 1e-3 of the
    largest magnitude (oracle, fp64)."""
    att = list(range(T))
    for _ in range(64):
        x = synth.x_rows(SEED, 0, seed_layer, H, att)
        _, lg = _oracle(codes, ws_, is_, x)
        srt = np.sort(lg, axis=1)
        bad = [t for t in range(T) if srt[t, -1] - srt[t, -2] < 1e-3 * max(1.0, np.abs(lg[t]).max())]
        if not bad:
            return x
        for t in bad:
            att[t] += T
    raise RuntimeError("no clear top-1")


def _check(codes, ws_, is_, x, am_ref=None):
    lg, am, xq = _run(codes, ws_, is_, x)
    xq_ref, lg_ref = _oracle(codes, ws_, is_, x)
    assert np.array_equal(xq, xq_ref), "activation codes differ"
    ok, worst = gate_f32(lg, lg_ref)
    assert ok, f"logit gate exceeded: {worst:.3f}"
    ref = np.argmax(lg_ref, axis=1) if am_ref is None else am_ref
    assert np.array_equal(am, ref), f"argmax {am.tolist()} != {list(ref)}"
    return worst


@pytest.mark.parametrize("rows,cols", [(1000, 256), (997, 320), (64, 4096)])
@pytest.mark.parametrize("T", [1, 2, 3, 4])
def test_fp8_gemv_small_ragged(rows, cols, T):
    # 997 rows: a last group of 5; 320 columns: five 64-wide pieces of the
    # 16-piece instance; 4096: the widest instance
    codes = synth.lm_head_fp8(SEED, 0, 7, rows, cols)[0]
    ws_, is_ = synth.FP8_LM_SCALES["wscale"], synth.FP8_LM_SCALES["iscale"]
    x = _clear_top(codes, ws_, is_, cols, T, 7)
    print(f"fp8 gemv {rows}x{cols} T={T}", flush=True)
    _check(codes, ws_, is_, x)


def test_fp8_gemv_exact_tie_to_lowest_row():
    rows, cols, T = 1000, 256, 4
    codes = synth.lm_head_fp8(SEED, 0, 8, rows, cols)[0].copy()
    ws_, is_ = synth.FP8_LM_SCALES["wscale"], synth.FP8_LM_SCALES["iscale"]
    x = _clear_top(codes, ws_, is_, cols, T, 8)
    _, lg = _oracle(codes, ws_, is_, x[:1])
    w_ = int(np.argmax(lg[0]))
    # the first token's best row copied to a lower and a higher index: an
    # exact tie, broken towards the lowest row
    for dst in (3, min(w_ + 1, rows - 1)):
        codes[dst] = codes[w_]
    _, lg = _oracle(codes, ws_, is_, x)
    ref = np.argmax(lg, axis=1)
    assert ref[0] == min(3, w_)
    _check(codes, ws_, is_, x, ref)


def test_fp8_gemv_every_weight_byte():
    # every finite E4M3FN byte (both signs, subnormals, 448) as a weight
    finite = np.array([b for b in range(256) if (b & 0x7F) != 0x7F], np.uint8)
    rows, cols = 256, 256
    codes = np.stack([np.roll(finite[np.arange(cols) % finite.size], r) for r in range(rows)]).astype(np.uint8)
    x = synth.x_rows(SEED, 0, 9, cols, [0, 1, 2, 3])
    lg, am, xq = _run(codes, 0.3, 2.0 ** -6, x)
    xq_ref, lg_ref = _oracle(codes, 0.3, 2.0 ** -6, x)
    assert np.array_equal(xq, xq_ref)
    ok, worst = gate_f32(lg, lg_ref)
    assert ok, worst


def test_fp8_lm_head_full_shape():
    V, H, T = 131072, 2688, 4
    codes, ws_, is_ = synth.lm_head_fp8(SEED, 0, 0, V, H)
    x = _clear_top(codes, ws_, is_, H, T, 10)
    print("fp8 lm_head 131072 x 2688, 4 tokens", flush=True)
    worst = _check(codes, ws_, is_, x)
    print(f"fp8 lm_head: worst logit ratio {worst:.4f}")
