"""GPU parity of the W4A4 grouped chunk, stage by stage against the oracle:
routing exact; the NVFP4 quantization of x bit-exact; h = relu(u)^2 within
the fp32 output gate; the quantization of the GPU's h bit-exact; y within
the bf16 output gate of the oracle's down projection and combine fed the
GPU's quantized h.  The end-to-end fp64 chain is reported, not gated (a
single h code flipped at a rounding midpoint moves a row by ~2e-3)."""
import numpy as np
import pytest
import torch

import gemm_router_fp32_amd as g
import oracle
import synth
from gpu_util import DEV, dev, host, upload_bank, upload_router
from inputs import SEED, x_with_clear_routing
from q4moe_testutil import bf16_bits_to_f64, bf16_rne_of_f32, gate_f32, gate_out

pytestmark = pytest.mark.gpu


def _run(router, ex, x_np, K):
    T = x_np.shape[0]
    H, I = ex.hidden, ex.inter
    y = torch.empty((T, H), dtype=torch.int16, device=DEV)
    ids = torch.empty((T, K), dtype=torch.int32, device=DEV)
    w = torch.empty((T, K), dtype=torch.float32, device=DEV)
    ws = g.q4moe_w4a4_grouped(router, ex, dev(x_np), y, ids, w)
    torch.cuda.synchronize()
    tp = g.q4moe_w4a4_grouped_taps(router, ex, T)
    b = host(ws)
    rows = T * K
    E = ex.n_experts

    def view(off, n, dt):
        return b[off: off + n * np.dtype(dt).itemsize].view(dt).copy()

    return dict(y=host(y, np.uint16), ids=host(ids), w=host(w),
                perm=view(tp.perm, rows, np.int32), offsets=view(tp.expert_offsets, E + 1, np.int32),
                xq_codes=view(tp.xq_codes, T * H // 2, np.uint8).reshape(T, H // 2),
                xq_scales=view(tp.xq_scales, T * H // 16, np.uint8).reshape(T, H // 16),
                h32=view(tp.h32, rows * I, np.float32).reshape(rows, I),
                hq_codes=view(tp.hq_codes, rows * I // 2, np.uint8).reshape(rows, I // 2),
                hq_scales=view(tp.hq_scales, rows * I // 16, np.uint8).reshape(rows, I // 16),
                y32=view(tp.y32, T * H, np.float32).reshape(T, H))


def _check(bank, wg, b, x, r, out, K, sample=None):
    T = x.shape[0]
    ob = oracle.Bank.from_dict(oracle.NVFP4, bank)
    # routing
    assert np.array_equal(out["ids"], r["ids"])
    np.testing.assert_allclose(out["w"], r["w"], rtol=1e-5)
    # dispatch: per expert, its pairs in token order
    perm, off = out["perm"], out["offsets"]
    assert off[0] == 0 and off[-1] == T * K and np.all(np.diff(off) >= 0)
    assert np.array_equal(np.sort(perm), np.arange(T * K))
    for e in range(len(off) - 1):
        pairs = perm[off[e]:off[e + 1]]
        assert np.all(r["ids"].reshape(-1)[pairs] == e)
        assert np.all(np.diff(pairs // K) > 0)
    inv = np.empty(T * K, np.int64)
    inv[perm] = np.arange(T * K)
    # x quantization: bit-exact on every token
    xq_c, xq_s = oracle.quant_nvfp4(bf16_bits_to_f64(x).astype(np.float32))
    assert np.array_equal(out["xq_codes"], xq_c) and np.array_equal(out["xq_scales"], xq_s)
    toks = np.arange(T) if sample is None else np.asarray(sample)
    sub_ids = r["ids"][toks]
    # up projection on the sampled tokens
    u = oracle.w4a4_up(ob, sub_ids, xq_c[toks], xq_s[toks])  # [Ts][K][I]
    rows = inv[(toks[:, None] * K + np.arange(K)[None, :])]   # dispatch rows [Ts][K]
    h_gpu = out["h32"][rows]                                   # [Ts][K][I]
    h_ref = np.maximum(u, 0.0) ** 2
    ok, worst_h = gate_f32(h_gpu.reshape(-1, h_gpu.shape[-1]), h_ref.reshape(-1, h_ref.shape[-1]))
    assert ok, f"h gate exceeded ({worst_h:.3f})"
    # quantization of the GPU's h: bit-exact
    hc, hs = oracle.quant_nvfp4(h_gpu.reshape(-1, h_gpu.shape[-1]))
    assert np.array_equal(out["hq_codes"][rows].reshape(hc.shape), hc)
    assert np.array_equal(out["hq_scales"][rows].reshape(hs.shape), hs)
    # down + combine fed the GPU's quantized h
    yhat = oracle.w4a4_down_combine(ob, sub_ids, r["w"][toks], out["hq_codes"][rows], out["hq_scales"][rows])
    ok, worst_y = gate_out(out["y"][toks], yhat)
    assert ok, f"y gate exceeded ({worst_y:.3f})"
    assert np.array_equal(out["y"], bf16_rne_of_f32(out["y32"]))
    return worst_h, worst_y


@pytest.mark.parametrize("T,H,I", [(64, 256, 192), (40, 320, 128)], ids=["h256", "h320"])
def test_w4a4_small_ragged(T, H, I):
    # h320: hidden 320 and inter 128 leave ragged ends everywhere: a last
    # down-GEMM column tile of 64, an up-GEMM chunk of 64 k, router
    # partitions of 2 or 3 blocks of 16, 20 quantizer blocks per row and a
    # combine workgroup with idle lanes
    E, K = 16, 6
    bank = synth.expert_bank(SEED, synth.FAM_W4A4, 0, E, H, I, "nvfp4")
    wg, b = synth.router(SEED, synth.FAM_W4A4, 0, E, H, 0.5 / np.sqrt(H))
    x, r, _ = x_with_clear_routing(SEED, synth.FAM_W4A4, 0, wg, b, T, K)
    out = _run(upload_router(wg, b, K), upload_bank(bank, "nvfp4"), x, K)
    wh, wy = _check(bank, wg, b, x, r, out, K)
    # end-to-end fp64 chain: reported only
    full = oracle.moe_w4a4(oracle.Bank.from_dict(oracle.NVFP4, bank), x, r["ids"], r["w"])
    _, worst_e2e = gate_out(out["y"], full["y"])
    flips = int(np.sum(out["hq_codes"][np.argsort(out["perm"])] != full["hq_codes"].reshape(T * K, -1)))
    print(f"small: h {wh:.3f}, y {wy:.3f}; end-to-end ratio {worst_e2e:.3f}, h code bytes differing {flips}")


@pytest.mark.parametrize("K", [1, 8])
def test_w4a4_top_k_range(K):
    # the smallest and the largest top-k: the dispatch reads every slot of a
    # token's ids with the slot index clamped to K - 1 and masks slots >= K
    T, E, H, I = 48, 16, 256, 192
    bank = synth.expert_bank(SEED, synth.FAM_W4A4, 2, E, H, I, "nvfp4")
    wg, b = synth.router(SEED, synth.FAM_W4A4, 2, E, H, 0.5 / np.sqrt(H))
    x, r, _ = x_with_clear_routing(SEED, synth.FAM_W4A4, 2, wg, b, T, K)
    out = _run(upload_router(wg, b, K), upload_bank(bank, "nvfp4"), x, K)
    wh, wy = _check(bank, wg, b, x, r, out, K)
    print(f"K={K}: h {wh:.3f}, y {wy:.3f}")


def test_w4a4_full_chunk():
    # every one of the 1024 tokens, every stage
    T, E, H, I, K = 1024, 128, 2688, 1856, 6
    bank = synth.expert_bank(SEED, synth.FAM_W4A4, 0, E, H, I, "nvfp4")
    wg, b = synth.router(SEED, synth.FAM_W4A4, 0, E, H, 0.5 / np.sqrt(H))
    x, r, att = x_with_clear_routing(SEED, synth.FAM_W4A4, 0, wg, b, T, K)
    out = _run(upload_router(wg, b, K), upload_bank(bank, "nvfp4"), x, K)
    counts = np.diff(out["offsets"])
    wh, wy = _check(bank, wg, b, x, r, out, K)
    print(f"full: tokens resampled {sum(a > 0 for a in att)}, per-expert counts min {counts.min()} "
          f"max {counts.max()} mean {counts.mean():.1f} std {counts.std():.1f}; h {wh:.3f}, y {wy:.3f}")


@pytest.mark.parametrize("shape", [(16, 2688, 1856), (16, 256, 192)], ids=["full-hidden", "one-chunk"])
def test_w4a4_skewed_routing(shape):
    # every token picks experts 0..5 (bias far above any score): 200 rows per
    # expert, so each GEMM runs M-tiles 64 + 64 + 64 + 8 for those experts
    # (the later M-tiles load their own weight chunks and dispatch rows) and
    # skips the idle ones; full-hidden streams 11 (up) and 8 (down) chunks,
    # one-chunk a single chunk each
    E, H, I = shape
    T, K = 200, 6
    bank = synth.expert_bank(SEED, synth.FAM_W4A4, 7, E, H, I, "nvfp4")
    wg, b = synth.router(SEED, synth.FAM_W4A4, 7, E, H, 0.5 / np.sqrt(H))
    b = b.copy()
    b[:K] += 10.0
    x, r, _ = x_with_clear_routing(SEED, synth.FAM_W4A4, 7, wg, b, T, K)
    assert set(np.unique(r["ids"])) == set(range(K))
    print(f"W4A4 skewed routing T={T} E={E} H={H} I={I}", flush=True)
    out = _run(upload_router(wg, b, K), upload_bank(bank, "nvfp4"), x, K)
    counts = np.diff(out["offsets"])
    assert np.array_equal(counts, np.array([T] * K + [0] * (E - K)))
    wh, wy = _check(bank, wg, b, x, r, out, K)
    print(f"skewed {H}x{I}: h {wh:.3f}, y {wy:.3f}")


@pytest.mark.parametrize("T", [1, 2, 8, 37, 200])
def test_w4a4_mid_batch(T):
    # the token counts between one-token decode and a prefill chunk: few rows
    # per expert, most experts idle or with one row (full shapes)
    E, H, I, K = 128, 2688, 1856, 6
    bank = synth.expert_bank(SEED + T, synth.FAM_W4A4, 1, E, H, I, "nvfp4")
    wg, b = synth.router(SEED + T, synth.FAM_W4A4, 1, E, H, 0.5 / np.sqrt(H))
    x, r, _ = x_with_clear_routing(SEED + T, synth.FAM_W4A4, 1, wg, b, T, K)
    out = _run(upload_router(wg, b, K), upload_bank(bank, "nvfp4"), x, K)
    wh, wy = _check(bank, wg, b, x, r, out, K)
    print(f"T={T}: experts used {int((np.diff(out['offsets']) > 0).sum())}; h {wh:.3f}, y {wy:.3f}")
