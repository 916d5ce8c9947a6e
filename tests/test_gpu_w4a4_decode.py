"""GPU parity of the single-token W4A4 decode (one launch, x and h quantized
to NVFP4 inside it), through the C-ABI, stage by stage against the oracle
on the same seeded inputs: routing exact; the x codes and scales bit-exact
against the oracle's quantizer of the same x; the h tap within the fp32
output gate of the oracle's up projection fed the GPU's x codes; the h
codes and scales bit-exact against the oracle's quantizer applied to the
GPU's h; y within the bf16 output gate of the oracle's down projection and
combine fed the GPU's h codes, and y == RNE(y32) bit for bit."""
import numpy as np
import pytest
import torch

import gemm_router_fp32_amd as g
import oracle
import synth
from gpu_util import DEV, dev, host, upload_bank, upload_router
from inputs import SEED, layer
from q4moe_testutil import bf16_bits_to_f64, bf16_rne_of_f32, gate_f32, gate_out

pytestmark = pytest.mark.gpu

K = 6


def run_w4a4_decode(router, ex, x_np, ws=None):
    H, I = ex.hidden, ex.inter
    T = x_np.shape[0]
    y = torch.empty((T, H), dtype=torch.int16, device=DEV)
    ids = torch.empty((T, K), dtype=torch.int32, device=DEV)
    w = torch.empty((T, K), dtype=torch.float32, device=DEV)
    ws = g.q4moe_w4a4_decode(router, ex, dev(x_np), y, ids, w, ws=ws)
    torch.cuda.synchronize()
    t = g.q4moe_w4a4_decode_taps(router, ex, T)
    b = host(ws)

    def view(off, n, dt):
        return b[off: off + n * np.dtype(dt).itemsize].view(dt).copy()

    return dict(y=host(y, np.uint16), ids=host(ids), w=host(w), ws=ws,
                y32=view(t.y32, T * H, np.float32).reshape(T, H),
                h32=view(t.h32, T * K * I, np.float32).reshape(T * K, I),
                xq_codes=view(t.xq_codes, T * H // 2, np.uint8).reshape(T, H // 2),
                xq_scales=view(t.xq_scales, T * H // 16, np.uint8).reshape(T, H // 16),
                hq_codes=view(t.hq_codes, T * K * I // 2, np.uint8).reshape(T * K, I // 2),
                hq_scales=view(t.hq_scales, T * K * I // 16, np.uint8).reshape(T * K, I // 16))


def check_w4a4_decode(L, out):
    r = L["route"]
    T = L["x"].shape[0]
    assert np.array_equal(out["ids"], r["ids"])
    np.testing.assert_allclose(out["w"], r["w"], rtol=1e-5)
    ob = oracle.Bank.from_dict(oracle.NVFP4, L["bank"])
    xc, xs = oracle.quant_nvfp4(bf16_bits_to_f64(L["x"]).astype(np.float32))
    assert np.array_equal(out["xq_codes"], xc) and np.array_equal(out["xq_scales"], xs), "x codes differ"
    u = oracle.w4a4_up(ob, r["ids"], out["xq_codes"], out["xq_scales"])  # [T][K][I]
    ok, worst_h = gate_f32(out["h32"], (np.maximum(u, 0.0) ** 2).reshape(T * K, -1))
    assert ok, f"h gate exceeded ({worst_h:.3f})"
    hc, hs = oracle.quant_nvfp4(out["h32"])
    assert np.array_equal(out["hq_codes"], hc) and np.array_equal(out["hq_scales"], hs), "h codes differ"
    yhat = oracle.w4a4_down_combine(ob, r["ids"], r["w"], out["hq_codes"], out["hq_scales"])
    ok, worst = gate_out(out["y"], yhat)
    assert ok, f"bf16 output gate exceeded: worst {worst:.3f}"
    ok32, worst32 = gate_f32(out["y32"], yhat)
    assert ok32, f"fp32 output gate exceeded: worst {worst32:.3f}"
    assert np.array_equal(out["y"], bf16_rne_of_f32(out["y32"]))
    # the end-to-end fp64 chain (its own h codes) is reported, not gated
    e2e = oracle.moe_w4a4(ob, L["x"], r["ids"], r["w"])
    ok_e, worst_e = gate_out(out["y"], e2e["y"])
    flips = int((e2e["hq_codes"].reshape(T * K, -1) != out["hq_codes"]).sum())
    return worst, worst_h, ok_e, worst_e, flips


@pytest.mark.parametrize("E,H,I", [(16, 256, 192), (32, 512, 320), (200, 2688, 256)])
def test_w4a4_decode_small(E, H, I):
    # (200, 2688): four polling waves, so the four others quantize x's 336
    # pieces in two passes
    L = layer(SEED + H, synth.FAM_W4A4, 0, E, H, I, 1, K, "nvfp4")
    out = run_w4a4_decode(upload_router(L["wg"], L["b"], K), upload_bank(L["bank"], "nvfp4"), L["x"])
    check_w4a4_decode(L, out)


def test_w4a4_decode_full_layer():
    L = layer(SEED, synth.FAM_W4A4, 0, 128, 2688, 1856, 1, K, "nvfp4")
    router, ex = upload_router(L["wg"], L["b"], K), upload_bank(L["bank"], "nvfp4")
    out = run_w4a4_decode(router, ex, L["x"])
    worst, worst_h, ok_e, worst_e, flips = check_w4a4_decode(L, out)
    print(f"w4a4 decode: worst bf16 ratio {worst:.3f}, h tap {worst_h:.5f}; end to end "
          f"{'within' if ok_e else 'outside'} the gate ({worst_e:.3f}), {flips} h code bytes differ")
    again = run_w4a4_decode(router, ex, L["x"], ws=out["ws"])
    assert np.array_equal(again["y32"].view(np.uint32), out["y32"].view(np.uint32))
    assert g.q4moe_ws_check(out["ws"]) == 0


def test_w4a4_decode_exact_activations_equal_w4a16():
    # x on the NVFP4 grid of its own block scale quantizes to itself, so the
    # W4A4 up projection sees the W4A16 one's x: h taps agree bit for bit
    L = layer(SEED + 7, synth.FAM_W4A4, 0, 16, 256, 192, 1, K, "nvfp4")
    xc, xs = oracle.quant_nvfp4(bf16_bits_to_f64(L["x"]).astype(np.float32))
    xg = oracle.dequant(oracle.NVFP4, xc, xs, 1.0)  # exact in bf16 (at most 6 significant bits)
    x_bits = (xg.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(bf16_bits_to_f64(x_bits), xg.astype(np.float64))
    router, ex = upload_router(L["wg"], L["b"], K), upload_bank(L["bank"], "nvfp4")
    a4 = run_w4a4_decode(router, ex, x_bits)
    xd = dev(x_bits)
    y = torch.empty((1, 256), dtype=torch.int16, device=DEV)
    ws = g.q4moe_w4a16_decode(router, ex, xd, y)
    torch.cuda.synchronize()
    t = g.q4moe_w4a16_decode_taps(router, ex, 1)
    h16 = host(ws)[t.h: t.h + K * 192 * 4].view(np.float32).reshape(K, 192)
    assert np.array_equal(a4["h32"].view(np.uint32), h16.view(np.uint32))


# --- with the FP8 shared expert (the W4A4 checkpoint's whole MoE block) -------

def run_w4a4_shared(router, ex, sh_dev, x_np):
    H, I, S = ex.hidden, ex.inter, sh_dev.inter
    T = x_np.shape[0]
    y = torch.empty((T, H), dtype=torch.int16, device=DEV)
    ids = torch.empty((T, K), dtype=torch.int32, device=DEV)
    w = torch.empty((T, K), dtype=torch.float32, device=DEV)
    ws = g.q4moe_w4a4_decode_shared(router, ex, sh_dev, dev(x_np), y, ids, w)
    torch.cuda.synchronize()
    t = g.q4moe_w4a4_decode_shared_taps(router, ex, sh_dev, T)
    b = host(ws)

    def view(off, n, dt):
        return b[off: off + n * np.dtype(dt).itemsize].view(dt).copy()

    return dict(y=host(y, np.uint16), ids=host(ids), w=host(w),
                y32=view(t.y32, T * H, np.float32).reshape(T, H),
                h32=view(t.h32, T * K * I, np.float32).reshape(T * K, I),
                xq_codes=view(t.xq_codes, T * H // 2, np.uint8).reshape(T, H // 2),
                xq_scales=view(t.xq_scales, T * H // 16, np.uint8).reshape(T, H // 16),
                hq_codes=view(t.hq_codes, T * K * I // 2, np.uint8).reshape(T * K, I // 2),
                hq_scales=view(t.hq_scales, T * K * I // 16, np.uint8).reshape(T * K, I // 16),
                sh_xq=view(t.sh_xq, T * H, np.uint8).reshape(T, H),
                sh_h32=view(t.sh_h32, T * S, np.float32).reshape(T, S),
                sh_hq=view(t.sh_hq, T * S, np.uint8).reshape(T, S))


@pytest.mark.parametrize("E,H,I,S,T", [(16, 256, 192, 128, 1), (200, 2688, 256, 192, 1), (128, 2688, 1856, 3712, 1),
                                       (16, 256, 192, 128, 3), (128, 2688, 1856, 3712, 4)])
def test_w4a4_decode_with_shared_expert(E, H, I, S, T):
    from test_gpu_shared import upload_shared
    L = layer(SEED + S, synth.FAM_W4A4, 1, E, H, I, T, K, "nvfp4")
    sh = synth.shared_fp8(SEED, synth.FAM_W4A4, S, H, S)
    out = run_w4a4_shared(upload_router(L["wg"], L["b"], K), upload_bank(L["bank"], "nvfp4"), upload_shared(sh),
                          L["x"])
    r = L["route"]
    assert np.array_equal(out["ids"], r["ids"])
    np.testing.assert_allclose(out["w"], r["w"], rtol=1e-5)
    ob = oracle.Bank.from_dict(oracle.NVFP4, L["bank"])
    xf = bf16_bits_to_f64(L["x"]).astype(np.float32)
    # routed stages
    xc, xs = oracle.quant_nvfp4(xf)
    assert np.array_equal(out["xq_codes"], xc) and np.array_equal(out["xq_scales"], xs)
    u = oracle.w4a4_up(ob, r["ids"], out["xq_codes"], out["xq_scales"]).reshape(T * K, I)
    ok, worst_h = gate_f32(out["h32"], np.maximum(u, 0.0) ** 2)
    assert ok, f"h gate exceeded ({worst_h:.3f})"
    hc, hs = oracle.quant_nvfp4(out["h32"])
    assert np.array_equal(out["hq_codes"], hc) and np.array_equal(out["hq_scales"], hs)
    # shared stages, token by token
    yhat = oracle.w4a4_down_combine(ob, r["ids"], r["w"], out["hq_codes"], out["hq_scales"])
    worst_sh = 0.0
    for t in range(T):
        assert np.array_equal(out["sh_xq"][t], oracle.fp8_quant(xf[t], sh["up_iscale"]))
        us = oracle.fp8_gemv(sh["up_codes"], out["sh_xq"][t], sh["up_wscale"], sh["up_iscale"])
        ok, wt = gate_f32(out["sh_h32"][t][None], (np.maximum(us, 0.0) ** 2)[None])
        assert ok, f"shared h gate exceeded ({wt:.3f})"
        worst_sh = max(worst_sh, wt)
        assert np.array_equal(out["sh_hq"][t], oracle.fp8_quant(out["sh_h32"][t], sh["down_iscale"]))
        # output: routed down + combine on the GPU's h codes, plus the shared down
        yhat[t] = yhat[t] + oracle.fp8_gemv(sh["down_codes"], out["sh_hq"][t], sh["down_wscale"], sh["down_iscale"])
    ok, worst = gate_out(out["y"], yhat)
    assert ok, f"bf16 output gate exceeded: worst {worst:.3f}"
    ok32, worst32 = gate_f32(out["y32"], yhat)
    assert ok32, f"fp32 output gate exceeded: worst {worst32:.3f}"
    assert np.array_equal(out["y"], bf16_rne_of_f32(out["y32"]))
    print(f"w4a4 + shared E={E}: worst bf16 ratio {worst:.3f}, h {worst_h:.5f}, shared h {worst_sh:.5f}")


@pytest.mark.parametrize("T", [2, 3, 5, 8])
@pytest.mark.parametrize("E,H,I", [(16, 256, 192), (12, 320, 448)])
def test_w4a4_decode_few_tokens_small(T, E, H, I):
    # 2-8 tokens: the small-batch kernels in their W4A4 form (4- and 8-token
    # instances), stage by stage
    L = layer(SEED + 3 * T + H, synth.FAM_W4A4, 0, E, H, I, T, K, "nvfp4")
    print(f"w4a4 decode T={T} E={E} H={H} I={I}", flush=True)
    out = run_w4a4_decode(upload_router(L["wg"], L["b"], K), upload_bank(L["bank"], "nvfp4"), L["x"])
    check_w4a4_decode(L, out)


@pytest.mark.parametrize("T", [2, 4, 5, 8])
def test_w4a4_decode_few_tokens_full_layer(T):
    L = layer(SEED + T, synth.FAM_W4A4, 0, 128, 2688, 1856, T, K, "nvfp4")
    router, ex = upload_router(L["wg"], L["b"], K), upload_bank(L["bank"], "nvfp4")
    print(f"w4a4 decode full layer T={T}", flush=True)
    out = run_w4a4_decode(router, ex, L["x"])
    worst, worst_h, ok_e, worst_e, flips = check_w4a4_decode(L, out)
    print(f"w4a4 decode T={T}: worst bf16 ratio {worst:.3f}, h tap {worst_h:.5f}; end to end "
          f"{'within' if ok_e else 'outside'} the gate ({worst_e:.3f}), {flips} h code bytes differ")


@pytest.mark.parametrize("T", [3, 7, 8])
def test_w4a4_moe_selects_by_token_count(T):
    # up to 7 tokens: one single-token q4moe_w4a4_decode launch per token;
    # more: the grouped pipeline.  Either way the output is that entry
    # point's, bit for bit.
    H = 2688
    L = layer(SEED + 11, synth.FAM_W4A4, 2, 128, H, 1856, T, K, "nvfp4")
    router, ex = upload_router(L["wg"], L["b"], K), upload_bank(L["bank"], "nvfp4")
    x = dev(L["x"])
    y = torch.empty((T, H), dtype=torch.int16, device=DEV)
    ids = torch.empty((T, K), dtype=torch.int32, device=DEV)
    w = torch.empty((T, K), dtype=torch.float32, device=DEV)
    g.q4moe_w4a4_moe(router, ex, x, y, ids, w)
    torch.cuda.synchronize()
    assert np.array_equal(host(ids), L["route"]["ids"])
    y2 = torch.empty_like(y)
    if T <= 7:
        for t in range(T):
            g.q4moe_w4a4_decode(router, ex, x[t:t + 1], y2[t:t + 1])
    else:
        g.q4moe_w4a4_grouped(router, ex, x, y2, torch.empty_like(ids), torch.empty_like(w))
    torch.cuda.synchronize()
    assert np.array_equal(host(y), host(y2))
