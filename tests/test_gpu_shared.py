"""GPU parity of the FP8 per-tensor W8A8 shared expert, through the C-ABI:
inside the single-token decode launch, and in its own two launches beside
the 2-4-token kernels; stage by stage against the oracle on the same seeded
inputs:

1. routing exact (ids) and gates to 1e-5;
2. x codes bit-exact against the oracle's quantizer of the same x;
3. the h tap (fp32 relu(u)^2) within the fp32 output gate of the oracle's
   up projection fed the GPU's x codes;
4. h codes bit-exact against the oracle's quantizer applied to the GPU's h;
5. y within the output gate of the oracle's routed output plus its shared
   down projection fed the GPU's h codes, and y == RNE(y32) bit for bit.

Stage-wise because a code decision taken on an fp32 value that lies within
rounding of a midpoint may differ between the fp32 kernel and the fp64
oracle; each stage is compared on the same quantized input."""
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
FAM_SH = 3


def upload_shared(sh):
    return g.SharedFp8(dev(sh["up_codes"]), dev(sh["down_codes"]), sh["up_wscale"], sh["up_iscale"],
                       sh["down_wscale"], sh["down_iscale"])


def run_shared(router, experts, shared, x_np, ws=None):
    x = dev(x_np)
    y = torch.empty((1, experts.hidden), dtype=torch.int16, device=DEV)
    ids = torch.empty((1, router.top_k), dtype=torch.int32, device=DEV)
    w = torch.empty((1, router.top_k), dtype=torch.float32, device=DEV)
    ws = g.q4moe_w4a16_decode_shared(router, experts, shared, x, y, ids, w, ws=ws)
    torch.cuda.synchronize()
    t = g.q4moe_w4a16_decode_shared_taps(router, experts, shared, 1)
    wsh = host(ws)
    H, S = experts.hidden, shared.inter
    return dict(y=host(y, np.uint16)[0], ids=host(ids), w=host(w),
                y32=wsh[t.y32: t.y32 + H * 4].view(np.float32).copy(),
                xq=wsh[t.xq: t.xq + H].copy(),
                h32=wsh[t.sh_h32: t.sh_h32 + S * 4].view(np.float32).copy(),
                hq=wsh[t.sh_hq: t.sh_hq + S].copy(), ws=ws)


def check_shared(L, sh, out):
    r = L["route"]
    assert np.array_equal(out["ids"], r["ids"])
    np.testing.assert_allclose(out["w"], r["w"], rtol=1e-5)
    x = L["x"][0]
    xf = bf16_bits_to_f64(x).astype(np.float32)
    assert np.array_equal(out["xq"], oracle.fp8_quant(xf, sh["up_iscale"])), "x codes differ"
    u = oracle.fp8_gemv(sh["up_codes"], out["xq"], sh["up_wscale"], sh["up_iscale"])
    ok, worst_h = gate_f32(out["h32"][None], (np.maximum(u, 0.0) ** 2)[None])
    assert ok, f"h tap gate exceeded: worst {worst_h:.3f}"
    assert np.array_equal(out["hq"], oracle.fp8_quant(out["h32"], sh["down_iscale"])), "h codes differ"
    ob = oracle.Bank.from_dict(oracle.NVFP4, L["bank"])
    yr, _ = oracle.moe_w4a16(ob, L["x"], r["ids"], r["w"])
    z = oracle.fp8_gemv(sh["down_codes"], out["hq"], sh["down_wscale"], sh["down_iscale"])
    yhat = yr[0] + z
    ok, worst = gate_out(out["y"][None], yhat[None])
    assert ok, f"bf16 output gate exceeded: worst {worst:.3f}"
    ok32, worst32 = gate_f32(out["y32"][None], yhat[None])
    assert ok32, f"fp32 output gate exceeded: worst {worst32:.3f}"
    assert np.array_equal(out["y"], bf16_rne_of_f32(out["y32"]))
    # the end-to-end oracle (its own x codes, fp64 u) agrees too
    full = oracle.shared_fp8(sh, x)
    ok_e2e, worst_e2e = gate_out(out["y"][None], (yr[0] + full["z"])[None])
    return worst, worst32, worst_h, ok_e2e, worst_e2e


@pytest.mark.parametrize("E,H,I,S", [(16, 256, 192, 128), (16, 256, 192, 64), (32, 512, 320, 192),
                                     (200, 2688, 256, 4096)])
def test_decode_shared_small(E, H, I, S):
    L = layer(SEED + S, synth.FAM_NVFP4, 0, E, H, I, 1, K, "nvfp4")
    sh = synth.shared_fp8(SEED, FAM_SH, S, H, S)
    out = run_shared(upload_router(L["wg"], L["b"], K), upload_bank(L["bank"], "nvfp4"), upload_shared(sh), L["x"])
    check_shared(L, sh, out)


def test_decode_shared_one_token_without_single_launch():
    # top-8 routing at hidden 2688 needs 8 x 336 down units, more than the
    # 2048 waves of the single launch: one token then takes the shared
    # expert's own launches and the small-batch kernels
    L = layer(SEED + 8, synth.FAM_NVFP4, 0, 16, 2688, 256, 1, 8, "nvfp4")
    sh = synth.shared_fp8(SEED, FAM_SH, 8, 2688, 256)
    out = run_shared(upload_router(L["wg"], L["b"], 8), upload_bank(L["bank"], "nvfp4"), upload_shared(sh), L["x"])
    check_shared(L, sh, out)


@pytest.fixture(scope="module")
def full_layer():
    L = layer(SEED, synth.FAM_NVFP4, 0, 128, 2688, 1856, 1, K, "nvfp4")
    sh = synth.shared_fp8(SEED, FAM_SH, 0, 2688, 3712)
    return L, sh, upload_bank(L["bank"], "nvfp4"), upload_router(L["wg"], L["b"], K), upload_shared(sh)


def test_decode_shared_full_layer(full_layer):
    L, sh, ex, router, shd = full_layer
    out = run_shared(router, ex, shd, L["x"])
    worst, worst32, worst_h, ok_e2e, worst_e2e = check_shared(L, sh, out)
    print(f"shared: worst bf16 ratio {worst:.3f}, fp32 {worst32:.4f}, h tap {worst_h:.5f}; "
          f"end to end {'within' if ok_e2e else 'outside'} the gate ({worst_e2e:.3f})")
    # a second call on the same workspace (next epoch) repeats bit for bit
    again = run_shared(router, ex, shd, L["x"], ws=out["ws"])
    assert np.array_equal(again["y32"].view(np.uint32), out["y32"].view(np.uint32))
    assert g.q4moe_ws_check(out["ws"]) == 0


def test_decode_shared_zero_weights_is_plain_decode(full_layer):
    # all-zero shared weights contribute +0 to every row, so y32 equals the
    # routed-only launch's bit for bit (same slot order, + 0)
    L, sh, ex, router, _ = full_layer
    zero = dict(sh, up_codes=np.zeros_like(sh["up_codes"]), down_codes=np.zeros_like(sh["down_codes"]))
    out = run_shared(router, ex, upload_shared(zero), L["x"])
    x = dev(L["x"])
    y = torch.empty((1, ex.hidden), dtype=torch.int16, device=DEV)
    ws = g.q4moe_w4a16_decode(router, ex, x, y)
    torch.cuda.synchronize()
    t = g.q4moe_w4a16_decode_taps(router, ex, 1)
    y32 = host(ws)[t.y32: t.y32 + ex.hidden * 4].view(np.float32)
    assert np.array_equal(out["y32"].view(np.uint32), y32.view(np.uint32))
    assert np.array_equal(out["y"], host(y, np.uint16)[0])
    assert not out["hq"].any() and not out["h32"].any()


def run_shared_multi(router, experts, shared, x_np):
    T = x_np.shape[0]
    x = dev(x_np)
    y = torch.empty((T, experts.hidden), dtype=torch.int16, device=DEV)
    ids = torch.empty((T, router.top_k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, router.top_k), dtype=torch.float32, device=DEV)
    ws = g.q4moe_w4a16_decode_shared(router, experts, shared, x, y, ids, w)
    torch.cuda.synchronize()
    t = g.q4moe_w4a16_decode_shared_taps(router, experts, shared, T)
    wsh = host(ws)
    H, S = experts.hidden, shared.inter
    return dict(y=host(y, np.uint16), ids=host(ids), w=host(w),
                y32=wsh[t.y32: t.y32 + T * H * 4].view(np.float32).reshape(T, H).copy(),
                xq=wsh[t.xq: t.xq + T * H].reshape(T, H).copy(),
                h32=wsh[t.sh_h32: t.sh_h32 + T * S * 4].view(np.float32).reshape(T, S).copy(),
                hq=wsh[t.sh_hq: t.sh_hq + T * S].reshape(T, S).copy())


def check_shared_multi(L, sh, out):
    r = L["route"]
    assert np.array_equal(out["ids"], r["ids"])
    np.testing.assert_allclose(out["w"], r["w"], rtol=1e-5)
    ob = oracle.Bank.from_dict(oracle.NVFP4 if L.get("fmt", "nvfp4") == "nvfp4" else oracle.INT4_G64, L["bank"])
    yr, _ = oracle.moe_w4a16(ob, L["x"], r["ids"], r["w"])
    worst = 0.0
    for t in range(L["x"].shape[0]):
        xf = bf16_bits_to_f64(L["x"][t]).astype(np.float32)
        assert np.array_equal(out["xq"][t], oracle.fp8_quant(xf, sh["up_iscale"])), f"token {t}: x codes differ"
        u = oracle.fp8_gemv(sh["up_codes"], out["xq"][t], sh["up_wscale"], sh["up_iscale"])
        ok, worst_h = gate_f32(out["h32"][t][None], (np.maximum(u, 0.0) ** 2)[None])
        assert ok, f"token {t}: h tap gate exceeded: worst {worst_h:.3f}"
        assert np.array_equal(out["hq"][t], oracle.fp8_quant(out["h32"][t], sh["down_iscale"])), \
            f"token {t}: h codes differ"
        z = oracle.fp8_gemv(sh["down_codes"], out["hq"][t], sh["down_wscale"], sh["down_iscale"])
        yhat = yr[t] + z
        ok, wt = gate_out(out["y"][t][None], yhat[None])
        assert ok, f"token {t}: bf16 output gate exceeded: worst {wt:.3f}"
        ok32, _ = gate_f32(out["y32"][t][None], yhat[None])
        assert ok32, f"token {t}: fp32 output gate exceeded"
        worst = max(worst, wt)
    assert np.array_equal(out["y"], bf16_rne_of_f32(out["y32"]))
    return worst


@pytest.mark.parametrize("T", [2, 3, 4])
@pytest.mark.parametrize("E,H,I,S", [(16, 256, 192, 128), (32, 512, 320, 192), (64, 1024, 256, 4096),
                                     (16, 256, 192, 64)])
def test_decode_shared_multi_token(T, E, H, I, S):
    L = layer(SEED + 7 * T + S, synth.FAM_NVFP4, 0, E, H, I, T, K, "nvfp4")
    sh = synth.shared_fp8(SEED, FAM_SH, S + T, H, S)
    out = run_shared_multi(upload_router(L["wg"], L["b"], K), upload_bank(L["bank"], "nvfp4"), upload_shared(sh),
                           L["x"])
    check_shared_multi(L, sh, out)


def test_decode_shared_multi_token_max_size():
    # every dimension at the library's limit (4096): the widest small-batch
    # instances and full LDS staging of 4 tokens x 4096 codes in both
    # shared-expert kernels
    L = layer(SEED + 4096, synth.FAM_NVFP4, 0, 16, 4096, 4096, 4, K, "nvfp4")
    sh = synth.shared_fp8(SEED, FAM_SH, 4096, 4096, 4096)
    out = run_shared_multi(upload_router(L["wg"], L["b"], K), upload_bank(L["bank"], "nvfp4"), upload_shared(sh),
                           L["x"])
    check_shared_multi(L, sh, out)


def test_decode_shared_multi_token_full_layer(full_layer):
    L1, sh, ex, router, shd = full_layer
    L = layer(SEED + 1, synth.FAM_NVFP4, 0, 128, 2688, 1856, 4, K, "nvfp4")
    ex4 = upload_bank(L["bank"], "nvfp4")
    out = run_shared_multi(upload_router(L["wg"], L["b"], K), ex4, shd, L["x"])
    worst = check_shared_multi(L, sh, out)
    print(f"shared, 4 tokens: worst bf16 ratio {worst:.3f}")
    # all-zero shared weights: y32 equals the routed-only path's bit for bit
    zero = dict(sh, up_codes=np.zeros_like(sh["up_codes"]), down_codes=np.zeros_like(sh["down_codes"]))
    outz = run_shared_multi(upload_router(L["wg"], L["b"], K), ex4, upload_shared(zero), L["x"])
    y = torch.empty((4, ex4.hidden), dtype=torch.int16, device=DEV)
    ws = g.q4moe_w4a16_decode(upload_router(L["wg"], L["b"], K), ex4, dev(L["x"]), y)
    torch.cuda.synchronize()
    t = g.q4moe_w4a16_decode_taps(upload_router(L["wg"], L["b"], K), ex4, 4)
    y32 = host(ws)[t.y32: t.y32 + 4 * ex4.hidden * 4].view(np.float32).reshape(4, -1)
    assert np.array_equal(outz["y32"].view(np.uint32), y32.view(np.uint32))
