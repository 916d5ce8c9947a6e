"""GPU parity of the shared expert beyond the small-batch and one-launch
forms: the FP8 W8A8 shared expert above 4 tokens and beside int4 routed
experts, and the 4-bit W4A16 shared expert (int4-g64 as the int4
checkpoint stores it, and NVFP4) for any token count; both run through the
grouped GEMMs as a one-expert dispatch of every token, and their output
joins the routed combine before the single rounding.

FP8: stage by stage as in test_gpu_shared (x codes bit-exact, the h tap
within the fp32 gate, h codes bit-exact on the GPU's h, y within the output
gate of the oracle's routed output plus the shared down projection of the
GPU's h codes).  4-bit: the h tap within the fp32 gate of the oracle's
shared up projection, y within the output gate of the oracle's routed plus
shared outputs (no quantization decision in between)."""
import numpy as np
import pytest
import torch

import gemm_router_fp32_amd as g
import oracle
import synth
from gpu_util import DEV, dev, host, upload_bank, upload_router
from inputs import SEED, layer
from q4moe_testutil import bf16_rne_of_f32, gate_f32, gate_out
from test_gpu_shared import FAM_SH, check_shared_multi, run_shared_multi, upload_shared

pytestmark = pytest.mark.gpu

K = 6


@pytest.mark.parametrize("fmt,T", [("nvfp4", 5), ("nvfp4", 8), ("int4", 1), ("int4", 2), ("int4", 5)])
@pytest.mark.parametrize("E,H,I,S", [(16, 256, 192, 128), (12, 320, 448, 192)])
def test_fp8_shared_grouped_small(fmt, T, E, H, I, S):
    fam = synth.FAM_NVFP4 if fmt == "nvfp4" else synth.FAM_INT4
    L = layer(SEED + 5 * T + S + H, fam, 0, E, H, I, T, K, fmt)
    sh = synth.shared_fp8(SEED, FAM_SH, S + T + H, H, S)
    print(f"fp8 shared (grouped) with {fmt} routed: E={E} H={H} I={I} S={S} T={T}", flush=True)
    out = run_shared_multi(upload_router(L["wg"], L["b"], K), upload_bank(L["bank"], fmt), upload_shared(sh), L["x"])
    check_shared_multi(L, sh, out)


@pytest.mark.parametrize("fmt,T", [("nvfp4", 37), ("int4", 8)])
def test_fp8_shared_grouped_full_layer(fmt, T):
    fam = synth.FAM_NVFP4 if fmt == "nvfp4" else synth.FAM_INT4
    L = layer(SEED + T, fam, 0, 128, 2688, 1856, T, K, fmt)
    sh = synth.shared_fp8(SEED, FAM_SH, 0, 2688, 3712)
    print(f"fp8 shared (grouped) full layer, {fmt} routed, T={T}", flush=True)
    out = run_shared_multi(upload_router(L["wg"], L["b"], K), upload_bank(L["bank"], fmt), upload_shared(sh), L["x"])
    worst = check_shared_multi(L, sh, out)
    print(f"fp8 shared full {fmt} T={T}: worst bf16 ratio {worst:.3f}", flush=True)


def _run_q4(router, ex, shx, x_np):
    T = x_np.shape[0]
    y = torch.empty((T, ex.hidden), dtype=torch.int16, device=DEV)
    ids = torch.empty((T, router.top_k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, router.top_k), dtype=torch.float32, device=DEV)
    ws = g.q4moe_w4a16_decode_shared_q4(router, ex, shx, dev(x_np), y, ids, w)
    torch.cuda.synchronize()
    t = g.q4moe_w4a16_decode_shared_q4_taps(router, ex, shx, T)
    b = host(ws)
    H, S = ex.hidden, shx.inter
    return dict(y=host(y, np.uint16), ids=host(ids), w=host(w),
                y32=b[t.y32: t.y32 + T * H * 4].view(np.float32).reshape(T, H).copy(),
                h32=b[t.sh_h32: t.sh_h32 + T * S * 4].view(np.float32).reshape(T, S).copy())


def _check_q4(L, shb, sh_fmt, out):
    r = L["route"]
    T = L["x"].shape[0]
    assert np.array_equal(out["ids"], r["ids"])
    np.testing.assert_allclose(out["w"], r["w"], rtol=1e-5)
    ob = oracle.Bank.from_dict(oracle.NVFP4 if L["fmt"] == "nvfp4" else oracle.INT4_G64, L["bank"])
    yr, _ = oracle.moe_w4a16(ob, L["x"], r["ids"], r["w"])
    osh = oracle.Bank.from_dict(oracle.NVFP4 if sh_fmt == "nvfp4" else oracle.INT4_G64, shb)
    zs, us = oracle.moe_w4a16(osh, L["x"], np.zeros((T, 1), np.int32), np.ones((T, 1)))
    ok, worst_h = gate_f32(out["h32"], np.maximum(us[:, 0, :], 0.0) ** 2)
    assert ok, f"shared h tap gate exceeded ({worst_h:.3f})"
    yhat = yr + zs
    ok, worst = gate_out(out["y"], yhat)
    assert ok, f"bf16 output gate exceeded ({worst:.3f})"
    ok32, worst32 = gate_f32(out["y32"], yhat)
    assert ok32, f"fp32 output gate exceeded ({worst32:.3f})"
    assert np.array_equal(out["y"], bf16_rne_of_f32(out["y32"]))
    return worst, worst_h


@pytest.mark.parametrize("fmt,sh_fmt,T", [("int4", "int4", 1), ("int4", "int4", 5), ("nvfp4", "int4", 3),
                                          ("nvfp4", "nvfp4", 1), ("nvfp4", "nvfp4", 8), ("int4", "nvfp4", 2)])
def test_q4_shared_small(fmt, sh_fmt, T):
    E, H, I, S = 16, 320, 448, 192
    fam = synth.FAM_NVFP4 if fmt == "nvfp4" else synth.FAM_INT4
    L = layer(SEED + 11 * T + len(sh_fmt), fam, 0, E, H, I, T, K, fmt)
    shb = synth.expert_bank(SEED, synth.FAM_INT4 if sh_fmt == "int4" else synth.FAM_NVFP4, 60 + T, 1, H, S, sh_fmt)
    print(f"{sh_fmt} shared with {fmt} routed: T={T}", flush=True)
    out = _run_q4(upload_router(L["wg"], L["b"], K), upload_bank(L["bank"], fmt), upload_bank(shb, sh_fmt), L["x"])
    _check_q4(L, shb, sh_fmt, out)


@pytest.mark.parametrize("T", [1, 4, 37])
def test_q4_shared_int4_checkpoint_full_layer(T):
    # the int4 checkpoint's MoE block: int4-g64 routed experts and an
    # int4-g64 shared expert (inter 3712)
    L = layer(SEED + T, synth.FAM_INT4, 0, 128, 2688, 1856, T, K, "int4")
    shb = synth.expert_bank(SEED, synth.FAM_INT4, 70, 1, 2688, 3712, "int4")
    print(f"int4 routed + int4 shared, full layer, T={T}", flush=True)
    out = _run_q4(upload_router(L["wg"], L["b"], K), upload_bank(L["bank"], "int4"), upload_bank(shb, "int4"),
                  L["x"])
    worst, worst_h = _check_q4(L, shb, "int4", out)
    print(f"int4 + int4 shared T={T}: worst bf16 ratio {worst:.3f}, shared h {worst_h:.4f}", flush=True)
