"""GPU parity of the W4A16 decode above four tokens, NVFP4 and int4-g64,
against the oracle on every token: ids bit-exact, gates within 1e-5, y
within the output gate, y equal to the nearest-even bf16 of its fp32 value,
and the h tap (pair order) within 2e-3 of the oracle's relu(u)^2.  The
decode entry takes the 8-token small-batch kernels for NVFP4 at 5-8 tokens
and the grouped path (per-expert dispatch, grouped MFMA GEMMs with fp16
activations) above that and for int4 from 3 tokens; the grouped entry point
is also run directly at 1-8 tokens."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import DEV, dev, host, run_decode, upload_bank, upload_router, ws_view
from inputs import SEED, layer, x_with_clear_routing
from q4moe_testutil import bf16_rne_of_f32, gate_f32, gate_out, unfloored_errors

import gemm_router_fp32_amd as g

pytestmark = pytest.mark.gpu

H, I, E, K = 2688, 1856, 128, 6


def _check(L, out, router, ex, label):
    ob = oracle.Bank.from_dict(oracle.NVFP4 if L["fmt"] == "nvfp4" else oracle.INT4_G64, L["bank"])
    r = L["route"]
    T, k = r["ids"].shape
    assert np.array_equal(out["ids"], r["ids"])
    np.testing.assert_allclose(out["w"], r["w"], rtol=1e-5)
    yhat, u = oracle.moe_w4a16(ob, L["x"], r["ids"], r["w"])
    ok, worst = gate_out(out["y"], yhat)
    assert ok, f"{label}: bf16 output gate exceeded: worst error / bound = {worst:.3f}"
    ok32, worst32 = gate_f32(out["y32"], yhat)
    assert ok32, f"{label}: fp32 output gate exceeded: worst {worst32:.3f}"
    assert np.array_equal(out["y"], bf16_rne_of_f32(out["y32"]))
    # h tap, rows (token, slot)
    taps = g.q4moe_w4a16_decode_taps(router, ex, T)
    h = ws_view(host(out["ws"]), taps.h, T * k * ex.inter, np.float32).reshape(T * k, ex.inter)
    okh, worsth = gate_f32(h, (np.maximum(u, 0.0) ** 2).reshape(T * k, ex.inter))
    assert okh, f"{label}: h tap gate exceeded: worst {worsth:.3f}"
    rel, rel_r, norm = unfloored_errors(out["y"], yhat)
    print(f"{label}: worst bf16 ratio {worst:.3f}, fp32 {worst32:.4f}, h {worsth:.4f}; "
          f"unfloored rel {rel:.2e} (after rounding {rel_r:.2e}), normwise {norm:.2e}", flush=True)


# --- small shapes with ragged tails --------------------------------------------
# (E, H, I): H = 320 and I = 448 end inside a 256-wide chunk and inside a
# 128-column tile; H = 640 runs a whole turn of the three-slot ring plus a
# remainder; E = 12 is not a multiple of 8 (the plain workgroup mapping)

@pytest.mark.parametrize("fmt", ["nvfp4", "int4"])
@pytest.mark.parametrize("shape,T", [((16, 320, 448), 5), ((16, 640, 192), 8), ((12, 256, 320), 37),
                                     ((16, 320, 448), 100)])
def test_midbatch_small_ragged(fmt, shape, T):
    En, Hn, In = shape
    fam = synth.FAM_NVFP4 if fmt == "nvfp4" else synth.FAM_INT4
    L = layer(SEED + T, fam, 0, En, Hn, In, T, K, fmt)
    router, ex = upload_router(L["wg"], L["b"], K), upload_bank(L["bank"], fmt)
    print(f"grouped W4A16 {fmt} E={En} H={Hn} I={In} T={T}", flush=True)
    out = run_decode(router, ex, L["x"])
    _check(L, out, router, ex, f"{fmt} {shape} T={T}")


@pytest.fixture(scope="module", params=["nvfp4", "int4"])
def full_layer(request):
    fmt = request.param
    fam = synth.FAM_NVFP4 if fmt == "nvfp4" else synth.FAM_INT4
    L = layer(SEED, fam, 0, E, H, I, 200, K, fmt)
    return L, upload_bank(L["bank"], fmt), upload_router(L["wg"], L["b"], K)


@pytest.mark.parametrize("T", [5, 8, 37, 200])
def test_midbatch_full_shape(full_layer, T):
    L, ex, router = full_layer
    Lt = dict(L, x=L["x"][:T], route={k: v[:T] for k, v in L["route"].items()})
    print(f"grouped W4A16 {L['fmt']} full shape T={T}", flush=True)
    out = run_decode(router, ex, Lt["x"])
    _check(Lt, out, router, ex, f"{L['fmt']} full T={T}")


@pytest.mark.parametrize("fmt", ["nvfp4", "int4"])
def test_midbatch_skewed_routing(fmt):
    # every token picks experts 0..5 (bias far above any score): 200 rows per
    # expert, so the up GEMM takes 7 M-tiles and the down GEMM 13
    fam = synth.FAM_NVFP4 if fmt == "nvfp4" else synth.FAM_INT4
    En, Hn, In, T = 16, 640, 448, 200
    bank = synth.expert_bank(SEED, fam, 5, En, Hn, In, fmt)
    wg, b = synth.router(SEED, fam, 5, En, Hn)
    b = b.copy()
    b[:K] += 10.0
    x, r, _ = x_with_clear_routing(SEED, fam, 5, wg, b, T, K)
    assert set(np.unique(r["ids"])) == set(range(K))
    L = dict(bank=bank, wg=wg, b=b, x=x, route=r, fmt=fmt)
    router, ex = upload_router(wg, b, K), upload_bank(bank, fmt)
    print(f"grouped W4A16 {fmt} skewed routing T={T}", flush=True)
    out = run_decode(router, ex, x)
    _check(L, out, router, ex, f"{fmt} skewed")


def test_midbatch_int4_wide_scale_range():
    # int4 group scales spread over 2^-24 .. 2^0 inside every row: the
    # per-row power of two must keep the large ones exact and the small
    # ones harmless
    En, Hn, In, T = 16, 640, 448, 24
    bank = synth.expert_bank(SEED, synth.FAM_INT4, 6, En, Hn, In, "int4")
    rng = np.random.default_rng(SEED + 6)
    for key in ("up_scales", "down_scales"):
        s = bank[key]
        mag = np.exp2(rng.uniform(-24.0, 0.0, size=s.shape)).astype(np.float32)
        bits = (mag.view(np.uint32) >> 16).astype(np.uint16)
        bank[key] = bits.reshape(s.shape)
    wg, b = synth.router(SEED, synth.FAM_INT4, 6, En, Hn)
    x, r, _ = x_with_clear_routing(SEED, synth.FAM_INT4, 6, wg, b, T, K)
    L = dict(bank=bank, wg=wg, b=b, x=x, route=r, fmt="int4")
    router, ex = upload_router(wg, b, K), upload_bank(bank, "int4")
    print("grouped W4A16 int4 wide scale range", flush=True)
    out = run_decode(router, ex, x)
    _check(L, out, router, ex, "int4 wide scales")


def test_midbatch_workspace_reuse_and_determinism(full_layer):
    # the same call twice on one workspace, after a different token count
    L, ex, router = full_layer
    a = run_decode(router, ex, L["x"][:37])
    run_decode(router, ex, L["x"][:8], ws=a["ws"])
    b = run_decode(router, ex, L["x"][:37], ws=a["ws"])
    assert np.array_equal(a["y"], b["y"]) and np.array_equal(a["y32"].view(np.uint32), b["y32"].view(np.uint32))


@pytest.mark.parametrize("T", [1, 2, 4, 5, 8])
def test_grouped_entry_few_tokens(full_layer, T):
    # the grouped path called directly at 1-4 tokens (where the decode entry
    # takes the single-launch or small-batch kernels)
    import torch
    L, ex, router = full_layer
    Lt = dict(L, x=L["x"][:T], route={k: v[:T] for k, v in L["route"].items()})
    y = torch.empty((T, H), dtype=torch.int16, device=DEV)
    ids = torch.empty((T, K), dtype=torch.int32, device=DEV)
    w = torch.empty((T, K), dtype=torch.float32, device=DEV)
    print(f"grouped entry {L['fmt']} T={T}", flush=True)
    ws = g.q4moe_w4a16_grouped(router, ex, dev(Lt["x"]), y, ids, w)
    torch.cuda.synchronize()
    taps = g.q4moe_w4a16_decode_taps(router, ex, T)
    y32 = ws_view(host(ws), taps.y32, T * H, np.float32).reshape(T, H)
    out = dict(y=host(y, np.uint16), ids=host(ids), w=host(w), y32=y32, ws=ws)
    _check(Lt, out, router, ex, f"{L['fmt']} grouped entry T={T}")
