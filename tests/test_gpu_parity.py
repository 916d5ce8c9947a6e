"""GPU parity: every entry point through the C-ABI against the oracle on
the same seeded inputs (small shapes with ragged tails, and the full
workload shapes)."""
import numpy as np
import pytest
import torch

import gemm_router_fp32_amd as g
import oracle
import synth
from gpu_util import DEV, dev, host, run_decode, upload_bank, upload_router
from inputs import SEED, layer, x_with_clear_routing
from q4moe_testutil import bf16_bits_to_f64, bf16_rne_of_f32, gate_f32, gate_out, pack, unfloored_errors

pytestmark = pytest.mark.gpu

H, I, E, K = 2688, 1856, 128, 6


def _bits_equal(a, b):
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    nan = np.isnan(a) & np.isnan(b)
    return bool(np.all(nan | (a.view(np.uint32) == b.view(np.uint32))))


# --- dequantization: bit-exact ---------------------------------------------

@pytest.mark.parametrize("gs", [1.0, 1.0 / 64, 0.3, 2.0 ** -135, 3.0e38])
def test_dequant_nvfp4_exhaustive(gs):
    codes = np.tile(pack(np.arange(16, dtype=np.uint8)), (256, 1))
    scales = np.arange(256, dtype=np.uint8).reshape(256, 1)
    gt = dev(np.array([gs], np.float32))
    out = torch.empty((256, 16), dtype=torch.float32, device=DEV)
    g.q4moe_dequant_ref(g.QMat(g.NVFP4, dev(codes), dev(scales), gt), out)
    torch.cuda.synchronize()
    assert _bits_equal(host(out), oracle.dequant(oracle.NVFP4, codes, scales, gs))


def test_dequant_int4_exhaustive():
    sb = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    sb = sb[np.isfinite(bf16_bits_to_f64(sb))]
    codes = np.tile(pack(np.tile(np.arange(16, dtype=np.uint8), 4)), (sb.size, 1))
    out = torch.empty((sb.size, 64), dtype=torch.float32, device=DEV)
    g.q4moe_dequant_ref(g.QMat(g.INT4_G64, dev(codes), dev(sb.reshape(-1, 1))), out)
    torch.cuda.synchronize()
    assert _bits_equal(host(out), oracle.dequant(oracle.INT4_G64, codes, sb.reshape(-1, 1)))


@pytest.mark.parametrize("fmt", ["nvfp4", "int4"])
def test_dequant_full_expert_matrix(fmt):
    mat = synth.nvfp4_matrix if fmt == "nvfp4" else synth.int4_matrix
    c, s = mat(SEED, 0, 0, synth.S_UP_CODES, synth.S_UP_SCALES, 5, I, H)
    gs = 1.0 / 64 if fmt == "nvfp4" else None
    q = g.QMat(g.NVFP4 if fmt == "nvfp4" else g.INT4_G64, dev(c), dev(s),
               None if gs is None else dev(np.array([gs], np.float32)))
    out = torch.empty((I, H), dtype=torch.float32, device=DEV)
    g.q4moe_dequant_ref(q, out)
    torch.cuda.synchronize()
    ref = oracle.dequant(oracle.NVFP4 if fmt == "nvfp4" else oracle.INT4_G64, c, s, gs or 1.0)
    assert _bits_equal(host(out), ref)


# --- router: ids exact, gates within 1e-5 ------------------------------------

@pytest.mark.parametrize("T", [1, 4, 37, 200, 1000])
def test_router_topk(T):
    # 1: fused-decode form; 4: the small-batch logits kernel; 37, 200: the
    # MFMA router GEMM one token block per wave; 1000: two blocks per wave,
    # with a ragged last 32-token tile
    wg, b = synth.router(SEED, 0, 3, E, H)
    x, r, _ = x_with_clear_routing(SEED, 0, 3, wg, b, T, K)
    router = upload_router(wg, b, K)
    ids = torch.empty((T, K), dtype=torch.int32, device=DEV)
    w = torch.empty((T, K), dtype=torch.float32, device=DEV)
    lg = torch.empty((T, E), dtype=torch.float32, device=DEV)
    g.q4moe_router_topk(router, dev(x), ids, w, lg)
    torch.cuda.synchronize()
    assert np.array_equal(host(ids), r["ids"])
    np.testing.assert_allclose(host(w), r["w"], rtol=1e-5)
    np.testing.assert_allclose(host(lg), r["logits"], rtol=1e-5, atol=1e-5)


# --- W4A16 decode --------------------------------------------------------------

def _check_decode(L, out):
    ob = oracle.Bank.from_dict(oracle.NVFP4 if L["fmt"] == "nvfp4" else oracle.INT4_G64, L["bank"])
    r = L["route"]
    assert np.array_equal(out["ids"], r["ids"])
    np.testing.assert_allclose(out["w"], r["w"], rtol=1e-5)
    yhat, _ = oracle.moe_w4a16(ob, L["x"], r["ids"], r["w"])
    ok, worst = gate_out(out["y"], yhat)
    assert ok, f"bf16 output gate exceeded: worst error / bound = {worst:.3f}"
    ok32, worst32 = gate_f32(out["y32"], yhat)
    assert ok32, f"fp32 output gate exceeded: worst {worst32:.3f}"
    assert np.array_equal(out["y"], bf16_rne_of_f32(out["y32"]))
    return worst, worst32


@pytest.mark.parametrize("fmt", ["nvfp4", "int4"])
@pytest.mark.parametrize("T", [1, 2, 3, 4])
def test_decode_small_ragged(fmt, T):
    # 16 experts, hidden 256 (8 chunks per row), inter 192 (6 chunks)
    fam = synth.FAM_NVFP4 if fmt == "nvfp4" else synth.FAM_INT4
    L = layer(SEED + T, fam, 0, 16, 256, 192, T, K, fmt)
    out = run_decode(upload_router(L["wg"], L["b"], K), upload_bank(L["bank"], fmt), L["x"])
    _check_decode(L, out)


@pytest.fixture(scope="module")
def layer0():
    L = layer(SEED, synth.FAM_NVFP4, 0, E, H, I, 4, K, "nvfp4")
    return L, upload_bank(L["bank"], "nvfp4"), upload_router(L["wg"], L["b"], K)


@pytest.mark.parametrize("T", [1, 4])
def test_decode_full_layer_nvfp4(layer0, T):
    L, ex, router = layer0
    Lt = dict(L, x=L["x"][:T], route={k: v[:T] for k, v in L["route"].items()})
    out = run_decode(router, ex, Lt["x"])
    worst, worst32 = _check_decode(Lt, out)
    print(f"T={T}: worst bf16 ratio {worst:.3f}, fp32 ratio {worst32:.5f}")


def test_decode_deterministic_and_gscale_metamorphic(layer0):
    L, ex, router = layer0
    x = L["x"][:1]
    a = run_decode(router, ex, x)
    b = run_decode(router, ex, x, ws=a["ws"])
    assert np.array_equal(a["y32"].view(np.uint32), b["y32"].view(np.uint32))
    assert g.q4moe_ws_check(a["ws"]) == 0
    # doubling every up_proj per-tensor scale scales u by 2, h and y by 4 exactly
    up_g2 = ex.t[4] * 2
    ex2 = g.Experts(g.NVFP4, ex.t[0], ex.t[1], ex.t[2], ex.t[3], up_g2, ex.t[5])
    c = run_decode(router, ex2, x)
    assert np.array_equal(c["y32"], 4 * a["y32"])
    dn_g2 = ex.t[5] * 2
    ex3 = g.Experts(g.NVFP4, ex.t[0], ex.t[1], ex.t[2], ex.t[3], ex.t[4], dn_g2)
    d = run_decode(router, ex3, x)
    assert np.array_equal(d["y32"], 2 * a["y32"])


@pytest.fixture(scope="module")
def layer0_int4():
    L = layer(SEED, synth.FAM_INT4, 0, E, H, I, 4, K, "int4")
    return L, upload_bank(L["bank"], "int4"), upload_router(L["wg"], L["b"], K)


@pytest.mark.parametrize("T", [1, 2, 3, 4])
def test_decode_full_layer_int4(layer0_int4, T):
    # T = 1: the one-launch decode; 2-4: k_router_logits, k_topk, k_up<3>, k_down
    L, ex, router = layer0_int4
    Lt = dict(L, x=L["x"][:T], route={k: v[:T] for k, v in L["route"].items()})
    out = run_decode(router, ex, Lt["x"])
    worst, worst32 = _check_decode(Lt, out)
    print(f"int4 T={T}: worst bf16 ratio {worst:.3f}, fp32 ratio {worst32:.5f}")


@pytest.mark.parametrize("fmt", ["nvfp4", "int4"])
def test_decode_23_layer_stack(fmt):
    """All 23 layers of the stack workloads, each against the oracle."""
    fam = synth.FAM_NVFP4 if fmt == "nvfp4" else synth.FAM_INT4
    buf = None
    worst = 0.0
    rel = rel_r = norm = 0.0
    for li in range(23):
        L = layer(SEED, fam, li, E, H, I, 1, K, fmt, bank_out=buf)
        buf = L["bank"]
        out = run_decode(upload_router(L["wg"], L["b"], K), upload_bank(L["bank"], fmt), L["x"])
        w, _ = _check_decode(L, out)
        worst = max(worst, w)
        # the errors the floored gate does not show, reported
        yhat, _ = oracle.moe_w4a16(oracle.Bank.from_dict(oracle.NVFP4 if fmt == "nvfp4" else oracle.INT4_G64,
                                                         L["bank"]), L["x"], L["route"]["ids"], L["route"]["w"])
        a, b_, c = unfloored_errors(out["y"], yhat)
        rel, rel_r, norm = max(rel, a), max(rel_r, b_), max(norm, c)
        torch.cuda.empty_cache()
    print(f"{fmt} stack: worst bf16 ratio {worst:.3f}; unfloored max relative error {rel:.3g}, "
          f"beyond the half-ulp rounding {rel_r:.3g}, normwise {norm:.3g}")


# --- lm_head GEMV + argmax -----------------------------------------------------

def test_gemv_small_and_ties():
    codes, scales = synth.nvfp4_matrix(SEED, 0, 0, synth.S_LM_CODES, synth.S_LM_SCALES, 0, 1000, 256)
    # tokens 1-3 drawn with a clear top-1 gap (fp32 against fp64 cannot swap them)
    att = [0, 1, 2, 3]
    for _ in range(64):
        x = synth.x_rows(SEED, 0, 0, 256, att)
        lg, _, gp = oracle.gemv_nvfp4(codes, scales, 1 / 64, x)
        bad = [t for t in range(1, 4) if gp[t] < 1e-3 * max(1.0, np.abs(lg[t]).max())]
        if not bad:
            break
        for t in bad:
            att[t] += 4
    w_ = int(np.argmax(oracle.gemv_nvfp4(codes, scales, 1 / 64, x[:1])[0][0]))
    # duplicate the first token's best row at lower and higher indices: an
    # exact tie, broken towards the lowest row
    for dst in (3, w_ + 1 if w_ + 1 < 1000 else 999):
        codes[dst], scales[dst] = codes[w_], scales[w_]
    lref, amref, gap = oracle.gemv_nvfp4(codes, scales, 1 / 64, x)
    assert amref[0] == min(3, w_) and gap[0] == 0.0
    q = g.QMat(g.NVFP4, dev(codes), dev(scales), dev(np.array([1 / 64], np.float32)))
    for T in (1, 2, 3, 4):
        logits = torch.empty((T, 1000), dtype=torch.float32, device=DEV)
        am = torch.empty(T, dtype=torch.int32, device=DEV)
        g.q4moe_w4a16_gemv(q, dev(x[:T]), logits, am)
        torch.cuda.synchronize()
        ok, worst = gate_f32(host(logits), lref[:T])
        assert ok, worst
        assert np.array_equal(host(am), amref[:T]), f"T={T}: argmax {host(am).tolist()} != {amref[:T].tolist()}"


def test_verify_step_moe_and_lm_head(layer0):
    """Four tokens through one NVFP4 layer, then the NVFP4 lm_head over the
    same four tokens; the lm_head is checked on the GPU's own bf16 y."""
    L, ex, router = layer0
    V = 131072
    codes, scales, gsc = synth.lm_head(SEED, 0, 0, V, H)
    ob = oracle.Bank.from_dict(oracle.NVFP4, L["bank"])
    attempts = list(L["attempts"])
    for _ in range(16):  # argmax near-tie rule on the oracle's chained result
        x = synth.x_rows(SEED, 0, 0, H, attempts)
        r = oracle.router(L["wg"], L["b"], x, K)
        yhat, _ = oracle.moe_w4a16(ob, x, r["ids"], r["w"])
        _, _, gap = oracle.gemv_nvfp4(codes, scales, gsc, oracle.bf16_round(yhat))
        lg, _, _ = oracle.gemv_nvfp4(codes, scales, gsc, oracle.bf16_round(yhat))
        bad = [t for t in range(4) if r["gap"][t] < 1e-4 or gap[t] < 1e-3 * max(1.0, np.abs(lg[t]).max())]
        if not bad:
            break
        for t in bad:
            attempts[t] += 1
    out = run_decode(router, ex, x)
    _check_decode(dict(L, x=x, route=r), out)
    q = g.QMat(g.NVFP4, dev(codes), dev(scales), dev(np.array([gsc], np.float32)))
    logits = torch.empty((4, V), dtype=torch.float32, device=DEV)
    am = torch.empty(4, dtype=torch.int32, device=DEV)
    g.q4moe_w4a16_gemv(q, dev(out["y"]), logits, am)
    torch.cuda.synchronize()
    lref, amref, _ = oracle.gemv_nvfp4(codes, scales, gsc, out["y"])
    ok, worst = gate_f32(host(logits), lref)
    assert ok, worst
    assert np.array_equal(host(am), amref)
