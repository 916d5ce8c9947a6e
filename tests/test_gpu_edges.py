"""GPU parity on edge cases, through the C-ABI, against the oracle.

* Exact key ties (duplicated router rows and biases; an all-zero W_g with
  pairwise-equal biases), inside the top 6 and at the 6th/7th boundary,
  through every top-k implementation: the one-launch decode (W4A16 NVFP4
  and int4, W4A4), the small-batch up kernel (2-4 NVFP4 tokens), and k_topk
  after the per-expert logits (int4 2-4 tokens, the router entry point) and
  after the fp32 MFMA router GEMM (16 tokens or more: the router entry
  point and the W4A4 grouped chunk).  ids bit-exact, the lower index first.
* Block scales drawn from every finite E4M3FN byte (subnormals, zeros, 448,
  negative bytes) with a per-tensor scale of 0.3, through the one-launch
  decode, the small-batch decode, the W4A4 decode, the W4A4 grouped chunk
  and the lm_head GEMV.
* Activation rows with a 2^40 dynamic range, all-zero rows and bf16
  subnormals (the fp16 staging of the lm_head and small-batch kernels).
* W4A4 with all-zero 16-blocks of x and of h.
* All-negative u (every up weight <= 0 against x >= 0): y = +0 exactly.
"""
import numpy as np
import pytest

import gemm_router_fp32_amd as g
import oracle
import synth
from gpu_util import dev, run_entry, run_gemv, upload_bank, upload_router
from inputs import GAP, SEED, x_with_clear_routing
from q4moe_testutil import bf16_bits_to_f64, bf16_rne_of_f32, gate_f32, gate_out
from test_gpu_w4a4 import _check as check_grouped, _run as run_grouped
from test_gpu_w4a4_decode import check_w4a4_decode, run_w4a4_decode

pytestmark = pytest.mark.gpu

K = 6
FAM_EDGE = 5  # a family of its own for these inputs


def _fmt_const(fmt):
    return oracle.NVFP4 if fmt == "nvfp4" else oracle.INT4_G64


def _check_y(bank, fmt, x, r, out):
    ob = oracle.Bank.from_dict(_fmt_const(fmt), bank)
    yhat, _ = oracle.moe_w4a16(ob, x, r["ids"], r["w"])
    ok, worst = gate_out(out["y"], yhat)
    assert ok, f"bf16 output gate exceeded: worst {worst:.3f}"
    return worst


def _route_ok(out, r, what):
    assert np.array_equal(out["ids"], r["ids"]), f"{what}: ids {out['ids'].tolist()} != {r['ids'].tolist()}"
    np.testing.assert_allclose(out["w"], r["w"], rtol=1e-5, err_msg=what)


def _f32_keys_agree(wg, b, x, r):
    """For all-zero logits the GPU keys are fl32(0.5 + b): check that their
    order (ties to the lower index) picks the oracle's ids."""
    key32 = np.float32(0.5) + b.astype(np.float32)
    order = np.lexsort((np.arange(b.size), -key32.astype(np.float64)))
    return np.array_equal(order[:K], r["ids"][0])


# --- exact ties ------------------------------------------------------------

def _dup_router(E, H):
    """A router whose token-0 keys hold the ties (t1, a), t2, (t3, c), (t4, d):
    two ties inside the top 6 and one at the 6th/7th boundary."""
    for li in range(64):
        wg, b = synth.router(SEED, FAM_EDGE, li, E, H)
        x0 = synth.x_rows(SEED, FAM_EDGE, li, H, [0])
        r = oracle.router(wg, b, x0, K)
        key = r["scores"][0] + b.astype(np.float64)
        order = [int(e) for e in np.argsort(-key, kind="stable")]
        if np.min(-np.diff(key[order[:8]])) < GAP:  # distinct keys far apart
            continue
        t = order[:7]
        rest = [e for e in range(E) if e not in t]
        pairs = ((t[0], rest[0]), (t[2], rest[-1]), (t[3], rest[len(rest) // 2]))
        for src, dst in pairs:
            wg[dst] = wg[src]
            b[dst] = b[src]
        r = oracle.router(wg, b, x0, K)
        assert r["gap"][0] == 0.0
        return wg, b, li, x0
    raise RuntimeError("no router found")


def _tie_tokens(wg, b, li, x0, T, redraw=True):
    """Token 0 holds the planted ties; tokens 1.. are drawn with no near tie
    (an exact tie, gap 0, is kept).  With an all-zero W_g every token routes
    on the bias alone (exact on both sides): nothing is redrawn."""
    H = wg.shape[1]
    att = [0] * T
    for _ in range(64):
        x = synth.x_rows(SEED, FAM_EDGE, li, H, att)
        x[0] = x0[0]
        r = oracle.router(wg, b, x, K)
        bad = [t for t in range(1, T) if redraw and 0.0 < r["gap"][t] < GAP]
        if not bad:
            return x, r
        for t in bad:
            att[t] += 1
    raise RuntimeError("no clear tokens found")


def _zero_router(E, H):
    """All-zero W_g and pairwise-equal biases: every key is 0.5 + b, tied in
    pairs (2i, 2i + 1)."""
    for li in range(64):
        _, b = synth.router(SEED, FAM_EDGE, 100 + li, E, H)
        b[1::2] = b[0::2][: b[1::2].size]
        wg = np.zeros((E, H), np.float32)
        x0 = synth.x_rows(SEED, FAM_EDGE, 100 + li, H, [0])
        r = oracle.router(wg, b, x0, K)
        if _f32_keys_agree(wg, b, x0, r):
            return wg, b, 100 + li, x0
    raise RuntimeError("no router found")


def _run_topk(router, x):
    import torch
    from gpu_util import DEV, host
    T = x.shape[0]
    ids = torch.empty((T, K), dtype=torch.int32, device=DEV)
    w = torch.empty((T, K), dtype=torch.float32, device=DEV)
    g.q4moe_router_topk(router, dev(x), ids, w)
    torch.cuda.synchronize()
    return dict(ids=host(ids), w=host(w))


@pytest.mark.parametrize("kind", ["dup", "zero"])
@pytest.mark.parametrize("E", [128, 200])
def test_ties_every_topk(kind, E):
    H, I = 256, 192
    wg, b, li, x0 = _dup_router(E, H) if kind == "dup" else _zero_router(E, H)
    router = upload_router(wg, b, K)
    x37, r37 = _tie_tokens(wg, b, li, x0, 37, redraw=kind == "dup")
    print(f"ties ({kind}, E={E}): token 0 ids {r37['ids'][0].tolist()}, gap {r37['gap'][0]}", flush=True)
    # router entry point: k_router_logits + k_topk (1, 4), MFMA GEMM + k_topk (37)
    for T in (1, 4, 37):
        _route_ok(_run_topk(router, x37[:T]), {k: v[:T] for k, v in r37.items()}, f"router_topk T={T}")
    for fmt in ("nvfp4", "int4"):
        bank = synth.expert_bank(SEED, FAM_EDGE, li, E, H, I, fmt)
        ex = upload_bank(bank, fmt)
        # one launch (wave_topk); NVFP4 2-4 tokens: k_small_up; int4: k_topk
        for T in ((1, 4) if fmt == "nvfp4" else (1, 2)):
            rT = {k: v[:T] for k, v in r37.items()}
            out = run_entry(g.q4moe_w4a16_decode, router, ex, x37[:T])
            _route_ok(out, rT, f"w4a16 {fmt} T={T}")
            _check_y(bank, fmt, x37[:T], rT, out)
        if fmt == "nvfp4":
            r1 = {k: v[:1] for k, v in r37.items()}
            out = run_w4a4_decode(router, ex, x37[:1])
            check_w4a4_decode(dict(bank=bank, x=x37[:1], route=r1), out)
            # the grouped chunk: fp32 MFMA router GEMM, then k_topk
            out = run_grouped(router, ex, x37, K)
            check_grouped(bank, wg, b, x37, r37, out, K)


# --- every finite E4M3FN scale byte, per-tensor scale 0.3 ---------------------

@pytest.fixture(scope="module")
def all_bytes_layer():
    E, H, I = 16, 2688, 1856
    bank = synth.expert_bank(SEED, FAM_EDGE, 200, E, H, I, "nvfp4", gscale=0.3,
                             scale_bytes=synth.E4M3_FINITE_BYTES)
    wg, b = synth.router(SEED, FAM_EDGE, 200, E, H)
    x, r, _ = x_with_clear_routing(SEED, FAM_EDGE, 200, wg, b, 64, K)
    return bank, wg, b, x, r, upload_bank(bank, "nvfp4"), upload_router(wg, b, K)


def test_all_scale_bytes_decode(all_bytes_layer):
    bank, wg, b, x, r, ex, router = all_bytes_layer
    for T in (1, 4):  # one launch; small-batch MFMA kernels
        rT = {k: v[:T] for k, v in r.items()}
        out = run_entry(g.q4moe_w4a16_decode, router, ex, x[:T])
        _route_ok(out, rT, f"T={T}")
        worst = _check_y(bank, "nvfp4", x[:T], rT, out)
        print(f"all scale bytes, w4a16 T={T}: worst bf16 ratio {worst:.3f}", flush=True)


def test_all_scale_bytes_w4a4(all_bytes_layer):
    bank, wg, b, x, r, ex, router = all_bytes_layer
    out = run_w4a4_decode(router, ex, x[:1])
    check_w4a4_decode(dict(bank=bank, x=x[:1], route={k: v[:1] for k, v in r.items()}), out)
    out = run_grouped(router, ex, x, K)
    wh, wy = check_grouped(bank, wg, b, x, r, out, K)
    print(f"all scale bytes, grouped T=64: h {wh:.3f}, y {wy:.3f}", flush=True)


def _clear_argmax_rows(codes, scales, gs, H, T, fam, transform=None):
    att = [0] * T
    for _ in range(64):
        x = synth.x_rows(SEED, fam, 0, H, att)
        if transform is not None:
            x = transform(x)
        lg, am, gap = oracle.gemv_nvfp4(codes, scales, gs, x)
        bad = [t for t in range(T) if 0.0 < gap[t] < 1e-3 * max(1.0, np.abs(lg[t]).max())]
        if not bad:
            return x, lg, am
        for t in bad:
            att[t] += 1
    raise RuntimeError("no clear argmax rows found")


def test_all_scale_bytes_lm_head():
    V, H = 4096, 2688
    codes, scales, gs = synth.lm_head(SEED, FAM_EDGE, 201, V, H, gscale=0.3, scale_bytes=synth.E4M3_FINITE_BYTES)
    q = g.QMat(g.NVFP4, dev(codes), dev(scales), dev(np.array([gs], np.float32)))
    x, lref, amref = _clear_argmax_rows(codes, scales, gs, H, 4, FAM_EDGE)
    for T in (1, 2, 3, 4):
        logits, am = run_gemv(q, x[:T])
        ok, worst = gate_f32(logits, lref[:T])
        assert ok, f"T={T}: logits gate exceeded ({worst:.3f})"
        assert np.array_equal(am, amref[:T]), f"T={T}: argmax {am.tolist()} != {amref[:T].tolist()}"


# --- activation dynamic range, zero rows, bf16 subnormals ---------------------

def _to_bits(f32):
    u = np.asarray(f32, np.float32).view(np.uint32)
    assert np.all((u & 0xFFFF) == 0)
    return (u >> 16).astype(np.uint16)


def _dyn(x):
    """Row 0: 2^40 dynamic range (32 elements x 2^20, 32 x 2^-20); row 1: all
    zero; row 2: 64 elements replaced by bf16 subnormals; row 3 as drawn."""
    x = x.copy()
    f = bf16_bits_to_f64(x).astype(np.float32)
    f[0, 0:32] *= np.float32(2.0 ** 20)
    f[0, 32:64] *= np.float32(2.0 ** -20)
    x[0] = _to_bits(f[0])
    x[1] = 0
    sub = (np.arange(64, dtype=np.uint16) % 127 + 1) | np.where(np.arange(64) % 2 == 1, 0x8000, 0).astype(np.uint16)
    x[2, 100:164] = sub
    return x


def test_dynamic_range_small_batch_and_one_launch():
    E, H, I = 128, 2688, 1856
    # a router whose zero row (bias-only routing) has a clear, fp32-safe order
    for li in range(300, 364):
        wg, b = synth.router(SEED, FAM_EDGE, li, E, H)
        r0 = oracle.router(wg, b, np.zeros((1, H), np.uint16), K)
        if r0["gap"][0] >= GAP and _f32_keys_agree(wg, b, None, r0):
            break
    x, r, _ = x_with_clear_routing(SEED, FAM_EDGE, li, wg, b, 4, K, transform=_dyn)
    bank = synth.expert_bank(SEED, FAM_EDGE, li, E, H, I, "nvfp4", experts=np.unique(r["ids"]))
    ex, router = upload_bank(bank, "nvfp4"), upload_router(wg, b, K)
    out = run_entry(g.q4moe_w4a16_decode, router, ex, x)  # small-batch MFMA kernels
    _route_ok(out, r, "T=4")
    assert np.all(out["y"][1] == 0), "an all-zero row gives y = +0"
    ob = oracle.Bank.from_dict(oracle.NVFP4, bank)
    yhat, _ = oracle.moe_w4a16(ob, x, r["ids"], r["w"])
    for t in (0, 2, 3):
        ok, worst = gate_out(out["y"][t:t + 1], yhat[t:t + 1])
        assert ok, f"token {t}: bf16 gate exceeded ({worst:.3f})"
    for t in (0, 1, 2):  # the one-launch decode on each special row
        o1 = run_entry(g.q4moe_w4a16_decode, router, ex, x[t:t + 1])
        _route_ok(o1, {k: v[t:t + 1] for k, v in r.items()}, f"one launch, row {t}")
        if t == 1:
            assert np.all(o1["y"] == 0)
        else:
            ok, worst = gate_out(o1["y"], yhat[t:t + 1])
            assert ok, f"one launch, row {t}: gate exceeded ({worst:.3f})"


def test_dynamic_range_lm_head():
    V, H = 2048, 2688
    codes, scales, gs = synth.lm_head(SEED, FAM_EDGE, 400, V, H)
    q = g.QMat(g.NVFP4, dev(codes), dev(scales), dev(np.array([gs], np.float32)))
    x, lref, amref = _clear_argmax_rows(codes, scales, gs, H, 4, FAM_EDGE + 1, transform=_dyn)
    logits, am = run_gemv(q, x)
    assert np.all(logits[1] == 0) and am[1] == 0, "zero row: every logit 0, argmax the lowest row"
    for t in (0, 2, 3):
        ok, worst = gate_f32(logits[t:t + 1], lref[t:t + 1])
        assert ok, f"token {t}: logits gate exceeded ({worst:.3f})"
    assert np.array_equal(am, amref)
    # a row of bf16 subnormals only, with a large per-tensor scale so that
    # the logits are normal fp32 numbers
    gsub = np.float32(2.0 ** 20)
    q2 = g.QMat(g.NVFP4, dev(codes), dev(scales), dev(np.array([gsub], np.float32)))
    xs = synth.x_rows(SEED, FAM_EDGE, 401, H, [0])
    xs = ((xs & 0x8000) | (synth.bytes_(synth.key(SEED, FAM_EDGE, 401, 99), H) % 127 + 1)).astype(np.uint16)
    lg, amg = run_gemv(q2, xs)
    lr, amr, gap = oracle.gemv_nvfp4(codes, scales, gsub, xs)
    assert np.all(np.isfinite(lg))
    ok, worst = gate_f32(lg, lr)
    assert ok, f"subnormal row: logits gate exceeded ({worst:.3f})"
    if gap[0] > 1e-3 * np.abs(lr).max():
        assert amg[0] == amr[0]


# --- W4A4: all-zero blocks of x and h ----------------------------------------

def test_w4a4_zero_blocks():
    E, H, I = 16, 2688, 1856
    bank = synth.expert_bank(SEED, FAM_EDGE, 500, E, H, I, "nvfp4")
    # up rows 0-15 and 32-47 of every expert are zero: h blocks 0 and 2 of
    # every (token, slot) row are exactly zero
    bank["up_codes"][:, 0:16] = 0
    bank["up_codes"][:, 32:48] = 0
    wg, b = synth.router(SEED, FAM_EDGE, 500, E, H)

    def zero_blocks(x):
        x = x.copy()
        x[:, 0:16] = 0
        x[:, 80:96] = 0
        x[:, 1600:1616] = 0
        x[:, 112:128] = 0x8000  # a block of negative zeros
        return x

    x, r, _ = x_with_clear_routing(SEED, FAM_EDGE, 500, wg, b, 16, K, transform=zero_blocks)
    ex, router = upload_bank(bank, "nvfp4"), upload_router(wg, b, K)
    out = run_w4a4_decode(router, ex, x[:1])
    check_w4a4_decode(dict(bank=bank, x=x[:1], route={k: v[:1] for k, v in r.items()}), out)
    assert np.all(out["xq_scales"][0, [0, 5, 100, 7]] == 0)
    assert np.all(out["hq_scales"][:, [0, 2]] == 0)
    out = run_grouped(router, ex, x, K)
    check_grouped(bank, wg, b, x, r, out, K)
    assert np.all(out["hq_scales"][:, [0, 2]] == 0)


# --- all-negative u: y = +0 exactly ------------------------------------------

@pytest.mark.parametrize("fmt", ["nvfp4", "int4"])
def test_all_negative_u_gives_positive_zero(fmt):
    E, H, I = 16, 2688, 1856
    bank = synth.expert_bank(SEED, FAM_EDGE, 600, E, H, I, fmt)
    bank["up_codes"] |= 0x88  # every up code negative (NVFP4 -0..-6, int4 -8..-1)
    wg, b = synth.router(SEED, FAM_EDGE, 600, E, H)
    x, r, _ = x_with_clear_routing(SEED, FAM_EDGE, 600, wg, b, 16, K, transform=lambda v: v & 0x7FFF)
    ex, router = upload_bank(bank, fmt), upload_router(wg, b, K)
    for T in (1, 2, 4):
        out = run_entry(g.q4moe_w4a16_decode, router, ex, x[:T])
        _route_ok(out, {k: v[:T] for k, v in r.items()}, f"{fmt} T={T}")
        assert np.all(out["y"] == 0), f"{fmt} T={T}: y is not +0 everywhere"
    if fmt == "nvfp4":
        out = run_w4a4_decode(router, ex, x[:1])
        assert np.all(out["y"] == 0) and np.all(out["hq_scales"] == 0)
        out = run_grouped(router, ex, x, K)
        assert np.all(out["y"] == 0) and np.all(out["hq_scales"] == 0)
        assert np.all(out["y32"].view(np.uint32) == 0)
