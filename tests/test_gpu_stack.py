"""GPU parity of the stacked single-token decode (q4moe_w4a16_decode_stack):
every layer of a stack against the oracle, and bit for bit against the
one-layer decode (q4moe_w4a16_decode) of the same layer and input.  Stacks
longer than one launch (24 layers) check the hand-over between launches; the
chained form (x of a layer = y of the one before) runs on layers whose down
scales keep y near unit size, so that a deep chain neither overflows nor
vanishes."""
import numpy as np
import pytest
import torch

import gemm_router_fp32_amd as g
import oracle
import synth
from gpu_util import DEV, dev, host, run_decode, upload_bank, upload_router
from inputs import GAP, SEED, layer
from q4moe_testutil import bf16_rne_of_f32, gate_out

pytestmark = pytest.mark.gpu

FULL = dict(E=128, H=2688, I=1856, K=6)
SMALL = dict(E=16, H=256, I=192, K=4)


def _run_stack(routers, banks, xs, H, K, chain=False):
    n = len(routers)
    xt = [None if x is None else dev(x) for x in xs]  # kept alive through the call
    ys = [torch.empty(H, dtype=torch.int16, device=DEV) for _ in range(n)]
    ids = [torch.empty(K, dtype=torch.int32, device=DEV) for _ in range(n)]
    w = [torch.empty(K, dtype=torch.float32, device=DEV) for _ in range(n)]
    g.q4moe_w4a16_decode_stack(routers, banks, xt, ys, chain=chain, ids=ids, w=w)
    torch.cuda.synchronize()
    return [host(y, np.uint16) for y in ys], [host(i) for i in ids], [host(v) for v in w]


def _oracle_bank(fmt, bank):
    return oracle.Bank.from_dict(oracle.NVFP4 if fmt == "nvfp4" else oracle.INT4_G64, bank)


def _fresh_stack(fmt, shape, n):
    """n independent layers (inputs with clear routing), uploaded, with the
    oracle's routing and y of each."""
    fam = synth.FAM_NVFP4 if fmt == "nvfp4" else synth.FAM_INT4
    routers, banks, xs, refs = [], [], [], []
    for li in range(n):
        L = layer(SEED, fam, li, shape["E"], shape["H"], shape["I"], 1, shape["K"], fmt)
        routers.append(upload_router(L["wg"], L["b"], shape["K"]))
        banks.append(upload_bank(L["bank"], fmt))
        xs.append(L["x"][0])
        r = L["route"]
        yhat, _ = oracle.moe_w4a16(_oracle_bank(fmt, L["bank"]), L["x"], r["ids"], r["w"])
        refs.append((r["ids"][0], r["w"][0], yhat[0]))
    return routers, banks, xs, refs


@pytest.mark.parametrize("fmt", ["nvfp4", "int4"])
@pytest.mark.parametrize("shape,n", [(FULL, 23), (SMALL, 30)], ids=["full-23", "small-30"])
def test_stack_independent_layers(fmt, shape, n):
    routers, banks, xs, refs = _fresh_stack(fmt, shape, n)
    ys, ids, w = _run_stack(routers, banks, xs, shape["H"], shape["K"])
    worst = 0.0
    for li in range(n):
        rid, rw, yhat = refs[li]
        assert np.array_equal(ids[li], rid), f"layer {li}: ids {ids[li]} != {rid}"
        np.testing.assert_allclose(w[li], rw, rtol=1e-5)
        ok, wr = gate_out(ys[li][None], yhat[None])
        assert ok, f"layer {li}: bf16 output gate exceeded ({wr:.3f})"
        worst = max(worst, wr)
        # the same layer through the one-layer launch: the same arithmetic
        one = run_decode(routers[li], banks[li], xs[li][None])
        assert np.array_equal(one["y"][0], ys[li]), f"layer {li}: stack y differs from the one-layer y"
    print(f"{fmt} {n}-layer stack: worst bf16 ratio {worst:.3f}")
    torch.cuda.empty_cache()


@pytest.mark.parametrize("shape,n", [(FULL, 4), (SMALL, 26)], ids=["full-4", "small-26"])
def test_stack_chained(shape, n):
    """NVFP4 layers chained through y.  Each layer's per-tensor down scales
    are divided by the rms of its y (an oracle dry run) so that y stays near
    unit size.  Per layer: the oracle's routing of the GPU's own input (its
    ids exact wherever the 6th/7th keys are clearly apart), y against the
    oracle under the GPU's routing, and the input equal to the previous
    layer's output bit for bit."""
    E, H, I, K = shape["E"], shape["H"], shape["I"], shape["K"]
    fam = synth.FAM_NVFP4
    routers, banks, obanks, rw = [], [], [], []
    x0 = None
    x = None
    for li in range(n):
        bank = synth.expert_bank(SEED, fam, 100 + li, E, H, I, "nvfp4")
        wg, b = synth.router(SEED, fam, 100 + li, E, H)
        if li == 0:
            L = layer(SEED, fam, 100, E, H, I, 1, K, "nvfp4")
            x0 = L["x"][0]
            x = x0
        r = oracle.router(wg, b, x[None], K)
        y, _ = oracle.moe_w4a16(_oracle_bank("nvfp4", bank), x[None], r["ids"], r["w"])
        s = float(np.sqrt(np.mean(np.asarray(y, np.float64) ** 2)))
        bank["down_gscale"] = (bank["down_gscale"] / np.float32(s if s > 0 else 1.0)).astype(np.float32)
        ob = _oracle_bank("nvfp4", bank)
        y, _ = oracle.moe_w4a16(ob, x[None], r["ids"], r["w"])
        x = bf16_rne_of_f32(np.asarray(y[0], np.float32)).astype(np.uint16)
        routers.append(upload_router(wg, b, K))
        banks.append(upload_bank(bank, "nvfp4"))
        obanks.append(ob)
        rw.append((wg, b))
    xs = [x0] + [None] * (n - 1)
    ys, ids, w = _run_stack(routers, banks, xs, H, K, chain=True)
    clear = 0
    for li in range(n):
        xin = x0 if li == 0 else ys[li - 1]
        r = oracle.router(rw[li][0], rw[li][1], xin[None], K)
        if r["gap"][0] >= GAP:
            clear += 1
            assert np.array_equal(ids[li], r["ids"][0]), f"layer {li}: ids {ids[li]} != {r['ids'][0]}"
            np.testing.assert_allclose(w[li], r["w"][0], rtol=1e-5)
        yhat, _ = oracle.moe_w4a16(obanks[li], xin[None], ids[li][None], w[li][None].astype(np.float64))
        ok, wr = gate_out(ys[li][None], yhat)
        assert ok, f"layer {li}: bf16 output gate exceeded ({wr:.3f})"
        assert np.abs(yhat).max() > 1e-3, f"layer {li}: y vanished"
    assert clear >= n // 2, f"only {clear} of {n} layers had a clear routing"
    torch.cuda.empty_cache()


def test_stack_validation():
    E, H, I, K = SMALL["E"], SMALL["H"], SMALL["I"], SMALL["K"]
    L = layer(SEED, synth.FAM_NVFP4, 0, E, H, I, 1, K, "nvfp4")
    r = upload_router(L["wg"], L["b"], K)
    ex = upload_bank(L["bank"], "nvfp4")
    y = torch.empty(H, dtype=torch.int16, device=DEV)
    x = dev(L["x"][0])
    L2 = layer(SEED, synth.FAM_NVFP4, 1, E, H, I + 64, 1, K, "nvfp4")
    ex2 = upload_bank(L2["bank"], "nvfp4")
    with pytest.raises(g.Q4moeError) as e:  # layers of different shapes
        g.q4moe_w4a16_decode_stack([r, r], [ex, ex2], [x, x], [y, y])
    assert e.value.status == g.EINVAL
    with pytest.raises(g.Q4moeError) as e:  # a missing x outside a chain
        g.q4moe_w4a16_decode_stack([r, r], [ex, ex], [x, None], [y, y])
    assert e.value.status == g.EINVAL
    # in a chain the later x are not read
    g.q4moe_w4a16_decode_stack([r, r], [ex, ex], [x, None], [y, y], chain=True)
    torch.cuda.synchronize()


@pytest.mark.parametrize("chain", [False, True])
def test_stack_fallback_shape(chain):
    """hidden 128: below what the single launch takes, so the stack runs one
    call per layer; the results equal the one-layer decode's bit for bit
    (chained: on the previous layer's y)."""
    E, H, I, K = 16, 128, 64, 4
    routers, banks, xs = [], [], []
    for li in range(3):
        L = layer(SEED + 11, synth.FAM_NVFP4, li, E, H, I, 1, K, "nvfp4")
        routers.append(upload_router(L["wg"], L["b"], K))
        banks.append(upload_bank(L["bank"], "nvfp4"))
        xs.append(L["x"][0])
    ys, ids, w = _run_stack(routers, banks, [xs[0]] + ([None] * 2 if chain else xs[1:]), H, K, chain=chain)
    for li in range(3):
        xin = xs[li] if not chain or li == 0 else ys[li - 1]
        one = run_decode(routers[li], banks[li], xin[None])
        assert np.array_equal(one["y"][0], ys[li]), f"layer {li}"
        assert np.array_equal(one["ids"][0], ids[li]), f"layer {li}"
