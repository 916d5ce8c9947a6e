"""Oracle router (fp32 router compute, sigmoid scores, bias used only to
select, top-k with lowest-index ties, renormalised gates), pinned by brute
force, invariants and sigmoid values with closed forms."""
import math

import numpy as np

import oracle
import synth
from q4moe_testutil import bf16_bits_to_f64


def _inputs(T=5, E=128, H=2688, seed=7):
    wg, b = synth.router(seed, synth.FAM_NVFP4, 0, E, H)
    x = synth.x_rows(seed, synth.FAM_NVFP4, 0, H, [0] * T)
    return wg, b, x


def test_router_brute_force():
    wg, b, x = _inputs()
    r = oracle.router(wg, b, x, 6)
    logits = bf16_bits_to_f64(x) @ wg.astype(np.float64).T
    np.testing.assert_allclose(r["logits"], logits, rtol=1e-12, atol=1e-12)
    s = 1.0 / (1.0 + np.exp(-logits))
    for t in range(x.shape[0]):
        key = r["scores"][t] + b.astype(np.float64)
        order = np.lexsort((np.arange(128), -key))
        assert list(r["ids"][t]) == list(order[:6])
        assert abs(r["w"][t].sum() - 1.0) < 1e-15
        np.testing.assert_allclose(r["w"][t], s[t, order[:6]] / s[t, order[:6]].sum(), rtol=1e-12)
        assert r["gap"][t] == key[order[5]] - key[order[6]]


def test_router_ties_go_to_lower_index():
    E, H = 16, 32
    wg = np.zeros((E, H), np.float32)
    b = np.zeros(E, np.float32)
    x = np.full((1, H), 0x3F80, np.uint16)  # x = 1
    r = oracle.router(wg, b, x, 4)
    assert list(r["ids"][0]) == [0, 1, 2, 3]
    b[9] = 1e-3
    b[12] = 1e-3
    r = oracle.router(wg, b, x, 4)
    assert list(r["ids"][0]) == [9, 12, 0, 1]
    np.testing.assert_array_equal(r["w"][0], [0.25] * 4)  # bias does not enter the gates


def test_router_sigmoid_closed_forms():
    # logit 0 -> score 1/2; logit ln 3 -> 3/4; logit -ln 3 -> 1/4
    E, H = 4, 16
    wg = np.zeros((E, H), np.float32)
    wg[1, 0] = np.float32(math.log(3.0))
    wg[2, 0] = np.float32(-math.log(3.0))
    b = np.array([0.0, 0.0, 0.0, -1.0], np.float32)
    x = np.zeros((1, H), np.uint16)
    x[0, 0] = 0x3F80
    r = oracle.router(wg, b, x, 3)
    assert r["scores"][0, 0] == 0.5
    assert abs(r["scores"][0, 1] - 0.75) < 1e-7 and abs(r["scores"][0, 2] - 0.25) < 1e-7
    assert list(r["ids"][0]) == [1, 0, 2]
    np.testing.assert_allclose(r["w"][0], [0.5, 1 / 3, 1 / 6], rtol=1e-6)


def test_router_invariants():
    wg, b, x = _inputs(T=3)
    r0 = oracle.router(wg, b, x, 6)
    # a constant shift of every bias leaves the selection and the gates unchanged
    r1 = oracle.router(wg, b + np.float32(0.25), x, 6)
    assert np.array_equal(r0["ids"], r1["ids"])
    np.testing.assert_allclose(r0["w"], r1["w"], rtol=0, atol=0)
    # relabelling experts (router rows and biases together) relabels the ids
    perm = np.random.default_rng(1).permutation(128)
    r2 = oracle.router(wg[perm], b[perm], x, 6)
    assert np.array_equal(perm[r2["ids"]], r0["ids"])
    np.testing.assert_array_equal(r2["w"], r0["w"])
    # top_k = E selects everything and gates equal scores / sum(scores)
    r3 = oracle.router(wg[:8], b[:8], x, 8)
    assert sorted(r3["ids"][0]) == list(range(8))
