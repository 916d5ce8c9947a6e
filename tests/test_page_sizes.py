"""Shapes and storage formats against the sizes the source pages print
(tests/golden/page_sizes.txt, one citation per line)."""
import numpy as np

import synth


def _page():
    d = {}
    for line in open(__file__.replace("test_page_sizes.py", "golden/page_sizes.txt")):
        line = line.split("#")[0].strip()
        if line:
            k, v = line.split()
            d[k] = float(v)
    return d


P = _page()
H, I, E, L, V = 2688, 1856, 128, 23, 131072


def test_shapes_are_the_pages():
    assert (H, I, E, L, V) == (P["hidden"], P["inter"], P["experts"], P["layers"], P["vocab"])
    assert P["top_k"] == 6


def test_int4_routed_expert_bytes():
    # int4 group 64 with one 2-byte scale per group reproduces 15.61 GB, and
    # the bf16 source 58.75 GB, for 128 experts x 23 layers x (up + down).
    bank = synth.bank_arrays(1, H, I, "int4", alloc=np.empty)
    per_expert = sum(bank[k].nbytes for k in ("up_codes", "up_scales", "down_codes", "down_scales"))
    weights = 2 * H * I
    assert round(per_expert * E * L / 1e9, 2) == P["routed_int4_gb"]
    assert round(weights * 2 * E * L / 1e9, 2) == P["routed_bf16_gb"]
    assert E * L == P["down_tensors"] and 2 * E * L == P["routed_tensors"]
    assert I % 64 == 0 and I % 128 != 0  # group 128 does not divide the down input


def test_nvfp4_down_scale_view():
    bank = synth.bank_arrays(E, H, I, "nvfp4", alloc=np.empty)
    ds = bank["down_scales"]
    assert ds.reshape(-1, ds.shape[-1]).shape == (P["scale_view_rows"], P["scale_view_cols"])


def test_lm_head_sizes():
    params = V * H
    assert round(params / 1e6) == P["lm_params_m"]
    assert int(params * 2 / 1e6) == P["lm_bf16_mb"]
    assert int(params // 2 / 1e6) == P["lm_nvfp4_mb"]  # 4-bit codes, as the page counts
