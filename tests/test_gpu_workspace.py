"""One workspace shared by every entry point (the stacked decode among
them), and the one-launch decode's bounded waits.

Every workspace starts with the same prefix (control words and the
one-launch decode's epoch-tagged hand-off values) at fixed offsets, written
by the one-launch decode only.  These tests run one zero-filled workspace
through a sequence of entry points, token counts and paths, and check each
one-token result bit for bit against the same call on a fresh workspace.

The timeout test forces the one-launch decode's waits to give up from the
host: one workgroup's epoch copy in the control words is seeded apart from
the others, so that the workgroups of one call disagree on its epoch and
some hand-offs never match.  Every wait is bounded, so the kernel still
ends; the call returns OK and the workspace flag reports the expired
waits."""
import numpy as np
import pytest
import torch

import gemm_router_fp32_amd as g
import synth
from gpu_util import DEV, dev, host, upload_bank, upload_router
from inputs import SEED, layer, x_with_clear_routing

pytestmark = pytest.mark.gpu

E, H, I, K = 128, 2688, 1856, 6
FW_EPOCH = 256  # control word index of workgroup 0's epoch copy


@pytest.fixture(scope="module")
def full_layer():
    L = layer(SEED, synth.FAM_W4A4, 2, E, H, I, 8, K, "nvfp4", sigma_g=0.5 / np.sqrt(H))
    return L, upload_bank(L["bank"], "nvfp4"), upload_router(L["wg"], L["b"], K)


def _decode(fn, router, ex, x_np, ws):
    T = x_np.shape[0]
    y = torch.empty((T, H), dtype=torch.int16, device=DEV)
    ids = torch.empty((T, K), dtype=torch.int32, device=DEV)
    w = torch.empty((T, K), dtype=torch.float32, device=DEV)
    fn(router, ex, dev(x_np), y, ids, w, ws=ws)
    torch.cuda.synchronize()
    return host(y, np.uint16), host(ids), host(w)


def _big_ws(router, ex):
    n = max(g.q4moe_w4a4_moe_ws_bytes(router, ex, 8), g.q4moe_w4a16_decode_ws_bytes(router, ex, 4),
            g.q4moe_router_topk_ws_bytes(router, 37), g.q4moe_quantize_weights_ws_bytes(256, 2688),
            g.q4moe_w4a4_decode_ws_bytes(router, ex, 1))
    return g.workspace(n)


def _same(a, b):
    return all(np.array_equal(u, v) for u, v in zip(a, b))


def test_workspace_reuse_across_paths(full_layer):
    L, ex, router = full_layer
    x8, x1, x2 = L["x"], L["x"][:1], L["x"][:2]
    print("entry-point sequence on one workspace, full shapes", flush=True)
    ref_a4 = _decode(g.q4moe_w4a4_moe, router, ex, x1, None)       # fresh workspaces
    ref_a16 = _decode(g.q4moe_w4a16_decode, router, ex, x1, None)
    ws = _big_ws(router, ex)
    # W4A4: the grouped pipeline (8 tokens), then one token (one launch)
    _decode(g.q4moe_w4a4_moe, router, ex, x8, ws)
    assert _same(_decode(g.q4moe_w4a4_moe, router, ex, x1, ws), ref_a4)
    # W4A16: the small-batch kernels (2 tokens), then one token
    _decode(g.q4moe_w4a16_decode, router, ex, x2, ws)
    assert _same(_decode(g.q4moe_w4a16_decode, router, ex, x1, ws), ref_a16)
    # the router, the weight quantizer and the lm_head GEMV on the same
    # workspace, then one token again
    ids = torch.empty((37, K), dtype=torch.int32, device=DEV)
    w = torch.empty((37, K), dtype=torch.float32, device=DEV)
    xr = synth.x_rows(SEED, 9, 0, H, [0] * 37)
    g.q4moe_router_topk(router, dev(xr), ids, w, ws=ws)
    wb = synth.bf16_normal(synth.key(3, 4, 0, 0), 256 * H).reshape(256, H)
    codes = torch.empty((256, H // 2), dtype=torch.uint8, device=DEV)
    sc = torch.empty((256, H // 16), dtype=torch.uint8, device=DEV)
    gs = torch.empty(1, dtype=torch.float32, device=DEV)
    g.q4moe_quantize_weights(dev(wb), codes, sc, gs, mode=g.WQ_MSE, ws=ws)
    logits = torch.empty((2, 256), dtype=torch.float32, device=DEV)
    g.q4moe_w4a16_gemv(g.QMat(g.NVFP4, codes, sc, gs), dev(x2), logits, torch.empty(2, dtype=torch.int32,
                                                                                     device=DEV), ws=ws)
    torch.cuda.synchronize()
    assert _same(_decode(g.q4moe_w4a16_decode, router, ex, x1, ws), ref_a16)
    assert _same(_decode(g.q4moe_w4a4_decode, router, ex, x1, ws), ref_a4)
    # the stacked decode (three layers sharing the bank, inputs rows 0-2),
    # each layer equal to its one-token call on a fresh workspace, then one
    # token again
    xs = [dev(L["x"][i]) for i in range(3)]
    ys = [torch.empty(H, dtype=torch.int16, device=DEV) for _ in range(3)]
    g.q4moe_w4a16_decode_stack([router] * 3, [ex] * 3, xs, ys, ws=ws)
    torch.cuda.synchronize()
    for i in range(3):
        one = _decode(g.q4moe_w4a16_decode, router, ex, L["x"][i:i + 1], None)
        assert np.array_equal(host(ys[i], np.uint16), one[0][0]), f"stacked layer {i}"
    assert _same(_decode(g.q4moe_w4a16_decode, router, ex, x1, ws), ref_a16)
    assert g.q4moe_ws_check(ws) == 0


def test_decode_bounded_waits_forced_from_host(full_layer):
    L, ex, router = full_layer
    x1 = L["x"][:1]
    ref = _decode(g.q4moe_w4a16_decode, router, ex, x1, None)
    ws = g.workspace(g.q4moe_w4a16_decode_ws_bytes(router, ex, 1))
    # epoch copies that disagree: workgroup 0 takes epoch 1001, the others
    # epoch 1, so hand-offs between workgroup 0 and the others never match
    # and those waits expire (each after its bounded count)
    ctrl = ws[:4096].view(torch.int32)
    ctrl[FW_EPOCH] = 1000
    torch.cuda.synchronize()
    print("one-launch decode with inconsistent epoch copies (waits expire by design)", flush=True)
    _decode(g.q4moe_w4a16_decode, router, ex, x1, ws)  # returns: every wait is bounded
    assert g.q4moe_ws_check(ws) & 1, "expired waits are reported through the workspace flag"
    # a workspace disturbed this way is re-initialised; then calls are correct
    g.q4moe_ws_init(ws)
    assert _same(_decode(g.q4moe_w4a16_decode, router, ex, x1, ws), ref)
    assert g.q4moe_ws_check(ws) == 0


@pytest.mark.parametrize("variant", ["w4a16", "int4", "w4a4", "shared", "w4a4_shared"])
def test_one_launch_repeated_calls(variant):
    # every call of the one-launch decode advances the epoch of each of its
    # workgroups; repeated calls on one workspace and on fresh workspaces
    # must all finish within their waits and agree bit for bit
    fmt = "int4" if variant == "int4" else "nvfp4"
    fam = synth.FAM_INT4 if fmt == "int4" else synth.FAM_W4A4
    L = layer(SEED + 3, fam, 4, 16, H, I, 1, K, fmt)
    ex, router = upload_bank(L["bank"], fmt), upload_router(L["wg"], L["b"], K)
    args, fn, wsb = (), g.q4moe_w4a16_decode, g.q4moe_w4a16_decode_ws_bytes
    if variant in ("shared", "w4a4_shared"):
        sh = synth.shared_fp8(SEED, 3, 4, H, 512)
        shd = g.SharedFp8(dev(sh["up_codes"]), dev(sh["down_codes"]), sh["up_wscale"], sh["up_iscale"],
                          sh["down_wscale"], sh["down_iscale"])
        args = (shd,)
        fn = g.q4moe_w4a16_decode_shared if variant == "shared" else g.q4moe_w4a4_decode_shared
        wsb = g.q4moe_w4a16_decode_shared_ws_bytes if variant == "shared" else g.q4moe_w4a4_decode_shared_ws_bytes
    elif variant == "w4a4":
        fn, wsb = g.q4moe_w4a4_decode, g.q4moe_w4a4_decode_ws_bytes
    x = dev(L["x"])

    def call(ws):
        y = torch.empty((1, H), dtype=torch.int16, device=DEV)
        fn(router, ex, *args, x, y, ws=ws)
        torch.cuda.synchronize()
        assert g.q4moe_ws_check(ws) == 0, "a bounded wait expired"
        return host(y, np.uint16)

    print(f"{variant}: 12 calls on one workspace, 4 on fresh ones", flush=True)
    ws = g.workspace(wsb(router, ex, *args, 1))
    first = call(ws)
    for _ in range(11):
        assert np.array_equal(call(ws), first)
    for _ in range(4):
        assert np.array_equal(call(g.workspace(wsb(router, ex, *args, 1))), first)
