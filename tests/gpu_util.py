"""Host <-> device plumbing for the GPU tests (torch tensors only carry memory)."""
import numpy as np
import torch

import gemm_router_fp32_amd as g

DEV = "cuda"


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def host(t, dtype=None):
    a = t.detach().cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def upload_bank(bank, fmt):
    t = {k: dev(v) for k, v in bank.items()}
    if fmt == "nvfp4":
        ex = g.Experts(g.NVFP4, t["up_codes"], t["up_scales"], t["down_codes"], t["down_scales"],
                       t["up_gscale"], t["down_gscale"])
    else:
        ex = g.Experts(g.INT4_G64, t["up_codes"], t["up_scales"], t["down_codes"], t["down_scales"])
    return ex


def upload_router(wg, b, k):
    return g.Router(dev(wg), dev(b), k)


def run_decode(router, experts, x_np, ws=None):
    T = x_np.shape[0]
    x = dev(x_np)
    y = torch.empty((T, experts.hidden), dtype=torch.int16, device=DEV)
    ids = torch.empty((T, router.top_k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, router.top_k), dtype=torch.float32, device=DEV)
    ws = g.q4moe_w4a16_decode(router, experts, x, y, ids, w, ws=ws)
    torch.cuda.synchronize()
    taps = g.q4moe_w4a16_decode_taps(router, experts, T)
    wsh = host(ws)
    y32 = wsh[taps.y32: taps.y32 + T * experts.hidden * 4].view(np.float32).reshape(T, experts.hidden)
    return dict(y=host(y, np.uint16), ids=host(ids), w=host(w), y32=y32.copy(), ws=ws)


def run_entry(fn, router, experts, x_np, ws=None, shared=None):
    """y bf16 bits, ids, w of one call of a decode-family entry point."""
    T = x_np.shape[0]
    y = torch.empty((T, experts.hidden), dtype=torch.int16, device=DEV)
    ids = torch.empty((T, router.top_k), dtype=torch.int32, device=DEV)
    w = torch.empty((T, router.top_k), dtype=torch.float32, device=DEV)
    args = (router, experts) if shared is None else (router, experts, shared)
    ws = fn(*args, dev(x_np), y, ids, w, ws=ws)
    torch.cuda.synchronize()
    return dict(y=host(y, np.uint16), ids=host(ids), w=host(w), ws=ws)


def ws_view(ws_host, off, n, dt):
    return ws_host[off: off + n * np.dtype(dt).itemsize].view(dt).copy()


def run_w4a4_decode(router, experts, x_np, ws=None):
    """The one-token W4A4 decode and its taps."""
    o = run_entry(g.q4moe_w4a4_decode, router, experts, x_np, ws)
    tp = g.q4moe_w4a4_decode_taps(router, experts, 1)
    b = host(o["ws"])
    H, I, K = experts.hidden, experts.inter, router.top_k
    o.update(y32=ws_view(b, tp.y32, H, np.float32)[None],
             h32=ws_view(b, tp.h32, K * I, np.float32).reshape(K, I),
             xq_codes=ws_view(b, tp.xq_codes, H // 2, np.uint8)[None],
             xq_scales=ws_view(b, tp.xq_scales, H // 16, np.uint8)[None],
             hq_codes=ws_view(b, tp.hq_codes, K * I // 2, np.uint8).reshape(K, I // 2),
             hq_scales=ws_view(b, tp.hq_scales, K * I // 16, np.uint8).reshape(K, I // 16))
    return o


def run_gemv(qmat, x_np):
    T = x_np.shape[0]
    logits = torch.empty((T, qmat.rows), dtype=torch.float32, device=DEV)
    am = torch.empty(T, dtype=torch.int32, device=DEV)
    g.q4moe_w4a16_gemv(qmat, dev(x_np), logits, am)
    torch.cuda.synchronize()
    return host(logits), host(am)
