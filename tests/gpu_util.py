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
