"""Benchmark: batch-1 routed-MoE decode through a 23-layer NVFP4 W4A16 stack.

One step = one token through 23 independent routed-MoE layers (hidden 2688,
expert intermediate 1856, 128 experts, top-6), each layer a router top-6,
up GEMV, relu^2, down GEMV and weighted combine in one launch, run one after
another on one stream.  The stack is captured once in a HIP graph and
replayed.  Inputs are seeded synthetic tensors resident in HBM before timing
starts.

Prints one JSON line: microseconds per layer (the metric) and achieved HBM
bandwidth against MI355X's 8 TB/s; the decode kernel's own duration (HIP
events around single launches) for the roofline; the other workloads (the
int4 group-64 stack, the W4A4 1024-token chunk, the four-token verify step
with the lm_head) as extra fields; and the oracle's CPU time on a bounded
sample of the same workload.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

H, I, E, K, LAYERS, V = 2688, 1856, 128, 6, 23, 131072
S_SHARED = 3712  # shared expert intermediate size (2 x 1856; derived from the checkpoint table's shared-expert bytes)
SEED = 20261202
PEAK_HBM_GBS = 8000.0
PEAK_F16_TFLOPS = 2500.0   # dense fp16/bf16 MFMA
TRAFFIC_PROFILE = "profiles/traffic_k_decode_nvfp4_stack.md"
PHASE_PROFILE = "profiles/k_decode_stack_phase_timeline_nvfp4.md"
MFMA_PROFILE = "profiles/k_grouped_gemm_mfma_counters_w4a4_1024.md"
METRIC = "µs per routed-MoE layer at batch 1 + achieved HBM GB/s (% of MI355X peak)"


def expert_bytes(fmt):
    """Codes + block scales (+ fp32 per-tensor scales) of one expert."""
    if fmt == "nvfp4":
        return 2 * (H * I // 2 + H * I // 16 + 4)
    return 2 * (H * I // 2 + H * I // 64 * 2)


def layer_bytes(fmt="nvfp4", n_experts_read=K, T=1):
    """Algorithmic HBM bytes of one decode layer: the selected experts'
    weights, the fp32 router (W_g and bias), x and y (bf16)."""
    return n_experts_read * expert_bytes(fmt) + E * H * 4 + E * 4 + T * H * 2 * 2


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="bound on the oracle CPU sample")
    ap.add_argument("--skip-cpu", action="store_true")
    ap.add_argument("--only-stack", action="store_true", help="time the NVFP4 decode stack only")
    ap.add_argument("--only-w4a4-chunk", action="store_true",
                    help="run the W4A4 1024-token chunk only (for counter passes); prints its dict")
    return ap.parse_args()


class Timer:
    def __init__(self, torch):
        self.torch = torch

    def __call__(self, fn, reps):
        t = self.torch
        e0, e1 = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        t.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        t.cuda.synchronize()
        return e0.elapsed_time(e1) / reps  # ms

    def each(self, fn, reps, before=None):
        """Per-rep times (ms) from events around each call; `before` runs
        untimed ahead of every rep (e.g. an eviction of the MALL)."""
        t = self.torch
        evs = [(t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)) for _ in range(reps)]
        t.cuda.synchronize()
        for a, b in evs:
            if before is not None:
                before()
            a.record()
            fn()
            b.record()
        t.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in evs])


def spread(ms, scale=1e3, nd=3):
    """median / p10 / p90 of per-rep times, scaled (default ms -> us)."""
    q = np.percentile(np.asarray(ms) * scale, [50, 10, 90])
    return {"median": round(float(q[0]), nd), "p10": round(float(q[1]), nd), "p90": round(float(q[2]), nd)}


class Evictor:
    """Reads 1 GiB so that nothing a timed rep reads is still held in the
    256 MB MALL or the L2s.  The eviction only reads: it leaves clean lines
    behind, as the small activation writes before a decode step would, so
    the timed rep does not pay for writing back the evictor's own data (a
    512 MiB copy as the eviction left the caches dirty and cost the
    lm_head ~10 us of write-backs)."""

    def __init__(self, torch):
        self.buf = torch.ones(1 << 27, dtype=torch.int64, device="cuda")
        torch.cuda.synchronize()

    def __call__(self):
        self.buf.sum()


def build_stack(torch, g, synth, fmt, shared=False, w4a4=False, n_tok=1):
    """The 23 layers, resident; with `shared`, each layer also carries the
    FP8 shared expert [S_SHARED x H] and runs the shared decode entry; with
    `w4a4`, each layer runs the single-token W4A4 decode entry; `n_tok`
    tokens per call."""
    from gpu_util import dev
    fam = synth.FAM_NVFP4 if fmt == "nvfp4" else synth.FAM_INT4
    layers, buf = [], None
    for li in range(LAYERS):
        bank = synth.expert_bank(SEED, fam, li, E, H, I, fmt, out=buf)
        buf = bank
        wg, b = synth.router(SEED, fam, li, E, H)
        x = synth.x_rows(SEED, fam, li, H, list(range(n_tok)))
        t = {k: dev(v) for k, v in bank.items()}
        if fmt == "nvfp4":
            ex = g.Experts(g.NVFP4, t["up_codes"], t["up_scales"], t["down_codes"], t["down_scales"],
                           t["up_gscale"], t["down_gscale"])
        else:
            ex = g.Experts(g.INT4_G64, t["up_codes"], t["up_scales"], t["down_codes"], t["down_scales"])
        r = g.Router(dev(wg), dev(b), K)
        L = dict(ex=ex, r=r, x=dev(x), y=torch.empty((n_tok, H), dtype=torch.int16, device="cuda"))
        L["w4a4"] = w4a4
        if shared:
            sh = synth.shared_fp8(SEED, fam, li, H, S_SHARED)
            L["sh"] = g.SharedFp8(dev(sh["up_codes"]), dev(sh["down_codes"]), sh["up_wscale"], sh["up_iscale"],
                                  sh["down_wscale"], sh["down_iscale"])
            wsb = (g.q4moe_w4a4_decode_shared_ws_bytes if w4a4 else g.q4moe_w4a16_decode_shared_ws_bytes)(
                r, ex, L["sh"], n_tok)
        else:
            wsb = (g.q4moe_w4a4_decode_ws_bytes if w4a4 else g.q4moe_w4a16_decode_ws_bytes)(r, ex, n_tok)
        L["ws"] = g.workspace(wsb)
        layers.append(L)
    log(f"{fmt} stack{' + shared expert' if shared else ''}{' (W4A4)' if w4a4 else ''} resident ({LAYERS} layers)")
    return layers


def decode_call(g, L):
    if L["w4a4"] and "sh" in L:
        g.q4moe_w4a4_decode_shared(L["r"], L["ex"], L["sh"], L["x"], L["y"], ws=L["ws"])
    elif L["w4a4"]:
        g.q4moe_w4a4_decode(L["r"], L["ex"], L["x"], L["y"], ws=L["ws"])
    elif "sh" in L:
        g.q4moe_w4a16_decode_shared(L["r"], L["ex"], L["sh"], L["x"], L["y"], ws=L["ws"])
    else:
        g.q4moe_w4a16_decode(L["r"], L["ex"], L["x"], L["y"], ws=L["ws"])


def time_stack(torch, g, layers, steps, warmup):
    stream = torch.cuda.current_stream()

    def step():
        for L in layers:
            decode_call(g, L)

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(stream)
    with torch.cuda.stream(s):
        step()
    stream.wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for _ in range(warmup):
        graph.replay()
    # events between consecutive replays: the K steps form one contiguous region
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for i in range(steps):
        graph.replay()
        evs[i + 1].record()
    torch.cuda.synchronize()
    per = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(steps)])
    ms_step = evs[0].elapsed_time(evs[-1]) / steps
    # the kernel's own duration: events just around single launches
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    durs = []
    for rep in range(4):
        for L in layers:
            e0.record()
            decode_call(g, L)
            e1.record()
            e1.synchronize()
            durs.append(e0.elapsed_time(e1))
    flags = max(g.q4moe_ws_check(L["ws"]) for L in layers)
    return ms_step, float(np.mean(durs[LAYERS:])), flags, per


def stack_launch_step(g, layers):
    """One call of q4moe_w4a16_decode_stack over the layers, and its workspace."""
    routers = [L["r"] for L in layers]
    banks = [L["ex"] for L in layers]
    xs = [L["x"][0] for L in layers]
    ys = [L["y"][0] for L in layers]
    ws = g.workspace(g.q4moe_w4a16_decode_stack_ws_bytes(routers[0], banks[0]))

    def step():
        g.q4moe_w4a16_decode_stack(routers, banks, xs, ys, ws=ws)
    return step, ws


def time_stack_launch(torch, g, layers, steps, warmup):
    """The same 23 layers through q4moe_w4a16_decode_stack: one launch per
    step, each layer starting its routing once the previous layer's y is
    complete (the order of the per-layer graph, without its launch gaps)."""
    step, ws = stack_launch_step(g, layers)

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(stream)
    with torch.cuda.stream(s):
        step()
    stream.wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for _ in range(warmup):
        graph.replay()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for i in range(steps):
        graph.replay()
        evs[i + 1].record()
    torch.cuda.synchronize()
    per = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(steps)])
    ms_step = evs[0].elapsed_time(evs[-1]) / steps
    return ms_step, g.q4moe_ws_check(ws), per


def bench_w4a4(torch, g, synth, steps):
    from gpu_util import dev
    T = 1024
    bank = synth.expert_bank(SEED, synth.FAM_W4A4, 0, E, H, I, "nvfp4")
    wg, b = synth.router(SEED, synth.FAM_W4A4, 0, E, H, 0.5 / np.sqrt(H))
    x = synth.x_rows(SEED, synth.FAM_W4A4, 0, H, [0] * T)
    t = {k: dev(v) for k, v in bank.items()}
    ex = g.Experts(g.NVFP4, t["up_codes"], t["up_scales"], t["down_codes"], t["down_scales"],
                   t["up_gscale"], t["down_gscale"])
    r = g.Router(dev(wg), dev(b), K)
    xt = dev(x)
    y = torch.empty((T, H), dtype=torch.int16, device="cuda")
    ids = torch.empty((T, K), dtype=torch.int32, device="cuda")
    w = torch.empty((T, K), dtype=torch.float32, device="cuda")
    ws = g.workspace(g.q4moe_w4a4_grouped_ws_bytes(r, ex, T))

    def run():
        g.q4moe_w4a4_grouped(r, ex, xt, y, ids, w, ws=ws)

    for _ in range(3):
        run()
    # 718 MB of weights per chunk exceed the 256 MB MALL: every rep streams from HBM
    per = Timer(torch).each(run, max(5, steps // 5))
    ms = float(np.median(per))
    weights = E * expert_bytes("nvfp4")
    flops = 2.0 * 2 * T * K * H * I
    byts = weights + E * H * 4 + 2 * T * H * 2
    log(f"w4a4 chunk: {ms * 1e3:.1f} us")
    return {"us": round(ms * 1e3, 2), "hbm_gbps": round(byts / (ms * 1e-3) / 1e9, 1),
            "tflops": round(flops / (ms * 1e-3) / 1e12, 2),
            "mfma_frac_of_fp16_peak": round(flops / (ms * 1e-3) / 1e12 / PEAK_F16_TFLOPS, 4),
            # MFMA pipe busy (counters, the committed profile of the grouped GEMMs)
            "mfma_busy_frac_counters": read_profile_value(os.path.join(ROOT, MFMA_PROFILE), "mfma_busy_frac",
                                                          ("csrc/q4moe_w4a4.hpp", "csrc/q4moe_device.hpp",
                                                           "csrc/q4moe_kernels.hpp")),
            "us_spread": spread(per), "bytes": byts, "flop": flops, "tokens": T}


def bench_verify(torch, g, synth, steps, stack_layer0):
    """Four tokens through one NVFP4 layer, then the NVFP4 lm_head over them."""
    from gpu_util import dev
    L = stack_layer0
    x4 = dev(synth.x_rows(SEED, synth.FAM_NVFP4, 0, H, [0] * 4))
    y4 = torch.empty((4, H), dtype=torch.int16, device="cuda")
    ws4 = g.workspace(g.q4moe_w4a16_decode_ws_bytes(L["r"], L["ex"], 4))
    ids4 = torch.empty((4, K), dtype=torch.int32, device="cuda")
    codes, scales, gsc = synth.lm_head(SEED, 0, 0, V, H)
    q = g.QMat(g.NVFP4, dev(codes), dev(scales), dev(np.array([gsc], np.float32)))
    logits = torch.empty((4, V), dtype=torch.float32, device="cuda")
    am = torch.empty(4, dtype=torch.int32, device="cuda")
    wsl = g.workspace(g.q4moe_w4a16_gemv_ws_bytes(q, 4))

    def moe():
        g.q4moe_w4a16_decode(L["r"], L["ex"], x4, y4, ids=ids4, ws=ws4)

    def head():
        g.q4moe_w4a16_gemv(q, y4, logits, am, ws=wsl)

    for _ in range(3):
        moe()
        head()
    # cold reps: the lm_head (198 MB) and the 4 tokens' experts fit in the MALL
    timer, evict = Timer(torch), Evictor(torch)
    reps = max(10, steps // 2)
    t_moe = timer.each(moe, reps, evict)
    t_head = timer.each(head, reps, evict)
    ms_moe, ms_head = float(np.median(t_moe)), float(np.median(t_head))
    n_union = len(np.unique(ids4.cpu().numpy()))
    moe_bytes = layer_bytes("nvfp4", n_union, 4)
    head_bytes = V * H // 2 + V * H // 16 + 4 + 4 * H * 2 + 4 * V * 4
    return {"moe_us": round(ms_moe * 1e3, 2), "moe_hbm_gbps": round(moe_bytes / (ms_moe * 1e-3) / 1e9, 1),
            "moe_us_spread": spread(t_moe), "experts_read": n_union,
            "lm_head_us": round(ms_head * 1e3, 2),
            "lm_head_hbm_gbps": round(head_bytes / (ms_head * 1e-3) / 1e9, 1),
            "lm_head_us_spread": spread(t_head), "cold": True, "reps": reps}


def bench_spec_step(torch, g, synth, steps):
    """One speculative decode step through one MoE layer (tests/spec_step.py):
    three drafter passes (W4A4 NVFP4 MoE on one token, FP8 lm_head GEMV +
    argmax), then the 4-token W4A16 NVFP4 verify MoE and the NVFP4 lm_head,
    captured as one graph and replayed cold (1 GiB read before each
    replay); the eager step and each stage are timed cold beside it."""
    from spec_step import DRAFT_LAYER, SpecStep
    st = SpecStep(torch, g, synth, SEED, x0=synth.x_rows(SEED, synth.FAM_W4A4, DRAFT_LAYER, H, [0])[0])
    for _ in range(3):
        st.step()
    graph = st.capture()
    timer, evict = Timer(torch), Evictor(torch)
    reps = max(10, steps // 2)
    t_graph = timer.each(graph.replay, reps, evict)
    t_eager = timer.each(st.step, reps, evict)
    t_draft = timer.each(lambda: st.draft(1), reps, evict)
    t_moe = timer.each(lambda: g.q4moe_w4a4_decode(st.drouter, st.dex, st.xv[0:1], st.xv[1:2], st.d_ids[0:1],
                                                   st.d_w[0:1], ws=st.d_ws[0]), reps, evict)
    t_fp8 = timer.each(lambda: g.q4moe_fp8_gemv(st.fp8, st.xv[1:2], st.d_logits[0:1], st.d_am[0:1], ws=st.f_ws[0]),
                       reps, evict)
    t_verify = timer.each(st.verify, reps, evict)
    fp8_bytes = V * H + H * 2 + V * 4
    out = {"graph_step_us": round(float(np.median(t_graph)) * 1e3, 2), "graph_step_us_spread": spread(t_graph),
           "eager_step_us": round(float(np.median(t_eager)) * 1e3, 2),
           "draft_pass_us": round(float(np.median(t_draft)) * 1e3, 2),
           "draft_moe_w4a4_us": round(float(np.median(t_moe)) * 1e3, 2),
           "draft_lm_head_fp8_us": round(float(np.median(t_fp8)) * 1e3, 2),
           "draft_lm_head_fp8_hbm_gbps": round(fp8_bytes / (float(np.median(t_fp8)) * 1e-3) / 1e9, 1),
           "verify_us": round(float(np.median(t_verify)) * 1e3, 2),
           "kernels_per_step": 3 * 3 + 4 + 2, "cold": True, "reps": reps}
    del graph, st
    torch.cuda.empty_cache()
    log(f"speculative step: {out}")
    return out


def bench_wquant(torch, g, synth, steps):
    """NVFP4 weight quantizer on one expert's up_proj (1856 x 2688 bf16):
    µs per matrix in both scale modes; bytes = bf16 in + codes and scales out."""
    from gpu_util import dev
    w = dev(synth.bf16_normal(synth.key(SEED, 4, 0, 0), I * H, 0.0, 0.02).reshape(I, H))
    codes = torch.empty((I, H // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((I, H // 16), dtype=torch.uint8, device="cuda")
    gs = torch.empty(1, dtype=torch.float32, device="cuda")
    ws = g.workspace(g.q4moe_quantize_weights_ws_bytes(I, H))
    nbytes = I * H * 2 + I * H // 2 + I * H // 16 + 4
    out = {"matrix": [I, H], "bytes": nbytes, "warm": True}
    for name, mode in (("max", g.WQ_MAX), ("mse", g.WQ_MSE)):
        for _ in range(3):
            g.q4moe_quantize_weights(w, codes, scales, gs, mode=mode, ws=ws)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = max(5, steps // 5)
        e0.record()
        for _ in range(reps):
            g.q4moe_quantize_weights(w, codes, scales, gs, mode=mode, ws=ws)
        e1.record()
        torch.cuda.synchronize()
        us = 1000.0 * e0.elapsed_time(e1) / reps
        out[f"{name}_us"] = round(us, 2)
        out[f"{name}_gbps"] = round(nbytes / (us * 1e-6) / 1e9, 1)
    log(f"weight quantizer: {out}")
    return out


MID_COUNTS = (1, 2, 3, 4, 5, 8, 16, 32, 64, 128, 256)


def bench_mid_batch(torch, g, synth, steps, fmt, layer=None):
    """One routed-MoE layer (full shapes) at T tokens, cold (1 GiB read
    before every rep, so no weight is left in the MALL or the L2s): µs per
    call through the decode entry point (which picks its path by T) and
    through the grouped path, the experts the T tokens select, and the HBM
    rate of the decode entry on their weights.  fmt "nvfp4" / "int4": the
    W4A16 entries on the stack's first layer; "w4a4": q4moe_w4a4_moe (one
    single-token launch per token up to Q4MOE_W4A4_PER_TOKEN_MAX_TOKENS),
    q4moe_w4a4_decode (one launch for one token, the one-pass small-batch
    kernels for 2-8) and q4moe_w4a4_grouped on a bank routed with logits ~N(0, 0.5^2)."""
    from gpu_util import dev
    fam = {"nvfp4": synth.FAM_NVFP4, "int4": synth.FAM_INT4, "w4a4": synth.FAM_W4A4}[fmt]
    if fmt == "w4a4":
        bank = synth.expert_bank(SEED, fam, 1, E, H, I, "nvfp4")
        t = {k: dev(v) for k, v in bank.items()}
        ex = g.Experts(g.NVFP4, t["up_codes"], t["up_scales"], t["down_codes"], t["down_scales"],
                       t["up_gscale"], t["down_gscale"])
        wg, b = synth.router(SEED, fam, 1, E, H, 0.5 / np.sqrt(H))
        r = g.Router(dev(wg), dev(b), K)
        entry, entry_ws = g.q4moe_w4a4_moe, g.q4moe_w4a4_moe_ws_bytes
        grouped, grouped_ws = g.q4moe_w4a4_grouped, g.q4moe_w4a4_grouped_ws_bytes
    else:
        ex, r = layer["ex"], layer["r"]
        entry, entry_ws = g.q4moe_w4a16_decode, g.q4moe_w4a16_decode_ws_bytes
        grouped, grouped_ws = g.q4moe_w4a16_grouped, g.q4moe_w4a16_grouped_ws_bytes
    timer, evict = Timer(torch), Evictor(torch)
    reps = max(5, steps // 10)
    out = {"cold": True, "reps": reps, "decode_us": {}, "grouped_us": {}, "decode_us_per_token": {},
           "experts_read": {}, "decode_hbm_gbps": {}}
    if fmt == "w4a4":
        out["one_pass_small_us"] = {}
    for T in MID_COUNTS:
        x = dev(synth.x_rows(SEED, fam, 1, H, [0] * T))
        y = torch.empty((T, H), dtype=torch.int16, device="cuda")
        ids = torch.empty((T, K), dtype=torch.int32, device="cuda")
        w = torch.empty((T, K), dtype=torch.float32, device="cuda")
        need = max(entry_ws(r, ex, T), grouped_ws(r, ex, T))
        if fmt == "w4a4" and T <= 8:
            need = max(need, g.q4moe_w4a4_decode_ws_bytes(r, ex, T))
        ws = g.workspace(need)
        calls = {"decode_us": lambda: entry(r, ex, x, y, ids, w, ws=ws),
                 "grouped_us": lambda: grouped(r, ex, x, y, ids, w, ws=ws)}
        if fmt == "w4a4" and T <= 8:
            calls["one_pass_small_us"] = lambda: g.q4moe_w4a4_decode(r, ex, x, y, ids, w, ws=ws)
        for name, fn in calls.items():
            fn()
            out[name][T] = round(float(np.median(timer.each(fn, reps, evict))) * 1e3, 2)
        n = len(np.unique(ids.cpu().numpy()))
        out["experts_read"][T] = n
        out["decode_us_per_token"][T] = round(out["decode_us"][T] / T, 2)
        nbytes = layer_bytes("int4" if fmt == "int4" else "nvfp4", n, T)
        out["decode_hbm_gbps"][T] = round(nbytes / (out["decode_us"][T] * 1e-6) / 1e9, 1)
        del ws
    log(f"mid-batch {fmt}: {out}")
    return out


def cpu_model():
    """The host CPU's model name and the cores this process may use."""
    name = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                name = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return name, len(os.sched_getaffinity(0))


def cpu_baseline(seconds, threads=None):
    """The oracle, as it stands, on layers of the NVFP4 stack until `seconds`
    of CPU work have run (with `threads` OpenMP threads, default: all);
    returns microseconds per layer, layers run and threads used."""
    import oracle
    import synth
    if threads is not None:
        oracle.set_threads(threads)
    done, t_total = 0, 0.0
    for li in range(LAYERS):
        wg, b = synth.router(SEED, synth.FAM_NVFP4, li, E, H)
        x = synth.x_rows(SEED, synth.FAM_NVFP4, li, H, [0])
        t0 = time.perf_counter()
        r = oracle.router(wg, b, x, K)
        t_total += time.perf_counter() - t0
        bank = synth.expert_bank(SEED, synth.FAM_NVFP4, li, E, H, I, "nvfp4", experts=r["ids"][0])
        ob = oracle.Bank.from_dict(oracle.NVFP4, bank)
        t0 = time.perf_counter()
        oracle.moe_w4a16(ob, x, r["ids"], r["w"])
        t_total += time.perf_counter() - t0
        done += 1
        if t_total >= seconds:
            break
    return 1e6 * t_total / done, done, oracle.threads()


def read_profile_value(path, key, sources=None):
    """A `key=value` line of a committed profile summary, with the kernel
    source hash it was measured on (None once the sources have changed)."""
    from gemm_router_fp32_amd.pmc_traffic import KERNEL_SOURCES, source_sha256
    if not os.path.exists(path):
        return None
    val, sha = None, None
    for line in open(path):
        line = line.strip().strip("`")
        if line.startswith(key + "="):
            val = float(line.split("=", 1)[1])
        if line.startswith("source_sha256="):
            sha = line.split("=", 1)[1]
    return val if (val is not None and sha == source_sha256(sources or KERNEL_SOURCES)) else None


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    import gemm_router_fp32_amd as g
    import synth

    torch.cuda.set_device(0)
    g.lib()
    if args.only_w4a4_chunk:
        src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
        torch.empty_like(src).copy_(src)  # the copy that calibrates the traffic counters
        print(json.dumps(bench_w4a4(torch, g, synth, args.steps)), flush=True)
        return
    # a plain copy of known size (256 MiB), to scale HBM traffic counters
    src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()

    layers = build_stack(torch, g, synth, "nvfp4")
    bytes_layer = layer_bytes()
    # the step: the 23 layers in one stacked launch (k_decode_stack), each
    # layer's routing starting once the previous layer's y is complete
    ms_step, flags, per_step = time_stack_launch(torch, g, layers, args.steps, args.warmup)
    us_layer = 1000.0 * ms_step / LAYERS
    gbs = bytes_layer / (us_layer * 1e-6) / 1e9
    log(f"nvfp4 stack, one launch: {ms_step:.4f} ms/step, {us_layer:.3f} us/layer, {gbs:.1f} GB/s; flags {flags}")
    # the same layers as a graph of one k_decode_fused launch per layer
    ms_g, ms_kernel, f_g, per_g = time_stack(torch, g, layers, args.steps, args.warmup)
    graph_nv = {"us_per_layer": round(1000.0 * ms_g / LAYERS, 3),
                "hbm_gbps": round(bytes_layer / (ms_g / LAYERS * 1e-3) / 1e9, 1),
                "tokens_per_s": round(1000.0 / ms_g, 1), "us_per_layer_spread": spread(per_g / LAYERS),
                "single_launch_us": round(ms_kernel * 1e3, 3), "flags": f_g}
    log(f"nvfp4 stack, graph of one launch per layer: {graph_nv}")
    # one layer alone, cold: 1 GiB read before each rep evicts the MALL and L2s
    t_cold = Timer(torch).each(lambda: decode_call(g, layers[0]), max(10, args.steps // 2), Evictor(torch))
    single_cold_us = float(np.median(t_cold)) * 1e3
    log(f"single layer, evicted, direct launch: {single_cold_us:.2f} us")

    extra = {"nvfp4_graph_of_launches": graph_nv}
    if not args.only_stack:
        extra["verify_step"] = bench_verify(torch, g, synth, args.steps, layers[0])
        log(f"verify step: {extra['verify_step']}")
        extra["mid_batch_nvfp4"] = bench_mid_batch(torch, g, synth, args.steps, "nvfp4", layers[0])
        del layers
        torch.cuda.empty_cache()
        int4 = build_stack(torch, g, synth, "int4")
        b4 = layer_bytes("int4")
        ms41, f41, per41 = time_stack_launch(torch, g, int4, args.steps, args.warmup)
        extra["int4_stack"] = {"us_per_layer": round(1000.0 * ms41 / LAYERS, 3),
                               "hbm_gbps": round(b4 / (ms41 / LAYERS * 1e-3) / 1e9, 1),
                               "tokens_per_s": round(1000.0 / ms41, 1), "us_per_layer_spread": spread(per41 / LAYERS),
                               "bytes_per_layer": b4, "launch": "one stacked launch", "flags": f41}
        log(f"int4 stack, one launch: {extra['int4_stack']}")
        ms4, mk4, f4, per4 = time_stack(torch, g, int4, args.steps, args.warmup)
        extra["int4_graph_of_launches"] = {"us_per_layer": round(1000.0 * ms4 / LAYERS, 3),
                                           "hbm_gbps": round(b4 / (ms4 / LAYERS * 1e-3) / 1e9, 1),
                                           "tokens_per_s": round(1000.0 / ms4, 1),
                                           "single_launch_us": round(mk4 * 1e3, 3),
                                           "us_per_layer_spread": spread(per4 / LAYERS), "flags": f4}
        log(f"int4 stack, graph of one launch per layer: {extra['int4_graph_of_launches']}")
        extra["mid_batch_int4"] = bench_mid_batch(torch, g, synth, args.steps, "int4", int4[0])
        del int4
        torch.cuda.empty_cache()
        shl = build_stack(torch, g, synth, "nvfp4", shared=True)
        mss, mks, fs, pers = time_stack(torch, g, shl, args.steps, args.warmup)
        bs = layer_bytes() + 2 * H * S_SHARED
        extra["shared_stack"] = {"us_per_layer": round(1000.0 * mss / LAYERS, 3),
                                 "hbm_gbps": round(bs / (mss / LAYERS * 1e-3) / 1e9, 1),
                                 "tokens_per_s": round(1000.0 / mss, 1), "single_launch_us": round(mks * 1e3, 3),
                                 "us_per_layer_spread": spread(pers / LAYERS),
                                 "bytes_per_layer": bs, "shared_inter": S_SHARED, "flags": fs}
        log(f"nvfp4 + fp8 shared expert stack: {extra['shared_stack']}")
        del shl
        torch.cuda.empty_cache()
        sh4 = build_stack(torch, g, synth, "nvfp4", shared=True, n_tok=4)
        ms4s, mk4s, f4s, per4s = time_stack(torch, g, sh4, args.steps, args.warmup)
        extra["shared_stack_4tok"] = {"us_per_layer": round(1000.0 * ms4s / LAYERS, 3),
                                      "tokens_per_s": round(4000.0 / ms4s, 1),
                                      "single_call_us": round(mk4s * 1e3, 3),
                                      "us_per_layer_spread": spread(per4s / LAYERS), "n_tok": 4,
                                      "shared_inter": S_SHARED, "flags": f4s}
        log(f"nvfp4 + fp8 shared expert stack, 4 tokens per call: {extra['shared_stack_4tok']}")
        del sh4
        torch.cuda.empty_cache()
        a4l = build_stack(torch, g, synth, "nvfp4", w4a4=True)
        msa, mka, fa, pera = time_stack(torch, g, a4l, args.steps, args.warmup)
        ba = layer_bytes()
        extra["w4a4_decode_stack"] = {"us_per_layer": round(1000.0 * msa / LAYERS, 3),
                                      "hbm_gbps": round(ba / (msa / LAYERS * 1e-3) / 1e9, 1),
                                      "tokens_per_s": round(1000.0 / msa, 1), "single_launch_us": round(mka * 1e3, 3),
                                      "us_per_layer_spread": spread(pera / LAYERS), "bytes_per_layer": ba,
                                      "flags": fa}
        log(f"nvfp4 W4A4 single-token stack: {extra['w4a4_decode_stack']}")
        del a4l
        torch.cuda.empty_cache()
        a4s = build_stack(torch, g, synth, "nvfp4", shared=True, w4a4=True)
        msb, mkb, fb, perb = time_stack(torch, g, a4s, args.steps, args.warmup)
        extra["w4a4_shared_stack"] = {"us_per_layer": round(1000.0 * msb / LAYERS, 3),
                                      "hbm_gbps": round(bs / (msb / LAYERS * 1e-3) / 1e9, 1),
                                      "tokens_per_s": round(1000.0 / msb, 1), "single_launch_us": round(mkb * 1e3, 3),
                                      "us_per_layer_spread": spread(perb / LAYERS), "bytes_per_layer": bs,
                                      "flags": fb}
        log(f"nvfp4 W4A4 + fp8 shared expert single-token stack: {extra['w4a4_shared_stack']}")
        del a4s
        torch.cuda.empty_cache()
        extra["spec_step"] = bench_spec_step(torch, g, synth, args.steps)
        extra["w4a4_chunk"] = bench_w4a4(torch, g, synth, args.steps)
        extra["weight_quantizer"] = bench_wquant(torch, g, synth, args.steps)
        extra["mid_batch_w4a4"] = bench_mid_batch(torch, g, synth, args.steps, "w4a4")

    cpu = None
    if not args.skip_cpu:
        model, avail = cpu_model()
        us_cpu, n, threads = cpu_baseline(args.cpu_seconds)
        us_1, n_1, _ = cpu_baseline(args.cpu_seconds / 2, threads=1)
        cpu = {"value": round(us_cpu, 1), "unit": "us/layer", "cores": threads, "kind": "oracle",
               "sample": f"{n} of the 23 layers, 1 token each (router + 6 experts), fp64 oracle",
               "cpu_model": model, "cores_available": avail,
               "one_thread": {"value": round(us_1, 1), "unit": "us/layer", "layers": n_1}}

    from gemm_router_fp32_amd.pmc_traffic import read_traffic
    # HBM bytes per launch from the committed counter passes (None once the
    # kernel's sources differ from the ones the counters were taken on)
    traffic = read_traffic(os.path.join(ROOT, TRAFFIC_PROFILE), "k_decode_stack<1,3,1>")
    out = {
        "metric": METRIC,
        "value": round(us_layer, 4),
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "routed-MoE decode stack: 23 NVFP4 W4A16 layers, batch 1, "
                               "hidden 2688, inter 1856, 128 experts, top-6",
                   "format": "nvfp4-w4a16", "layers": LAYERS, "tokens": 1, "graph": True,
                   "launch": "the 23 layers in one q4moe_w4a16_decode_stack launch per step (graph-captured); "
                             "each layer starts its routing once the previous layer's y is complete"},
        "hbm_gbps": round(gbs, 1),
        "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
        "tokens_per_s": round(1000.0 / ms_step, 1),
        "bytes_per_layer": bytes_layer,
        "us_per_layer_spread": spread(per_step / LAYERS),
        # the stack reads 806 MB per step, > the 256 MB MALL: every layer is
        # cold; one layer alone through its own launch (k_decode_fused):
        "single_launch_us": round(ms_kernel * 1e3, 3),
        # one layer alone with every cache evicted first (direct launch)
        "single_layer_cold_us": round(single_cold_us, 3),
        # the decode's expert phase (first up-load issue to the last down
        # GEMV) from the committed phase timeline of the measurement build
        "expert_phase_gbps": read_profile_value(os.path.join(ROOT, PHASE_PROFILE), "expert_phase_gbps"),
        # one k_decode_stack launch per step (23 layers): its average
        # duration is the timed region over the steps graph replays; achieved
        # = 23 layers' algorithmic bytes per launch / that duration
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": traffic,
                     "traffic_unit": "bytes/launch (23 layers)", "traffic_source": TRAFFIC_PROFILE,
                     "kernel": "k_decode_stack", "kernel_us": round(ms_step * 1e3, 3),
                     "bytes_per_launch": bytes_layer * LAYERS},
        "workspace_flags": max(flags, f_g),
        "extra": extra,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
