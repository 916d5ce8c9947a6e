"""Benchmark: batch-1 routed-MoE decode through a 23-layer NVFP4 W4A16 stack.

One step = one token through 23 independent routed-MoE layers (hidden 2688,
expert intermediate 1856, 128 experts, top-6), each layer a router top-6,
up GEMV, relu^2, down GEMV and weighted combine, run one after another on
one stream.  The stack is captured once in a HIP graph and replayed.
Inputs are seeded synthetic tensors resident in HBM before timing starts.

Prints one JSON line (metric: microseconds per layer, plus achieved HBM
bandwidth against MI355X's 8 TB/s), with the oracle's CPU time on a
bounded sample of the same workload beside it.
"""
import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

H, I, E, K, LAYERS = 2688, 1856, 128, 6, 23
SEED = 20261202
PEAK_HBM_GBS = 8000.0
METRIC = "µs per routed-MoE layer at batch 1 + achieved HBM GB/s (% of MI355X peak)"


def layer_bytes(E_=E, H_=H, I_=I, k=K, T=1):
    """Algorithmic HBM bytes of one NVFP4 decode layer: the k selected
    experts' codes and E4M3 scales (up and down) and fp32 per-tensor scales,
    the fp32 router (W_g and bias), x and y (bf16)."""
    expert = 2 * (H_ * I_ // 2 + H_ * I_ // 16 + 4)
    return k * expert + E_ * H_ * 4 + E_ * 4 + T * H_ * 2 * 2


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-graph", action="store_true", help="time direct launches instead of a graph replay")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="bound on the oracle CPU sample")
    ap.add_argument("--skip-cpu", action="store_true")
    return ap.parse_args()


def build_stack(torch, g, synth):
    """Generate the 23 layers on the host (one reused buffer) and upload."""
    from gpu_util import dev
    layers = []
    buf = None
    for li in range(LAYERS):
        bank = synth.expert_bank(SEED, synth.FAM_NVFP4, li, E, H, I, "nvfp4", out=buf)
        buf = bank
        wg, b = synth.router(SEED, synth.FAM_NVFP4, li, E, H)
        x = synth.x_rows(SEED, synth.FAM_NVFP4, li, H, [0])
        t = {k: dev(v) for k, v in bank.items()}
        ex = g.Experts(g.NVFP4, t["up_codes"], t["up_scales"], t["down_codes"], t["down_scales"],
                       t["up_gscale"], t["down_gscale"])
        r = g.Router(dev(wg), dev(b), K)
        xt = dev(x)
        y = torch.empty((1, H), dtype=torch.int16, device="cuda")
        ws = g.workspace(g.q4moe_w4a16_decode_ws_bytes(r, ex, 1))
        layers.append(dict(ex=ex, r=r, x=xt, y=y, ws=ws))
        print(f"[bench] layer {li} resident", file=sys.stderr, flush=True)
    return layers


def cpu_baseline(seconds):
    """The oracle, as it stands, on layers of the same stack until `seconds`
    of CPU work have run; returns microseconds per layer."""
    import oracle
    import synth
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


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1", "n_gpus": args.gpus}))
        sys.exit(2)
    import torch

    import gemm_router_fp32_amd as g
    import synth
    sys.path.insert(0, os.path.join(ROOT, "tests"))

    torch.cuda.set_device(0)
    g.lib()
    layers = build_stack(torch, g, synth)
    stream = torch.cuda.current_stream()

    def step():
        for L in layers:
            g.q4moe_w4a16_decode(L["r"], L["ex"], L["x"], L["y"], ws=L["ws"])

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    graph = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(stream)
        with torch.cuda.stream(s):
            step()  # warm the capture stream
        stream.wait_stream(s)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()

    run = graph.replay if graph is not None else step
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    ev0.record()
    for _ in range(args.steps):
        run()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms_total = ev0.elapsed_time(ev1)
    ms_step = ms_total / args.steps
    us_layer = 1000.0 * ms_step / LAYERS
    bytes_layer = layer_bytes()
    gbs = bytes_layer / (us_layer * 1e-6) / 1e9
    print(f"[bench] {args.steps} steps: {ms_step:.4f} ms/step, {us_layer:.3f} us/layer, {gbs:.1f} GB/s "
          f"(wall {wall:.3f} s)", file=sys.stderr, flush=True)

    cpu = None
    if not args.skip_cpu:
        us_cpu, n, threads = cpu_baseline(args.cpu_seconds)
        cpu = {"value": round(us_cpu, 1), "unit": "us/layer", "cores": threads, "kind": "oracle",
               "sample": f"{n} of the 23 layers, 1 token each (router + 6 experts), fp64 oracle"}

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
                   "format": "nvfp4-w4a16", "layers": LAYERS, "tokens": 1,
                   "graph": graph is not None},
        "hbm_gbps": round(gbs, 1),
        "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
        "tokens_per_s": round(1000.0 / ms_step, 1),
        "bytes_per_layer": bytes_layer,
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
