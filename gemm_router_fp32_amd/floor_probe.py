"""Floor measurements for the one-launch decode, from the measurement build
libq4moe_probe.so (csrc/q4moe_probe.hip): what one launch can stream from
HBM, what an empty launch of the decode's shape costs inside a 23-node
graph, and the decode's in-kernel phase timeline inside the 23-layer stack.
Prints a markdown report.  Meant to run under rocprofv3 --kernel-trace
--stats (the kernel durations of the stream and empty probes come from its
summary too):

    python -m gemm_router_fp32_amd.floor_probe stream
    python -m gemm_router_fp32_amd.floor_probe launch
    python -m gemm_router_fp32_amd.floor_probe phase [nvfp4|int4]
"""
import ctypes
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PROBE_SO = os.path.join(HERE, "libq4moe_probe.so")
LAYER_BYTES = 35062832  # one NVFP4 decode layer: 6 experts, the fp32 router, x and y


def _lib():
    if not os.path.exists(PROBE_SO):
        raise SystemExit("libq4moe_probe.so is not built (gemm_router_fp32_amd.build.build(probe=True))")
    return ctypes.CDLL(PROBE_SO)


def _events(torch):
    return torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)


def stream(torch):
    """Cold streaming reads of one layer's bytes and of the 23-layer stack's,
    at a few grid sizes; 1 GiB read before each rep evicts the caches."""
    L = _lib()
    L.q4p_stream.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    big = torch.ones(23 * LAYER_BYTES // 16 * 16 // 8, dtype=torch.int64, device="cuda")
    sink = torch.empty(1 << 22, dtype=torch.int32, device="cuda")
    evict = torch.ones(1 << 27, dtype=torch.int64, device="cuda")
    print("| bytes | grid (x 256 threads) | median us | GB/s |\n|---|---|---|---|")
    for nbytes in (LAYER_BYTES // 16 * 16, big.numel() * 8):
        for grid in (256, 512, 1024, 2048, 4096):
            ts = []
            for rep in range(12):
                evict.sum()
                e0, e1 = _events(torch)
                e0.record()
                assert L.q4p_stream(ctypes.c_void_p(big.data_ptr()), nbytes, grid, ctypes.c_void_p(sink.data_ptr()),
                                    s) == 0
                e1.record()
                e1.synchronize()
                if rep >= 2:
                    ts.append(e0.elapsed_time(e1) * 1e3)
            us = float(np.median(ts))
            print(f"| {nbytes} | {grid} | {us:.2f} | {nbytes / (us * 1e-6) / 1e9:.1f} |", flush=True)


def launch(torch):
    """The device-side cost between the nodes of a 23-node graph: kernels of
    the decode's shape (256 x 512) that each hold the GPU for 15 us (so the
    host stays ahead of the device) record their first start and last end on
    the device clock; the gap from one node's end to the next one's start is
    what a launch costs inside a graph replay.  Also: the duration of an
    empty kernel of that shape (from the rocprofv3 trace of this run)."""
    L = _lib()
    L.q4p_empty.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    L.q4p_spin.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_ulonglong, ctypes.c_void_p,
                           ctypes.c_void_p]
    out = torch.empty(1 << 16, dtype=torch.int32, device="cuda")
    t = torch.empty(2 * 23, dtype=torch.int64, device="cuda")
    print("| graph of 23 nodes | gap end -> next start, median (us) | p10 | p90 |\n|---|---|---|---|")
    for grid, block in ((256, 512), (256, 256), (1024, 256)):
        def step():
            s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            for i in range(23):
                assert L.q4p_spin(grid, block, i, 1500, ctypes.c_void_p(t.data_ptr()), s) == 0
        step()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        gaps = []
        for rep in range(30):
            t.view(-1, 2)[:, 0].fill_(np.iinfo(np.int64).max)
            t.view(-1, 2)[:, 1].fill_(0)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            v = t.view(-1, 2).cpu().numpy().astype(np.float64)
            if rep >= 3:
                gaps += list((v[1:, 0] - v[:-1, 1]) * 0.01)
        q = np.percentile(gaps, [50, 10, 90])
        print(f"| spin kernels {grid} x {block} | {q[0]:.2f} | {q[1]:.2f} | {q[2]:.2f} |", flush=True)
    # empty kernels of the decode's shape: their duration is in the trace
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    for _ in range(200):
        assert L.q4p_empty(256, 512, ctypes.c_void_p(out.data_ptr()), s) == 0
    torch.cuda.synchronize()
    print("\n(200 empty 256 x 512 launches follow; their durations are in the kernel trace)")


def phase(torch, fmt, stack=False):
    """Phase timeline of the one-launch decode inside the 23-layer stack's
    graph replays (medians over the layers of the median, and of the
    maximum, over workgroups), the shader clock and the gaps between
    layers, and the expert phase's HBM rate: the selected experts' bytes
    over the time from the first up-load issue to the end of the down
    GEMVs.  stack: the 23 layers in one stacked launch per replay (a layer's
    start is then its workgroups' entry into the layer)."""
    import gemm_router_fp32_amd.q4moe as q
    sys.path.insert(0, ROOT)
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    L = _lib()
    for name, (res, args) in q._SIGS.items():
        f = getattr(L, name)
        f.restype, f.argtypes = res, args
    L.q4p_read.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    q._LIB = L  # every call below goes to the measurement build
    import gemm_router_fp32_amd as g
    import synth
    import bench
    layers = bench.build_stack(torch, g, synth, fmt)
    if stack:
        ms, flags, _ = bench.time_stack_launch(torch, g, layers, 20, 5)
        step, _ws = bench.stack_launch_step(g, layers)
    else:
        ms, _, flags, _ = bench.time_stack(torch, g, layers, 20, 5)

        def step():
            for Ly in layers:
                bench.decode_call(g, Ly)
    graph = torch.cuda.CUDAGraph()
    step()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    for _ in range(3):
        graph.replay()
    torch.cuda.synchronize()
    buf = np.zeros((32, 256, 48), np.uint64)
    n = ctypes.c_uint(0)
    assert L.q4p_read(buf.ctypes.data, ctypes.byref(n)) == 0
    slots = [(n.value - 23 + i) % 32 for i in range(23)]
    names = {0: "start", 1: "router done", 2: "scores in", 3: "top-k done", 8: "up loads issued",
             9: "up GEMV done", 4: "down loads issued", 5: "h in", 6: "down done", 7: "combine done (wave 0)",
             10: "end (all waves)"}
    order = [0, 1, 2, 3, 8, 4, 9, 5, 6, 7, 10]
    rel = []
    for s_ in slots:
        b = buf[s_].astype(np.float64)
        rel.append((b[:, :11] - b[:, 0].min()) * 0.01)  # us from the first workgroup's start
    med = np.median(np.stack([[np.median(r[:, p]) for p in order] for r in rel]), axis=0)
    mx = np.median(np.stack([[np.max(r[:, p]) for p in order] for r in rel]), axis=0)
    how = "one stacked launch per replay" if stack else "graph replay of one launch per layer"
    print(f"{fmt} stack: {ms * 1000 / 23:.3f} us per layer ({how}, measurement build), flags {flags}\n")
    print("| phase | median over workgroups (us) | max over workgroups (us) |\n|---|---|---|")
    for i, p in enumerate(order):
        print(f"| {names[p]} | {med[i]:.2f} | {mx[i]:.2f} |")
    clk, gaps, spans, starts = [], [], [], []
    for s_ in slots:
        b = buf[s_].astype(np.float64)
        clk.append(np.median((b[:, 12] - b[:, 11]) / ((b[:, 10] - b[:, 0]) * 1e-8) / 1e9))
        starts.append((b[:, 0].min(), b[:, 10].max()))
    for i in range(22):
        gaps.append((starts[i + 1][0] - starts[i][1]) * 0.01)
    spans = [(e - s0) * 0.01 for s0, e in starts]
    t_up = med[order.index(8)]
    t_dn = mx[order.index(6)]
    expert_bytes = 6 * (2 * (2688 * 1856 // 2 + 2688 * 1856 // 16 + 4)) if fmt == "nvfp4" else \
        6 * (2 * (2688 * 1856 // 2 + 2688 * 1856 // 64 * 2))
    print(f"\nshader clock during the kernel: {np.median(clk):.3f} GHz (median over layers)")
    print(f"first start to last end: {np.median(spans):.2f} us; gap to the next layer's first start: "
          f"{np.median(gaps):.2f} us (median)")
    print(f"expert phase: up loads issued (median {t_up:.2f} us) to down done (max {t_dn:.2f} us): "
          f"{t_dn - t_up:.2f} us for {expert_bytes} expert bytes = "
          f"{expert_bytes / ((t_dn - t_up) * 1e-6) / 1e9:.1f} GB/s")
    print(f"expert_phase_gbps={expert_bytes / ((t_dn - t_up) * 1e-6) / 1e9:.1f}")
    # per-wave marks: 0 up GEMV done, 1 h published and down loads issued,
    # 2 h polled into LDS, 3 down GEMV done (every wave of every workgroup)
    wm = []
    for s_ in slots:
        b = buf[s_].astype(np.float64)
        w = b[:, 16:48].reshape(-1, 8, 4)
        wm.append((w - b[:, 0].min()) * 0.01)
    wm = np.stack(wm)  # [layers, wgs, waves, 4]
    steps = [("up GEMV done", wm[..., 0]), ("h published, down loads issued", wm[..., 1]),
             ("h polled into LDS", wm[..., 2]), ("down GEMV done", wm[..., 3])]
    print("\n| per-wave mark | median (us) | p90 | max |\n|---|---|---|---|")
    for name, v in steps:
        print(f"| {name} | {np.median(v):.2f} | {np.median(np.percentile(v, 90, axis=(1, 2))):.2f} | "
              f"{np.median(v.max(axis=(1, 2))):.2f} |")
    durs = [("publish + down-load issue", wm[..., 1] - wm[..., 0]), ("barrier + h poll", wm[..., 2] - wm[..., 1]),
            ("barrier + down GEMV", wm[..., 3] - wm[..., 2])]
    print("\n| per-wave span | median (us) | p90 | max |\n|---|---|---|---|")
    for name, v in durs:
        print(f"| {name} | {np.median(v):.2f} | {np.median(np.percentile(v, 90, axis=(1, 2))):.2f} | "
              f"{np.median(v.max(axis=(1, 2))):.2f} |")


def main():
    import torch
    torch.cuda.set_device(0)
    what = sys.argv[1] if len(sys.argv) > 1 else "stream"
    if what == "stream":
        stream(torch)
    elif what == "launch":
        launch(torch)
    elif what == "phase":
        phase(torch, sys.argv[2] if len(sys.argv) > 2 else "nvfp4", "--stack" in sys.argv)
    else:
        raise SystemExit(f"unknown measurement {what}")


if __name__ == "__main__":
    main()
