"""MFMA utilisation and wait counters of the grouped GEMMs from two
rocprofv3 counter passes over the W4A4 1024-token chunk (CSV output):

    pass 1: --pmc MfmaUtil   (derived: SQ_VALU_MFMA_BUSY_CYCLES summed over
            SIMDs / (GRBM_GUI_ACTIVE * SIMD_NUM), percent)
    pass 2: --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_WAIT_ANY SQ_WAVE_CYCLES
            SQ_BUSY_CU_CYCLES SQ_INSTS_VALU_MFMA_MOPS_F16 GRBM_GUI_ACTIVE

Prints a markdown summary per kernel: MFMA busy (percent of the SIMD
cycles while the GPU is active), the share of wave cycles spent waiting
(SQ_WAIT_ANY / SQ_WAVE_CYCLES, both in quad-cycles), and the fp16 MFMA
flops the counters saw (MOPS x 512), with `mfma_busy_frac=` for the
benchmark and a SHA-256 of the GEMM sources.

    python -m gemm_router_fp32_amd.mfma_counters PASS1.csv PASS2.csv --kernel k_grouped_gemm
"""
import argparse
import collections
import csv

from gemm_router_fp32_amd.pmc_traffic import source_sha256

GEMM_SOURCES = ("csrc/q4moe_w4a4.hpp", "csrc/q4moe_device.hpp", "csrc/q4moe_kernels.hpp")


def _per_kernel(path):
    out = collections.defaultdict(lambda: collections.defaultdict(list))
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            out[r["Kernel_Name"]][r["Counter_Name"]].append(float(r["Counter_Value"]))
    return out


def summarize(p1, p2, kernel, commands):
    a, b = _per_kernel(p1), _per_kernel(p2)
    lines = ["# MFMA utilisation and waits of the grouped GEMMs (rocprofv3 counters)", "", "Commands:", ""]
    lines += [f"    {c}" for c in commands] + [""]
    lines += ["| kernel | dispatches | MfmaUtil % (pass 1) | MFMA busy cycles / SIMD / dispatch | "
              "wave cycles waiting % | fp16 MFMA GFLOP / dispatch |", "|---|---|---|---|---|---|"]
    busy = []
    for name in sorted(a):
        if kernel not in name:
            continue
        util = a[name].get("MfmaUtil", [])
        c = b.get(name, {})
        n = max(1, len(c.get("SQ_WAVE_CYCLES", [1])))
        wait = sum(c.get("SQ_WAIT_ANY", [0])) / max(1.0, sum(c.get("SQ_WAVE_CYCLES", [1])))
        mfb = sum(c.get("SQ_VALU_MFMA_BUSY_CYCLES", [0])) / n / 1024.0  # 256 CUs x 4 SIMDs
        gflop = sum(c.get("SQ_INSTS_VALU_MFMA_MOPS_F16", [0])) * 512 / n / 1e9
        u = sum(util) / max(1, len(util))
        busy.append(u)
        lines.append(f"| `{name[:70]}` | {len(util)} | {u:.1f} | {mfb:.0f} | {100 * wait:.1f} | {gflop:.2f} |")
    lines += ["", f"mfma_busy_frac={(sum(busy) / max(1, len(busy))) / 100:.4f}",
              f"source_sha256={source_sha256(GEMM_SOURCES)}"]
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("pass1")
    ap.add_argument("pass2")
    ap.add_argument("--kernel", default="k_grouped_gemm")
    ap.add_argument("--command", action="append", default=[])
    a = ap.parse_args()
    print(summarize(a.pass1, a.pass2, a.kernel, a.command))


if __name__ == "__main__":
    main()
