"""HBM traffic per kernel launch from two rocprofv3 counter passes.

Pass 1 collects FETCH_SIZE, pass 2 WRITE_SIZE (KiB per dispatch, CSV output).
Both are scaled by what the same counter reads for the first
`__amd_rocclr_copyBuffer` dispatch of the profiled program, a plain copy of
known size (bench.py starts with a 256 MiB device copy): on gfx950 FETCH_SIZE
counts a 128-byte read request as 64 bytes, so the copy's reading fixes the
factor.  An optional third pass with the TCC_EA0_RDREQ_{32B,64B,128B}_sum
counters gives the read bytes by request size as a cross-check.

The summary also records a SHA-256 of the kernel sources, so that a reader
(bench.py) can tell whether the counters still describe the current kernel.

    python -m gemm_router_fp32_amd.pmc_traffic FETCH.csv WRITE.csv [RDSZ.csv] \
        --copy-bytes 268435456 --kernel k_decode_
"""
import argparse
import collections
import csv
import hashlib
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# the fused decode kernel and the device helpers it inlines
KERNEL_SOURCES = ("csrc/q4moe_fused.hpp", "csrc/q4moe_device.hpp", "csrc/q4moe_kernels.hpp")


def source_sha256(sources=KERNEL_SOURCES):
    h = hashlib.sha256()
    for rel in sources:
        with open(os.path.join(HERE, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def per_kernel(rows, counter):
    out = collections.defaultdict(list)
    for r in rows:
        if r["Counter_Name"] == counter:
            out[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return out


def copy_reading(rows, counter):
    cp = [r for r in rows if r["Counter_Name"] == counter and r["Kernel_Name"] == "__amd_rocclr_copyBuffer"]
    if not cp:
        raise SystemExit(f"no __amd_rocclr_copyBuffer dispatch with {counter}")
    first = min(cp, key=lambda r: int(r["Dispatch_Id"]))
    return float(first["Counter_Value"])


def summarize(fetch_csv, write_csv, rdsz_csv, copy_bytes, kernel_filter, commands):
    fr, wr = _rows(fetch_csv), _rows(write_csv)
    kib = copy_bytes / 1024.0
    f_fac = kib / copy_reading(fr, "FETCH_SIZE")
    w_fac = kib / copy_reading(wr, "WRITE_SIZE")
    fk, wk = per_kernel(fr, "FETCH_SIZE"), per_kernel(wr, "WRITE_SIZE")
    sized = {}
    if rdsz_csv:
        rs = _rows(rdsz_csv)
        parts = {c: per_kernel(rs, c) for c in
                 ("TCC_EA0_RDREQ_32B_sum", "TCC_EA0_RDREQ_64B_sum", "TCC_EA0_RDREQ_128B_sum")}
        for name in parts["TCC_EA0_RDREQ_128B_sum"]:
            n = [sum(parts[c].get(name, [0])) / max(1, len(parts[c].get(name, [1]))) for c in parts]
            sized[name] = 32 * n[0] + 64 * n[1] + 128 * n[2]
    lines = ["# HBM traffic per launch (rocprofv3 counters)", ""]
    lines += ["Commands:", ""] + [f"    {c}" for c in commands] + [""]
    lines += [f"Copy calibration ({copy_bytes} B, first __amd_rocclr_copyBuffer dispatch): "
              f"FETCH_SIZE x {f_fac:.5f}, WRITE_SIZE x {w_fac:.5f}", ""]
    lines += ["| kernel | launches | FETCH_SIZE KiB | WRITE_SIZE KiB | scaled read MB | scaled write MB | "
              "read MB by request size |", "|---|---|---|---|---|---|---|"]
    machine = []
    for name in sorted(fk, key=lambda n: -sum(fk[n])):
        if name == "__amd_rocclr_copyBuffer" or name.startswith("void at::"):
            continue
        f = sum(fk[name]) / len(fk[name])
        w = sum(wk.get(name, [0.0])) / max(1, len(wk.get(name, [])))
        rd, wb = f * f_fac * 1024, w * w_fac * 1024
        s = f"{sized[name] / 1e6:.2f}" if name in sized else "-"
        lines.append(f"| `{name[:72]}` | {len(fk[name])} | {f:.1f} | {w:.1f} | {rd / 1e6:.2f} | {wb / 1e6:.3f} | {s} |")
        if kernel_filter and kernel_filter in name:
            short = name.split("(")[0].replace("void ", "").replace("q4moe::", "").replace(" ", "")
            machine.append(f"traffic {short} bytes_per_launch={int(round(rd + wb))} read={int(round(rd))} "
                           f"write={int(round(wb))}")
    lines += ["", f"source_sha256 {source_sha256()}"] + machine
    return "\n".join(lines) + "\n"


def read_traffic(path, kernel):
    """bytes per launch of `kernel` from a summary, or None when the file is
    missing or the kernel sources changed since the counters were taken."""
    if not os.path.exists(path):
        return None
    sha, val = None, None
    with open(path) as f:
        for line in f:
            if line.startswith("source_sha256 "):
                sha = line.split()[1]
            elif line.startswith(f"traffic {kernel} "):
                val = int(line.split("bytes_per_launch=")[1].split()[0])
    return val if sha == source_sha256() else None


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("fetch")
    ap.add_argument("write")
    ap.add_argument("rdsz", nargs="?")
    ap.add_argument("--copy-bytes", type=int, default=256 << 20)
    ap.add_argument("--kernel", default="k_decode_")
    ap.add_argument("--command", action="append", default=[])
    a = ap.parse_args()
    print(summarize(a.fetch, a.write, a.rdsz, a.copy_bytes, a.kernel, a.command), end="")
