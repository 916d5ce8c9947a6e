"""Build libq4moe.so in-tree with hipcc for gfx950 (and the measurement build
libq4moe_probe.so, which only gemm_router_fp32_amd/floor_probe.py loads)."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SO = os.path.join(HERE, "libq4moe.so")
SOURCES = [os.path.join(HERE, "csrc", "q4moe_api.hip")]
PROBE_SO = os.path.join(HERE, "libq4moe_probe.so")
PROBE_SOURCES = [os.path.join(HERE, "csrc", "q4moe_probe.hip")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 instructions stay off in every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"),
]


def _start(sources, out, verbose):
    cmd = [HIPCC] + FLAGS + sources + ["-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True)


def _finish(proc, out, verbose):
    _, stderr = proc.communicate()
    err = "\n".join(l for l in stderr.splitlines() if "packed-fp32-ops" not in l)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(out + ".tmp", out)
    return out


def build(verbose=False, probe=False):
    """Compile libq4moe.so (and, with probe, libq4moe_probe.so at the same time)."""
    jobs = [(_start(SOURCES, SO, verbose), SO)]
    if probe:
        jobs.append((_start(PROBE_SOURCES, PROBE_SO, verbose), PROBE_SO))
    for proc, out in jobs:
        _finish(proc, out, verbose)
    return SO


if __name__ == "__main__":
    print(build(verbose=True, probe="--probe" in sys.argv))
