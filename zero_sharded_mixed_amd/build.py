"""Build libzero_shard.so (every HIP source under csrc/) and libzero_probe.so (the bandwidth
probes under probe/) for gfx950 with hipcc, in place, and libzero_shard_smallgrid.so: the same
sources with every grid capped at SMALL_GRID_CAP blocks, which the tests run to check that the
kernels' loops over their work items give the same results as the one-shot grids."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB = os.path.join(HERE, "libzero_shard.so")
PROBE_LIB = os.path.join(HERE, "libzero_probe.so")
SMALL_GRID_LIB = os.path.join(HERE, "libzero_shard_smallgrid.so")
SMALL_GRID_CAP = 37  # blocks per launch: every block then takes many work items in turn
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall", "-Werror",
    "-fno-gpu-flush-denormals-to-zero",                      # keep fp16/fp32 subnormals exact
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",  # no packed fp32 instructions
    "-Wno-unused-command-line-argument",
]


def sources() -> list:
    return sorted(glob.glob(os.path.join(HERE, "csrc", "*.hip")))


def probe_sources() -> list:
    return sorted(glob.glob(os.path.join(HERE, "probe", "*.hip")))


def _hipcc(srcs: list, out: str, verbose: bool, extra: tuple = ()) -> str:
    tmp = out + f".tmp{os.getpid()}"
    cmd = [HIPCC, *FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-I", os.path.join(HERE, "csrc"), *srcs,
           "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed building {os.path.basename(out)}")
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Compile the three libraries (every call compiles); returns the pipeline library's path."""
    _hipcc(probe_sources(), PROBE_LIB, verbose)
    _hipcc(sources(), SMALL_GRID_LIB, verbose, (f"-DZS_GRID_CAP={SMALL_GRID_CAP}",))
    return _hipcc(sources(), LIB, verbose)


if __name__ == "__main__":
    print(build(verbose=True))
