"""Builds libmoe_hotpath.so (gfx950) in-tree with hipcc; libmoe_ceiling.so,
the benchmark's read-stream and MFMA-rate probes (not part of the hot path's C
ABI); and libmoe_hotpath_trace.so, the same sources with the clock-stamp trace
compiled in (MOE_TRACE=1, csrc/trace.h), which `python -m
combine_expert_histogram_amd.trace` loads.

Usage: python -m combine_expert_histogram_amd.build [-v] [--no-trace]
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libmoe_hotpath.so")
SOURCES = ["api.hip", "layout.hip", "quant.hip", "gemm1.hip", "stage2.hip", "combine.hip"]
TRACE_LIB = os.path.join(PKG, "libmoe_hotpath_trace.so")
CEILING_LIB = os.path.join(PKG, "libmoe_ceiling.so")
CEILING_SOURCES = ["ceiling.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        # no fast-math: the quant's IEEE divisions must stay correctly rounded
        "-fno-fast-math", "-ffp-contract=on",
        # keep the compiler from emitting packed fp32 arithmetic
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
        f"-I{INCLUDE}", f"-I{CSRC}",
    ]


def _link(sources: list[str], out: str, verbose: bool, extra: tuple[str, ...] = ()) -> str:
    srcs = [os.path.join(CSRC, s) for s in sources]
    tmp = out + ".tmp"
    cmd = [hipcc(), *flags(), *extra, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


def build(verbose: bool = False, trace: bool = True) -> str:
    _link(CEILING_SOURCES, CEILING_LIB, verbose)
    if trace:
        _link(SOURCES, TRACE_LIB, verbose, ("-DMOE_TRACE=1",))
    return _link(SOURCES, LIB, verbose)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, trace="--no-trace" not in sys.argv))
