"""Builds libgsrast.so (the HIP library behind include/gsrast.h) in-tree for gfx950."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libgsrast.so")
SOURCES = ["api.hip", "preprocess.hip", "scan.hip", "depth_sort.hip", "sort.hip", "binning.hip", "composite.hip", "backward.hip", "schedule.hip",
           "splat2d.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared",
    "--offload-arch=gfx950",
    # packed fp32 instructions stay off: the compiler must not form v_pk_* fp32 ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-o", tmp, *srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # the host pass does not know the gfx950 feature flag and says so once per file
    lines = [l for l in res.stdout.splitlines() if "is not a recognized feature for this target" not in l]
    if lines and (verbose or res.returncode):
        print("\n".join(lines), flush=True)
    if res.returncode:
        raise subprocess.CalledProcessError(res.returncode, cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
