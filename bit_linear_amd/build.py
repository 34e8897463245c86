"""Compile the HIP sources into the in-tree shared library libdvssq.so (gfx950)."""
from __future__ import annotations

import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdvssq.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed-FP32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    # host symbols hidden: only the C ABI of include/dvssq.h is exported
    "-Xarch_host", "-fvisibility=hidden",
]


def build(verbose: bool = False) -> str:
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    errs = [l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if res.returncode != 0:
        sys.stderr.write("\n".join(errs) + "\n")
        raise RuntimeError(f"hipcc failed ({res.returncode})")
    if verbose and errs:
        sys.stderr.write("\n".join(errs) + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
