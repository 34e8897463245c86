"""Compile the HIP sources into the in-tree shared library libdvssq.so (gfx950).

Each source is compiled to an object of its own (in parallel), then the objects
are linked into the library.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libdvssq.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed-FP32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
    # host symbols hidden: only the C ABI of include/dvssq.h is exported
    "-Xarch_host", "-fvisibility=hidden",
]


def _filter(stderr: str) -> list[str]:
    return [l for l in stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]


def build(verbose: bool = False) -> str:
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4)), 16))
    with tempfile.TemporaryDirectory(prefix="dvssq_build_") as tmpd:
        def compile_one(src):
            obj = os.path.join(tmpd, os.path.basename(src) + ".o")
            cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            res = subprocess.run(cmd, capture_output=True, text=True)
            return src, obj, res

        with cf.ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(compile_one, srcs))
        failed = False
        for src, _, res in results:
            errs = _filter(res.stderr)
            if res.returncode != 0:
                failed = True
                sys.stderr.write(f"{os.path.basename(src)}:\n" + "\n".join(errs) + "\n")
            elif verbose and errs:
                sys.stderr.write("\n".join(errs) + "\n")
        if failed:
            raise RuntimeError("hipcc failed")
        tmp = LIB + ".tmp"
        cmd = [HIPCC, *FLAGS, "-shared", *[o for _, o, _ in results], "-o", tmp]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            sys.stderr.write("\n".join(_filter(res.stderr)) + "\n")
            raise RuntimeError(f"hipcc link failed ({res.returncode})")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
