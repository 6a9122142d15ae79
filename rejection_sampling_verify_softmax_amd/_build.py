"""Build libsd.so (the HIP/gfx950 library behind include/sd.h) in-tree.

One hipcc invocation compiles every csrc/*.hip file for gfx950 and links the
shared library next to this file. Flags:
  -O3 -std=c++17 -fPIC -shared --offload-arch=gfx950
  -ffp-contract=off                       no implicit FMA: products and sums are
                                          rounded exactly as written (fused
                                          multiply-adds are explicit builtins)
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                          no packed fp32 VALU instructions
  -mcode-object-version=5                 loadable by the HIP runtime torch ships
"""
from __future__ import annotations

import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libsd.so")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP toolchain is required to build libsd")


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, extra_flags=()) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-ffp-contract=off", "-mcode-object-version=5",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-Wno-unused-function",
           "-I", INCLUDE, "-I", CSRC, *extra_flags, "-o", tmp, *sources()]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("libsd build failed")
    if verbose and r.stderr.strip():
        # hipcc's host pass warns about the device-only target feature; harmless
        lines = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l]
        if lines:
            sys.stderr.write("\n".join(lines) + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
