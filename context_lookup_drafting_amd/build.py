"""Build liblcd.so (the HIP library) in-tree for gfx950 with hipcc.

    python -m context_lookup_drafting_amd.build
"""

from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "liblcd.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed-FP32 instructions are disabled for every HIP translation unit.  The
# atomic optimizer is off: it turns a single lane's fetch-and-add into a wave
# reduction that waits for the returned value immediately, which would put a
# full memory round trip in front of the scan's first loads.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", INCLUDE,
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, extra=()) -> str:
    tmp = LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra, *sources(), "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building liblcd.so")
    if verbose:
        sys.stderr.write(res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
