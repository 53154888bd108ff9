"""Build the HIP library ``libq4q8mmq.so`` in-tree for gfx950 with hipcc.

Every HIP source under ``csrc/`` is compiled into one shared library that
exports the C ABI of ``include/mmq.h``.  Packed fp32 instructions are
disabled (``-packed-fp32-ops``); fast-math is never used, so fp32 division
stays correctly rounded.
"""
from __future__ import annotations

import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libq4q8mmq.so")
ARCH = "gfx950"

HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", "--offload-arch=" + ARCH,
               "-Wall", "-Wno-unused-result",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build_library(out: str = LIB, extra_flags=(), verbose: bool = False) -> str:
    """Compile every csrc/*.hip into ``out`` (atomically replaced)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc, *HIPCC_FLAGS, *extra_flags, *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library(verbose=True))
