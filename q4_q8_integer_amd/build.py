"""Build the HIP library ``libq4q8mmq.so`` in-tree for gfx950 with hipcc.

Every HIP source under ``csrc/`` is compiled to an object (in parallel) and
the objects are linked into one shared library that exports the C ABI of
``include/mmq.h``.  Packed fp32 instructions are disabled
(``-packed-fp32-ops``); fast-math is never used, so fp32 division stays
correctly rounded.

"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import shutil
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libq4q8mmq.so")
ARCH = "gfx950"

HIPCC_FLAGS = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
               "-Wall", "-Wno-unused-result",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
SOURCE_FLAGS = {}   # per-source extra flags (none at present)


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build_library(out: str = LIB, extra_flags=(), verbose: bool = False) -> str:
    """Compile every csrc/*.hip and link ``out`` (atomically replaced)."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    work = tempfile.mkdtemp(prefix="q4q8build")
    try:
        def compile_one(src):
            obj = os.path.join(work, os.path.basename(src) + ".o")
            cmd = [hipcc, *HIPCC_FLAGS, *SOURCE_FLAGS.get(os.path.basename(src), []),
                   *extra_flags, "-c", src, "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.run(cmd, check=True)
            return obj
        jobs = min(8, os.cpu_count() or 1)
        with concurrent.futures.ThreadPoolExecutor(jobs) as pool:
            objs = list(pool.map(compile_one, sources()))
        tmp = out + ".tmp%d" % os.getpid()
        cmd = [hipcc, "-shared", "-fPIC", "--offload-arch=" + ARCH, *objs, "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    finally:
        shutil.rmtree(work, ignore_errors=True)
    return out


if __name__ == "__main__":
    print(build_library(verbose=True))
