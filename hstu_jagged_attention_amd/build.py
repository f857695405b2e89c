"""Build the in-tree HIP library ``libhstu.so`` for gfx950 with hipcc.

Usage: ``python -m hstu_jagged_attention_amd.build`` (or ``build()``). The
library lands next to this file, where the binding loads it from.
"""
from __future__ import annotations

import os
import subprocess
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libhstu.so")
SOURCES = [os.path.join(CSRC, "hstu_kernels.hip"), os.path.join(CSRC, "hstu_scratch.hip"),
           os.path.join(CSRC, "hstu_abi.cpp")]
HEADERS = [os.path.join(ROOT, "include", "hstu.h"), os.path.join(CSRC, "hstu_internal.h")]

ARCH = "gfx950"
# Packed fp32 VALU forms are kept out of the generated code on purpose.
FLAGS = ["-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
         "-packed-fp32-ops", "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp"
    cmd = [hipcc()] + FLAGS + ["-I", os.path.join(ROOT, "include"), "-I", CSRC] + SOURCES + ["-o", tmp]
    t0 = time.time()
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed ({r.returncode}): {' '.join(cmd)}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} in {time.time() - t0:.1f}s")
    return LIB


def is_stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(s) > t for s in SOURCES + HEADERS)


if __name__ == "__main__":
    build(verbose=True)
