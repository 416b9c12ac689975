"""Build libmdn.so (the C-ABI library) for gfx950 with hipcc, in-tree.

Usage: ``python -m linear_attention_sequence_mdn_amd.build`` (or ``build()``).
Objects go to ``_build/`` next to this file; the library to
``linear_attention_sequence_mdn_amd/libmdn.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmdn.so")
SOURCES = ["mdn_api.cpp", "mdn_step.hip", "mdn_intra.hip", "mdn_chunk.hip", "mdn_gates.hip", "mdn_bwd.hip"]
HEADERS = ["mdn_device.h", "mdn_internal.h", "mdn_lds.h"]
ARCH = os.environ.get("MDN_OFFLOAD_ARCH", "gfx950")

# Packed fp32 vector ops are disabled: the compiler may otherwise form
# v_pk_* fp32 instructions from ordinary float code.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", "-I", os.path.join(HERE, "..", "include")]


def _hipcc():
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), "hipcc"):
        if os.path.sep not in c or os.path.exists(c):
            return c
    return "hipcc"


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *COMMON, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    subprocess.run(cmd, check=True)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libmdn.so; always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.run([_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs], check=True)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
