"""Build libmdn.so (the C-ABI library) for gfx950 with hipcc, in-tree.

Usage: ``python -m linear_attention_sequence_mdn_amd.build`` (or ``build()``).
Objects go to ``_build/`` next to this file; the library to
``linear_attention_sequence_mdn_amd/libmdn.so``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libmdn.so")
SOURCES = ["mdn_api.cpp", "mdn_step.hip", "mdn_intra.hip", "mdn_chunk.hip", "mdn_fwd.hip", "mdn_gates.hip",
           "mdn_bwd.hip"]
HEADERS = ["mdn_device.h", "mdn_internal.h", "mdn_lds.h"]
ARCH = os.environ.get("MDN_OFFLOAD_ARCH", "gfx950")

# Packed fp32 vector ops are disabled for the device code: without the
# feature switch the compiler forms v_pk_fma/mul/add_f32 from ordinary float
# (and float2) code.  hipcc also hands the switch to the host pass, which
# warns that it does not know the feature; that warning is harmless.  After
# compiling, every object's gfx950 code is disassembled and the build fails
# if any packed fp32 instruction is present (check_no_packed_fp32).
# Matrix-core results go to ordinary VGPRs (-amdgpu-mfma-vgpr-form): where the
# compiler would otherwise put accumulators in AGPRs (the intra and backward
# kernels), every later use costs a v_accvgpr_read; the other kernels compile
# to the same code either way.  Measured: backward 860.7 -> 854.1 us (three
# alternating bench runs), the forward unchanged.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mllvm", "-amdgpu-mfma-vgpr-form",
          "-Wall", "-Wno-unused-function", "-I", os.path.join(HERE, "..", "include")]


def _hipcc():
    for c in (os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "bin", "hipcc"), "hipcc"):
        if os.path.sep not in c or os.path.exists(c):
            return c
    return "hipcc"


def _llvm_tool(name):
    return os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin", name)


PACKED_FP32 = re.compile(r"\bv_pk_(fma|mul|add)_f32\b")


def check_no_packed_fp32(obj: str) -> None:
    """Disassemble the gfx950 code object bundled in `obj` (built here) and
    raise if it holds a packed fp32 instruction."""
    folder, base = os.path.split(os.path.abspath(obj))
    # extracts the bundled code objects next to `obj`, as <obj>.<n>.<target>
    subprocess.run([_llvm_tool("llvm-objdump"), "--offloading", base], check=True, cwd=folder,
                   stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    parts = [f for f in os.listdir(folder) if f.startswith(base + ".")]
    try:
        dev = [f for f in parts if f"amdgcn-amd-amdhsa--{ARCH}" in f]
        if not dev:
            raise RuntimeError(f"{obj}: no {ARCH} code object found to check")
        for f in dev:
            asm = subprocess.run([_llvm_tool("llvm-objdump"), "-d", os.path.join(folder, f)], check=True,
                                 capture_output=True, text=True).stdout
            hits = sorted({m.group(0) for m in PACKED_FP32.finditer(asm)})
            if hits:
                raise RuntimeError(f"{obj}: packed fp32 instructions in the device code: {hits}")
    finally:
        for f in parts:
            os.remove(os.path.join(folder, f))


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *COMMON, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    subprocess.run(cmd, check=True)
    if src.endswith(".hip"):
        check_no_packed_fp32(obj)
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
