"""The build's packed-fp32 guard (CPU: hipcc cross-compiles gfx950 here).

A float2 multiply-add compiled without the feature switch yields packed fp32
instructions, which the check must reject; the same source built with the
library's flags must pass it."""
import os
import shutil
import subprocess

import pytest

from linear_attention_sequence_mdn_amd import build as B

SRC = r"""
#include <hip/hip_runtime.h>
__global__ void axpy2(float2* a, const float2* b, float s) {
    const int i = threadIdx.x + blockIdx.x * blockDim.x;
    float2 x = a[i], y = b[i];
    x.x = x.x * s + y.x; x.y = x.y * s + y.y;
    x.x *= y.x; x.y *= y.y;
    a[i] = x;
}
"""

pytestmark = pytest.mark.skipif(not os.path.exists(B._hipcc()) and shutil.which("hipcc") is None,
                                reason="hipcc not installed")


def _build(tmp_path, flags):
    src = tmp_path / "axpy2.hip"
    src.write_text(SRC)
    obj = tmp_path / ("with.o" if flags else "without.o")
    base = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={B.ARCH}"]
    subprocess.run([B._hipcc(), *base, *flags, "-x", "hip", "-c", str(src), "-o", str(obj)], check=True,
                   capture_output=True)
    return str(obj)


def test_guard_rejects_packed_fp32(tmp_path):
    obj = _build(tmp_path, [])
    with pytest.raises(RuntimeError, match="packed fp32"):
        B.check_no_packed_fp32(obj)
    # the extracted code objects are removed again
    assert sorted(os.listdir(tmp_path)) == ["axpy2.hip", "without.o"]


def test_guard_passes_with_the_library_flags(tmp_path):
    obj = _build(tmp_path, ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"])
    B.check_no_packed_fp32(obj)
