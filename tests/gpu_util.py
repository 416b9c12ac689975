"""Helpers for the GPU parity tests (tests call the HIP path only through the
C ABI, via the thin binding, and compare it with the fp64 oracle)."""
from __future__ import annotations

import sys

import numpy as np

# Tolerances on max|gpu - ref| / max|ref| over a whole output tensor: 1e-4 for
# fp32 inputs and 2e-2 for bf16 inputs (bf16 operands on the matrix cores,
# fp32 accumulation and fp32 state).
TOL = {"f32": 1e-4, "bf16": 2e-2}


def torch_mod():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    return torch


def dev(x, dtype="f32"):
    """numpy float32 array (values exact in dtype) -> contiguous device tensor."""
    torch = torch_mod()
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).cuda()
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def host(t):
    return t.float().cpu().numpy().astype(np.float64)


def rel_err(got, ref):
    ref = np.asarray(ref, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    denom = np.abs(ref).max()
    if denom == 0:
        return float(np.abs(got).max())
    return float(np.abs(got - ref).max() / denom)


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run_chunk(x, C=None, S0=None, M0=None, **kw):
    """Run mdn_chunk_fwd on a ChunkInputs; returns host fp64 (O, S_T, M_T, Vt)."""
    import linear_attention_sequence_mdn_amd as mdn
    torch = torch_mod()
    C = x.C if C is None else C
    s0 = x.S0 if S0 is None else S0
    m0 = x.M0 if M0 is None else M0
    args = [dev(x.q, x.dtype), dev(x.k, x.dtype), dev(x.v, x.dtype), dev(x.alpha), dev(x.mu),
            dev(x.beta), dev(x.eta), None if s0 is None else dev(s0), None if m0 is None else dev(m0)]
    out = mdn.chunk_fwd(*args, C=C, **kw)
    torch.cuda.synchronize()
    return tuple(host(t) for t in out)
