"""Seeded synthetic inputs for the MDN hot path.

This module is shared by the oracle side (tests, CPU baseline) and the GPU side
(tests, bench).  It holds none of the method's arithmetic: it only draws
random numbers and maps them through the gate parametrisation that produces
the recurrence's inputs.  It imports nothing from the HIP binding or from the
oracle.

Recipe (fixed draw order, ``numpy.random.default_rng(seed)``, fp64 draws):

1. q, k, v ~ N(0, 1), shape ``[B, H, T, d]``; every k_t is L2-normalised over dk.
2. x, a, b, each ``[B, H, T]``: x ~ N(0,1); a ~ N(0,1) (or U[a_lo, a_hi]);
   b ~ N(0,1).
3. log mu ~ U[mu_lo, mu_hi).
4. eta = tanh(x) + 1;  theta = arctan(eta * s) with s = 1;
   alpha = cos^2(theta) * sigmoid(a);  beta = sin^2(theta) * sigmoid(b);
   mu = exp(log mu).
   This is the stable gate parametrisation of the MDN summary at
   paper.rainbus.top (method walk-through, step 6) and of the ijyty.com
   article on MDN (section 5): alpha_max + beta_max = 1, eta in (0, 2).
5. Optional S0, M0 ~ N(0, std^2) (drawn after the gates).

q, k, v are rounded to the compute dtype (bf16: round-to-nearest-even) here,
so that the oracle and the GPU receive bit-identical values; gates and states
are fp32.  The workloads (shapes) mirror the pages' layer shapes and lengths:
the 4k training length and the 16k long-context length of the ijyty.com
article (section 7) stand in for the pages' datasets, none of which is used.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Iterator, Optional

import numpy as np


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float values to the nearest bf16 (ties to even); returns float32."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    u = (u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    return u.astype(np.uint32).view(np.float32)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _gates(x, a, b, logmu, s=1.0):
    eta = np.tanh(x) + 1.0
    theta = np.arctan(eta * s)
    alpha = np.cos(theta) ** 2 * _sigmoid(a)
    beta = np.sin(theta) ** 2 * _sigmoid(b)
    mu = np.exp(logmu)
    return alpha, mu, beta, eta


@dataclass
class ChunkInputs:
    B: int
    H: int
    T: int
    dk: int
    dv: int
    C: int
    dtype: str                   # "f32" or "bf16": dtype of q, k, v, O, Vtilde
    q: np.ndarray                # float32 [B,H,T,dk], values exact in ``dtype``
    k: np.ndarray
    v: np.ndarray                # float32 [B,H,T,dv]
    alpha: np.ndarray            # float32 [B,H,T]
    mu: np.ndarray
    beta: np.ndarray
    eta: np.ndarray
    S0: Optional[np.ndarray] = None   # float32 [B,H,dk,dv] or None (zero)
    M0: Optional[np.ndarray] = None
    meta: dict = field(default_factory=dict)


def make_chunk_inputs(B, H, T, dk, dv=None, C=64, dtype="bf16", seed=0,
                      mu_range=(-1.0, 0.0), a_range=None, state_std=None) -> ChunkInputs:
    """Draw one chunk-forward workload following the recipe above."""
    dv = dk if dv is None else dv
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, T, dk))
    k = rng.standard_normal((B, H, T, dk))
    v = rng.standard_normal((B, H, T, dv))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    x = rng.standard_normal((B, H, T))
    if a_range is None:
        a = rng.standard_normal((B, H, T))
    else:
        a = rng.uniform(a_range[0], a_range[1], (B, H, T))
    b = rng.standard_normal((B, H, T))
    logmu = rng.uniform(mu_range[0], mu_range[1], (B, H, T))
    alpha, mu, beta, eta = _gates(x, a, b, logmu)
    S0 = M0 = None
    if state_std is not None:
        S0 = (rng.standard_normal((B, H, dk, dv)) * state_std).astype(np.float32)
        M0 = (rng.standard_normal((B, H, dk, dv)) * state_std).astype(np.float32)
    cast = round_to_bf16 if dtype == "bf16" else (lambda t: np.asarray(t, dtype=np.float32))
    return ChunkInputs(B, H, T, dk, dv, C, dtype, cast(q), cast(k), cast(v),
                       alpha.astype(np.float32), mu.astype(np.float32),
                       beta.astype(np.float32), eta.astype(np.float32), S0, M0,
                       meta=dict(seed=seed, mu_range=mu_range, a_range=a_range,
                                 state_std=state_std))


@dataclass
class DecodeStep:
    q: np.ndarray      # float32 [B,H,dk] (values exact in dtype)
    k: np.ndarray
    v: np.ndarray      # float32 [B,H,dv]
    alpha: np.ndarray  # float32 [B,H]
    mu: np.ndarray
    beta: np.ndarray
    eta: np.ndarray


def decode_steps(B, H, dk, dv=None, steps=128, dtype="bf16", seed=3,
                 mu_range=(-1.0, 0.0)) -> Iterator[DecodeStep]:
    """Per-step decode inputs: each step draws q, k, v, x, a, b, log mu in order."""
    dv = dk if dv is None else dv
    rng = np.random.default_rng(seed)
    cast = round_to_bf16 if dtype == "bf16" else (lambda t: np.asarray(t, dtype=np.float32))
    for _ in range(steps):
        q = rng.standard_normal((B, H, dk))
        k = rng.standard_normal((B, H, dk))
        v = rng.standard_normal((B, H, dv))
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        x = rng.standard_normal((B, H))
        a = rng.standard_normal((B, H))
        b = rng.standard_normal((B, H))
        logmu = rng.uniform(mu_range[0], mu_range[1], (B, H))
        alpha, mu, beta, eta = _gates(x, a, b, logmu)
        yield DecodeStep(cast(q), cast(k), cast(v), alpha.astype(np.float32),
                         mu.astype(np.float32), beta.astype(np.float32), eta.astype(np.float32))


# The five workloads: the tiny correctness case, the 400M-layer and 1.3B-layer
# chunk shapes (4k training length), the decode step and the 16k long-context
# case with momentum near its clamp and alpha near its upper bound.
CONFIGS = {
    0: dict(kind="chunk", B=1, H=1, T=64, dk=16, dv=16, C=16, dtype="f32", seed=0),
    1: dict(kind="chunk", B=8, H=8, T=4096, dk=128, dv=128, C=64, dtype="bf16", seed=1),
    2: dict(kind="chunk", B=4, H=16, T=4096, dk=128, dv=128, C=64, dtype="bf16", seed=2,
            state_std=0.02),
    3: dict(kind="decode", B=256, H=16, dk=128, dv=128, steps=128, dtype="bf16", seed=3),
    4: dict(kind="chunk", B=1, H=16, T=16384, dk=128, dv=128, C=64, dtype="bf16", seed=4,
            mu_range=(-2.0, -1.5), a_range=(5.0, 10.0)),
}

CONFIG_NAMES = {
    0: "tiny-f32 B1 H1 T64 d16 C16",
    1: "400M-layer B8 H8 T4096 d128 C64 bf16",
    2: "1.3B-layer B4 H16 T4096 d128 C64 bf16 S0/M0~N(0,0.02)",
    3: "decode B256 H16 d128 bf16 x128 steps",
    4: "long-context B1 H16 T16384 d128 C64 bf16 logmu~U[-2,-1.5]",
}


def config_inputs(index: int) -> ChunkInputs:
    """Inputs of a chunk-forward workload by index (0, 1, 2 or 4)."""
    c = dict(CONFIGS[index])
    assert c.pop("kind") == "chunk"
    return make_chunk_inputs(**c)


@dataclass
class VarlenInputs:
    """A packed variable-length batch: sequence i is tokens [cu[i], cu[i+1])
    of every head; per-sequence states are [nseq, H, dk, dv]."""
    H: int
    T: int                       # packed length = sum of lengths
    dk: int
    dv: int
    C: int
    dtype: str
    lengths: np.ndarray          # int64 [nseq]
    cu: np.ndarray               # int32 [nseq + 1]
    q: np.ndarray                # float32 [H,T,dk]
    k: np.ndarray
    v: np.ndarray                # float32 [H,T,dv]
    alpha: np.ndarray            # float32 [H,T]
    mu: np.ndarray
    beta: np.ndarray
    eta: np.ndarray
    S0: Optional[np.ndarray] = None   # float32 [nseq,H,dk,dv] or None (zero)
    M0: Optional[np.ndarray] = None


def serving_lengths(total, lo, hi, seed=0) -> np.ndarray:
    """Sequence lengths ~ U{lo..hi} drawn until they sum to ``total`` (the
    last one cut to fit): the length mix of a packed prefill batch."""
    rng = np.random.default_rng(seed)
    out, acc = [], 0
    while acc < total:
        n = int(min(rng.integers(lo, hi + 1), total - acc))
        out.append(n)
        acc += n
    return np.asarray(out, dtype=np.int64)


def make_varlen_inputs(H, lengths, dk, dv=None, C=64, dtype="bf16", seed=0,
                       mu_range=(-1.0, 0.0), state_std=None) -> VarlenInputs:
    """Packed batch with the chunk recipe above: q, k, v and gates drawn as
    for one ``[1, H, sum(lengths)]`` workload, then the per-sequence initial
    states (if ``state_std``) as ``[nseq, H, dk, dv]``."""
    lengths = np.asarray(lengths, dtype=np.int64)
    T = int(lengths.sum())
    x = make_chunk_inputs(1, H, T, dk, dv, C=C, dtype=dtype, seed=seed, mu_range=mu_range)
    dv = x.dv
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    S0 = M0 = None
    if state_std is not None:
        rng = np.random.default_rng(seed + 7919)
        S0 = (rng.standard_normal((len(lengths), H, dk, dv)) * state_std).astype(np.float32)
        M0 = (rng.standard_normal((len(lengths), H, dk, dv)) * state_std).astype(np.float32)
    return VarlenInputs(H, T, dk, dv, C, dtype, lengths, cu, x.q[0], x.k[0], x.v[0],
                        x.alpha[0], x.mu[0], x.beta[0], x.eta[0], S0, M0)


@dataclass
class GateInputs:
    """Raw projection outputs for the gate pre-operation: x, a, b, mu_log
    ``[B, H, T]`` fp32, q, k ``[B, H, T, dk]`` (values exact in ``dtype``)
    and one correction scalar d per head."""
    x: np.ndarray
    a: np.ndarray
    b: np.ndarray
    mu_log: np.ndarray
    q: np.ndarray
    k: np.ndarray
    d: np.ndarray
    dtype: str


def make_gate_inputs(B, H, T, dk, dtype="bf16", seed=0, mu_range=(-3.0, 0.5)) -> GateInputs:
    """Draw order: x, a, b ~ N(0, 1); mu_log ~ U[mu_range) (wide enough to
    exercise both ends of the clamp); q, k ~ N(0, 1); d ~ U[0, 1) per head."""
    rng = np.random.default_rng(seed)
    f32 = lambda t: np.asarray(t, dtype=np.float32)
    x = f32(rng.standard_normal((B, H, T)))
    a = f32(rng.standard_normal((B, H, T)))
    b = f32(rng.standard_normal((B, H, T)))
    mu_log = f32(rng.uniform(mu_range[0], mu_range[1], (B, H, T)))
    q = rng.standard_normal((B, H, T, dk))
    k = rng.standard_normal((B, H, T, dk))
    if dtype == "bf16":
        q, k = round_to_bf16(q), round_to_bf16(k)
    d = f32(rng.uniform(0.0, 1.0, H))
    return GateInputs(x, a, b, mu_log, f32(q), f32(k), d, dtype)
