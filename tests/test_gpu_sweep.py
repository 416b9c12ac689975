"""Seeded random sweep of shapes and gate regimes: the chunk forward, the
backward and the decode step against the fp64 oracle, every output compared
as a whole tensor.  The cases are drawn once from a fixed seed, so a failure
names a reproducible case; each case prints its parameters before it runs."""
import numpy as np
import pytest

import oracle
from linear_attention_sequence_mdn_amd import inputs
from tests.gpu_util import TOL, dev, host, note, rel_err, run_chunk, torch_mod
from tests.test_gpu_bwd import GRADS, ref_bwd, run_bwd, upstream

pytestmark = pytest.mark.gpu

NAMES = ("O", "S_T", "M_T", "Vtilde")
# gate regimes: the workloads' default draw, and strong momentum with alpha
# near its bound (the long-context recipe)
REGIMES = {"default": dict(), "strong": dict(mu_range=(-2.0, -1.5), a_range=(5.0, 10.0))}


def _draw(n, seed, dims=(16, 32, 64, 128), tmax=300):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        dtype = ("f32", "bf16")[rng.integers(2)]
        d = int(rng.choice(dims))
        C = int(rng.choice((16, 32, 64)))
        # lengths: empty-ish, shorter than a chunk, exact multiples and ragged
        T = int(rng.choice((1, C - 1, C, C + 1, 2 * C, int(rng.integers(2, tmax + 1)))))
        T = max(T, 1)
        B, H = int(rng.integers(1, 4)), int(rng.integers(1, 5))
        state = (None, 0.02 if dtype == "bf16" else 0.3)[rng.integers(2)]
        regime = ("default", "strong")[rng.integers(2)]
        cases.append((i, dtype, d, C, T, B, H, state, regime))
    return cases


FWD_CASES = _draw(24, 2026)
BWD_CASES = _draw(8, 2027, dims=(16, 32, 64), tmax=160)


def _inputs(i, dtype, d, C, T, B, H, state, regime, salt):
    return inputs.make_chunk_inputs(B, H, T, d, C=C, dtype=dtype, seed=salt + 17 * i, state_std=state,
                                    **REGIMES[regime])


@pytest.mark.parametrize("case", FWD_CASES, ids=lambda c: "fwd%02d-%s-d%d-C%d-T%d-B%dH%d-%s-%s" % (
    c[0], c[1], c[2], c[3], c[4], c[5], c[6], "S" if c[7] else "0", c[8]))
def test_sweep_chunk_forward(case):
    i, dtype, d, C, T, B, H, state, regime = case
    x = _inputs(*case, salt=5000)
    note(f"sweep fwd {case}")
    got = run_chunk(x)
    ref = oracle.fwd(x.q, x.k, x.v, x.alpha, x.mu, x.beta, x.eta, x.S0, x.M0)
    errs = {n: rel_err(g, r) for n, g, r in zip(NAMES, got, ref)}
    note("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    for n, e in errs.items():
        assert e <= TOL[dtype], (case, n, e)


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "bwd%02d-%s-d%d-C%d-T%d-B%dH%d-%s-%s" % (
    c[0], c[1], c[2], c[3], c[4], c[5], c[6], "S" if c[7] else "0", c[8]))
def test_sweep_chunk_backward(case):
    i, dtype, d, C, T, B, H, state, regime = case
    x = _inputs(*case, salt=7000)
    dO, dST, dMT = upstream(x, 60 + i, with_states=bool(i % 2))
    note(f"sweep bwd {case}")
    got = run_bwd(x, dO, dST, dMT)
    ref = ref_bwd(x, dO, dST, dMT)
    errs = {n: rel_err(got[n], ref[n]) for n in GRADS}
    note("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    for n, e in errs.items():
        assert e <= TOL[dtype], (case, n, e)


@pytest.mark.parametrize("dtype,d,B,H,steps,seed", [("f32", 16, 3, 2, 40, 1), ("bf16", 32, 5, 3, 30, 2),
                                                      ("f32", 64, 2, 2, 20, 3), ("bf16", 128, 4, 2, 25, 4),
                                                      ("bf16", 64, 7, 1, 33, 5)])
def test_sweep_decode_steps(dtype, d, B, H, steps, seed):
    """Consecutive mdn_step calls from a nonzero state against the oracle's
    step, every step's o and the final states compared."""
    import linear_attention_sequence_mdn_amd as mdn
    torch = torch_mod()
    rng = np.random.default_rng(8000 + seed)
    S0 = (rng.standard_normal((B, H, d, d)) * 0.05).astype(np.float32)
    M0 = (rng.standard_normal((B, H, d, d)) * 0.05).astype(np.float32)
    S, M = dev(S0), dev(M0)
    Sr, Mr = S0.astype(np.float64), M0.astype(np.float64)
    note(f"sweep decode {dtype} d={d} B={B} H={H} steps={steps}")
    worst = 0.0
    for st in inputs.decode_steps(B, H, d, steps=steps, dtype=dtype, seed=8100 + seed):
        o = mdn.step(dev(st.q, dtype), dev(st.k, dtype), dev(st.v, dtype), dev(st.alpha), dev(st.mu),
                     dev(st.beta), dev(st.eta), S, M)
        orf, _, _, _ = oracle.step(st.q, st.k, st.v, st.alpha, st.mu, st.beta, st.eta, Sr, Mr, inplace=True)
        worst = max(worst, rel_err(host(o), orf))
    torch.cuda.synchronize()
    es, em = rel_err(host(S), Sr), rel_err(host(M), Mr)
    note(f"  o={worst:.2e} S={es:.2e} M={em:.2e}")
    assert worst <= TOL[dtype] and es <= TOL[dtype] and em <= TOL[dtype]


@pytest.mark.parametrize("dtype,d,C,T,B,H", [("bf16", 128, 64, 130, 2, 80), ("bf16", 128, 32, 70, 3, 55),
                                             ("f32", 128, 32, 40, 2, 37)])
def test_grid_beyond_one_wave_of_workgroups(dtype, d, C, T, B, H):
    """More heads than the device holds inter workgroups at once (each uses
    most of a compute unit's LDS), so the workgroups run in several rounds;
    B*H both a multiple of 8 (the XCD-aware head map) and not."""
    x = inputs.make_chunk_inputs(B, H, T, d, C=C, dtype=dtype, seed=600 + d + H,
                                 state_std=0.02 if dtype == "bf16" else 0.3)
    note(f"chunk {dtype} d={d} C={C} T={T} B={B} H={H}: {B * H} heads")
    got = run_chunk(x)
    ref = oracle.fwd(x.q, x.k, x.v, x.alpha, x.mu, x.beta, x.eta, x.S0, x.M0)
    errs = {n: rel_err(g, r) for n, g, r in zip(NAMES, got, ref)}
    note("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    for n, e in errs.items():
        assert e <= TOL[dtype], (n, e)


@pytest.mark.parametrize("dtype,d,C,T,B,H", [("bf16", 128, 64, 130, 2, 80), ("bf16", 64, 64, 70, 3, 55),
                                             ("f32", 64, 32, 40, 2, 37)])
def test_bwd_grid_beyond_one_wave_of_workgroups(dtype, d, C, T, B, H):
    """The backward with more heads than the device holds carry workgroups at
    once (one per compute unit at d = 128), so they run in several rounds;
    B*H both a multiple of 8 (the XCD-aware head map) and not.  Every gradient
    is compared as a whole tensor."""
    x = inputs.make_chunk_inputs(B, H, T, d, C=C, dtype=dtype, seed=900 + d + H,
                                 state_std=0.02 if dtype == "bf16" else 0.3)
    dO, dST, dMT = upstream(x, 70 + H)
    note(f"bwd {dtype} d={d} C={C} T={T} B={B} H={H}: {B * H} heads")
    got = run_bwd(x, dO, dST, dMT)
    ref = ref_bwd(x, dO, dST, dMT)
    errs = {n: rel_err(got[n], ref[n]) for n in GRADS}
    note("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    for n, e in errs.items():
        assert e <= TOL[dtype], (n, e)
