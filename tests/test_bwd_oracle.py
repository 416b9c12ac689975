"""Pins of the fp64 reverse-mode oracle (``oracle.bwd``), CPU only.

The gradients are checked against central finite differences of the pinned
forward oracle (brute force on tiny inputs, every input element), against
the closed form the beta = 0 reduction gives, and across the 64-token replay
segments.  Planted mistakes in a copy of the reverse-mode source must fail.
"""
import ctypes
import os
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
from tests import pins

NAMES = ("q", "k", "v", "alpha", "mu", "beta", "eta")
GRADS = ("dq", "dk", "dv", "dalpha", "dmu", "dbeta", "deta")


def loss_terms(seed, T, dk, dv):
    rng = np.random.default_rng(500 + seed)
    return (rng.standard_normal((T, dv)), rng.standard_normal((dk, dv)), rng.standard_normal((dk, dv)))


def loss(p, dO, dST, dMT):
    O, ST, MT, _ = oracle.fwd(*(p[n] for n in NAMES), p["S0"], p["M0"])
    return float((O * dO).sum() + (ST * dST).sum() + (MT * dMT).sum())


def finite_differences(p, dO, dST, dMT, h=1e-6):
    out = {}
    for n, g in list(zip(NAMES, GRADS)) + [("S0", "dS0"), ("M0", "dM0")]:
        x = p[n]
        d = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            keep = x[idx]
            x[idx] = keep + h
            lp = loss(p, dO, dST, dMT)
            x[idx] = keep - h
            lm = loss(p, dO, dST, dMT)
            x[idx] = keep
            d[idx] = (lp - lm) / (2 * h)
        out[g] = d
    return out


def max_rel(a, b):
    return max(np.abs(a[n] - b[n]).max() / max(np.abs(b[n]).max(), 1e-30) for n in b)


def check_fd(bwd=oracle.bwd, seed=1, T=9, dk=3, dv=2, mu_range=(-1.0, 0.0)):
    p = pins.rng_problem(seed, T=T, dk=dk, dv=dv, mu_range=mu_range)
    dO, dST, dMT = loss_terms(seed, T, dk, dv)
    got = bwd(*(p[n] for n in NAMES), p["S0"], p["M0"], dO=dO, dST=dST, dMT=dMT)
    ref = finite_differences(p, dO, dST, dMT)
    return max_rel(got, ref)


@pytest.mark.parametrize("seed,T,dk,dv,mu_range", [(1, 9, 3, 2, (-1.0, 0.0)), (2, 5, 2, 4, (-3.0, -2.0)),
                                                   (3, 1, 3, 3, (-1.0, 0.0)), (4, 12, 4, 3, (-0.2, 0.0))])
def test_gradients_match_finite_differences(seed, T, dk, dv, mu_range):
    assert check_fd(seed=seed, T=T, dk=dk, dv=dv, mu_range=mu_range) < 1e-6


def test_gradients_across_replay_segments():
    # T = 70 crosses the 64-token checkpoint boundary; compare a sample of
    # elements on both sides of it with finite differences
    p = pins.rng_problem(7, T=70, dk=2, dv=2)
    dO, dST, dMT = loss_terms(7, 70, 2, 2)
    got = oracle.bwd(*(p[n] for n in NAMES), p["S0"], p["M0"], dO=dO, dST=dST, dMT=dMT)
    h = 1e-6
    for n, g in (("v", "dv"), ("alpha", "dalpha"), ("mu", "dmu"), ("k", "dk")):
        for t in (0, 30, 63, 64, 65, 69):
            idx = (t,) if p[n].ndim == 1 else (t, 1)
            keep = p[n][idx]
            p[n][idx] = keep + h
            lp = loss(p, dO, dST, dMT)
            p[n][idx] = keep - h
            lm = loss(p, dO, dST, dMT)
            p[n][idx] = keep
            fd = (lp - lm) / (2 * h)
            assert abs(got[g][idx] - fd) <= 1e-6 * max(1.0, abs(fd)), (n, t)


def test_beta_zero_closed_form():
    # beta = 0 leaves S_t = abar_t S0 (the momentum never reaches S), so with
    # only dS_T given: dS0 = abar_T dS_T and dalpha_t = abar_T / alpha_t <S0, dS_T>
    p = pins.rng_problem(8, T=6)
    p["beta"][:] = 0.0
    dST = np.random.default_rng(1).standard_normal(p["S0"].shape)
    g = oracle.bwd(*(p[n] for n in NAMES), p["S0"], p["M0"], dST=dST)
    abar = np.prod(p["alpha"])
    assert np.allclose(g["dS0"], abar * dST, rtol=1e-13, atol=1e-14)
    assert np.allclose(g["dalpha"], abar / p["alpha"] * (p["S0"] * dST).sum(), rtol=1e-12)
    for n in ("dq", "dv", "dmu", "deta", "dM0"):
        assert np.abs(g[n]).max() < 1e-14


def test_zero_upstream_gradient_gives_zero():
    p = pins.rng_problem(9, T=5)
    g = oracle.bwd(*(p[n] for n in NAMES), p["S0"], p["M0"])
    for v in g.values():
        assert not v.any()


# Planted mistakes in a copy of the reverse-mode source: each must fail the
# finite-difference pin.
SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "mdn_oracle.c")
MUTANTS = {
    "drop_state_term_in_vtilde": ("Sh[i * dv + j] = alpha * Sh[i * dv + j] - alpha * k[i] * dv_out[j];",
                                  "Sh[i * dv + j] = alpha * Sh[i * dv + j];"),
    "beta_sign": ("db -= Mn[i] * Sh[i];", "db += Mn[i] * Sh[i];"),
    "momentum_from_old_state": ("db -= Mn[i] * Sh[i];", "db -= Mp[i] * Sh[i];"),
    "no_beta_into_momentum": ("Mh[i] -= beta * Sh[i];", "Mh[i] -= 0.0 * Sh[i];"),
    "readout_previous_state": ("acc += Sn[i * dv + j] * dout[j];", "acc += Sp[i * dv + j] * dout[j];"),
    "missing_alpha_in_dk": ("dk_out[i] += alpha * dp;", "dk_out[i] += dp;"),
    "eta_dropped_in_dv": ("dv_out[j] = -eta * acc;", "dv_out[j] = -acc;"),
    "mu_not_applied": ("for (long i = 0; i < dk * dv; ++i) Mh[i] *= mu;",
                       "for (long i = 0; i < dk * dv; ++i) Mh[i] *= 1.0;"),
}


def mutant_bwd(name, tmpdir):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, name
    c, so = os.path.join(tmpdir, name + ".c"), os.path.join(tmpdir, name + ".so")
    with open(c, "w") as f:
        f.write(src.replace(old, new))
    subprocess.check_call(["gcc", "-O1", "-fPIC", "-shared", "-std=c99", "-o", so, c])
    lib = ctypes.CDLL(so)
    d = ctypes.POINTER(ctypes.c_double)
    L = ctypes.c_long
    lib.mdn_oracle_bwd.argtypes = [L, L, L, L] + [d] * 7 + [ctypes.c_void_p] * 2 + [d] + [ctypes.c_void_p] * 2 + [d] * 9

    def bwd(q, k, v, alpha, mu, beta, eta, S0, M0, dO, dST, dMT):
        T, dk = q.shape
        dv = v.shape[-1]
        arr = [np.ascontiguousarray(a, dtype=np.float64) for a in (q, k, v, alpha, mu, beta, eta)]
        S0, M0, dO, dST, dMT = (np.ascontiguousarray(a, dtype=np.float64) for a in (S0, M0, dO, dST, dMT))
        out = dict(dq=np.zeros((T, dk)), dk=np.zeros((T, dk)), dv=np.zeros((T, dv)), dalpha=np.zeros(T),
                   dmu=np.zeros(T), dbeta=np.zeros(T), deta=np.zeros(T), dS0=np.zeros((dk, dv)),
                   dM0=np.zeros((dk, dv)))
        P = lambda a: a.ctypes.data_as(d)
        lib.mdn_oracle_bwd(1, T, dk, dv, *(P(a) for a in arr), S0.ctypes.data, M0.ctypes.data, P(dO),
                           dST.ctypes.data, dMT.ctypes.data,
                           *(P(out[n]) for n in ("dq", "dk", "dv", "dalpha", "dmu", "dbeta", "deta", "dS0", "dM0")))
        return out
    return bwd


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    with tempfile.TemporaryDirectory() as tmp:
        assert check_fd(bwd=mutant_bwd(name, tmp)) > 1e-3, name


@pytest.mark.parametrize("seed,T,dk,dv,C,mu_range", [(1, 9, 3, 2, 4, (-1.0, 0.0)), (2, 40, 4, 3, 16, (-3.0, -2.0)),
                                                     (3, 70, 5, 4, 64, (-1.0, 0.0)), (4, 33, 3, 3, 8, (-0.3, 0.0)),
                                                     (5, 16, 2, 2, 1, (-1.0, 0.0))])
def test_chunk_restatement_of_the_backward(seed, T, dk, dv, C, mu_range):
    # the chunkwise reverse mode (states replayed from Vtilde, reverse carry of
    # dS/dM, coefficient adjoints to the gates) equals the token reverse mode
    from oracle import chunk_ref
    p = pins.rng_problem(seed, T=T, dk=dk, dv=dv, mu_range=mu_range)
    dO, dST, dMT = loss_terms(seed, T, dk, dv)
    ref = oracle.bwd(*(p[n] for n in NAMES), p["S0"], p["M0"], dO=dO, dST=dST, dMT=dMT)
    got = chunk_ref.chunk_bwd_head(*(p[n] for n in NAMES), p["S0"], p["M0"], dO, dST, dMT, C)
    assert max_rel(got, ref) < 1e-12
