"""Pins of the packed variable-length oracle (CPU only).

A packed batch is the recurrence (MDN summary, paper.rainbus.top, method
walk-through step 1) restarted at every sequence start from that sequence's
own state.  The pins tie ``oracle.fwd_varlen`` to properties that definition
fixes, not to a copy of itself: a sequence split at any token and resumed
from the carried state reproduces the unsplit run (so each sequence reads its
own S0 and writes its own slice and S_T); tokens of one sequence never reach
another; empty sequences return their initial state; per-head states follow
the [nseq, H] layout.
"""
import inspect
import textwrap

import numpy as np
import pytest

import oracle
from tests import pins

NAMES = ("q", "k", "v", "alpha", "mu", "beta", "eta")


def _heads(seeds, T):
    """[H, T, .] arrays from one single-head problem per seed."""
    ps = [pins.rng_problem(s, T=T) for s in seeds]
    return {n: np.stack([p[n] for p in ps]) for n in NAMES + ("S0", "M0")}


def check_split_resume(fv=oracle.fwd_varlen):
    # one head-pair sequence of 23 tokens, cut into packed pieces 0|7|9|7
    # whose initial states are the states the unsplit run reaches at the cuts
    p = _heads([31, 32], T=23)
    full = oracle.fwd(*(p[n] for n in NAMES), p["S0"], p["M0"])
    cuts = [0, 0, 7, 16, 23]
    S0 = np.zeros((4, 2) + p["S0"].shape[1:])
    M0 = np.zeros_like(S0)
    for i, c in enumerate(cuts[:-1]):
        _, S, M, _ = oracle.fwd(*(p[n][:, :c] for n in NAMES), p["S0"], p["M0"])
        S0[i], M0[i] = S, M
    O, ST, MT, Vt = fv(*(p[n] for n in NAMES), cuts, S0, M0)
    assert np.allclose(O, full[0], rtol=1e-12, atol=1e-12)
    assert np.allclose(Vt, full[3], rtol=1e-12, atol=1e-12)
    assert np.allclose(ST[-1], full[1], rtol=1e-12, atol=1e-12)
    assert np.allclose(MT[-1], full[2], rtol=1e-12, atol=1e-12)
    # the empty first piece returns its initial state, the others the
    # state at their end, which is the next piece's start
    assert np.array_equal(ST[0], S0[0]) and np.array_equal(MT[0], M0[0])
    for i in range(1, 3):
        assert np.allclose(ST[i], S0[i + 1], rtol=1e-12, atol=1e-12)
        assert np.allclose(MT[i], M0[i + 1], rtol=1e-12, atol=1e-12)


def check_isolation(fv=oracle.fwd_varlen):
    p = _heads([41, 42, 43], T=30)
    cu = [0, 11, 11, 30]
    S0 = np.stack([p["S0"], 0.5 * p["S0"], -p["S0"]])
    M0 = np.stack([p["M0"], 0.5 * p["M0"], -p["M0"]])
    base = fv(*(p[n] for n in NAMES), cu, S0, M0)
    q = dict(p)
    q["v"] = p["v"].copy()
    q["v"][:, :11] += 1.0                         # change sequence 0 only
    q["alpha"] = p["alpha"].copy()
    q["alpha"][:, :11] *= 0.5
    pert = fv(*(q[n] for n in NAMES), cu, S0, M0)
    assert np.array_equal(base[0][:, 11:], pert[0][:, 11:])
    assert np.array_equal(base[1][1:], pert[1][1:]) and np.array_equal(base[2][1:], pert[2][1:])
    assert np.abs(base[0][:, :11] - pert[0][:, :11]).max() > 1e-3
    assert np.abs(base[1][0] - pert[1][0]).max() > 1e-3


def check_own_state(fv=oracle.fwd_varlen):
    p = _heads([51, 52], T=12)
    cu = [0, 5, 12]
    rng = np.random.default_rng(5)
    S0 = rng.standard_normal((2, 2) + p["S0"].shape[1:])
    M0 = rng.standard_normal((2, 2) + p["M0"].shape[1:])
    O, ST, MT, Vt = fv(*(p[n] for n in NAMES), cu, S0, M0)
    for i, (a, b) in enumerate(zip(cu[:-1], cu[1:])):
        for h in range(2):
            o, st, mt, vt = oracle.fwd(*(p[n][h, a:b] for n in NAMES), S0[i, h], M0[i, h])
            assert np.array_equal(O[h, a:b], o) and np.array_equal(Vt[h, a:b], vt)
            assert np.array_equal(ST[i, h], st) and np.array_equal(MT[i, h], mt)


def check_zero_state(fv=oracle.fwd_varlen):
    p = _heads([61], T=9)
    cu = [0, 4, 9]
    z = np.zeros((2, 1) + p["S0"].shape[1:])
    a = fv(*(p[n] for n in NAMES), cu)
    b = fv(*(p[n] for n in NAMES), cu, z, z)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def check_prefill_decode(fv=oracle.fwd_varlen):
    # the prefill -> decode handoff: S_T, M_T of a packed prefill feed the
    # one-token step, which must give the next token of the unsplit run
    p = _heads([71, 72], T=14)
    cu = [0, 13]
    _, ST, MT, _ = fv(*(p[n][:, :13] for n in NAMES), cu, p["S0"][None], p["M0"][None])
    o, S, M, vt = oracle.step(*(p[n][:, 13] for n in NAMES), ST[0], MT[0])
    full = oracle.fwd(*(p[n] for n in NAMES), p["S0"], p["M0"])
    assert np.allclose(o, full[0][:, 13], rtol=1e-12, atol=1e-12)
    assert np.allclose(vt, full[3][:, 13], rtol=1e-12, atol=1e-12)
    assert np.allclose(S, full[1], rtol=1e-12, atol=1e-12) and np.allclose(M, full[2], rtol=1e-12, atol=1e-12)


CHECKS = (check_split_resume, check_isolation, check_own_state, check_zero_state, check_prefill_decode)


@pytest.mark.parametrize("check", CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check()


# Planted mistakes in a copy of fwd_varlen, each a plausible slip; every one
# must fail at least one pin above.
MUTANTS = {
    "state_carried_across_sequences": (
        "s0 = None if S0 is None else S0[i]",
        "s0 = (None if S0 is None else S0[i]) if i == 0 else ST[i - 1]"),
    "states_in_reverse_order": (
        "s0 = None if S0 is None else S0[i]", "s0 = None if S0 is None else S0[nseq - 1 - i]"),
    "bounds_one_token_long": (
        "a, b = int(cu[i]), int(cu[i + 1])", "a, b = int(cu[i]), min(int(cu[i + 1]) + 1, T)"),
    "empty_sequence_zero_state": (
        "ST[i] = 0.0 if s0 is None else s0", "ST[i] = 0.0"),
    "head_state_transposed": (
        "m0 = None if M0 is None else M0[i]",
        "m0 = None if M0 is None else M0[i][::-1]"),
}


def _mutant(old, new):
    src = textwrap.dedent(inspect.getsource(oracle.fwd_varlen))
    assert src.count(old) == 1, old
    ns = dict(vars(oracle))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    return ns["fwd_varlen"]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    fv = _mutant(*MUTANTS[name])
    failed = 0
    for check in CHECKS:
        try:
            check(fv)
        except AssertionError:
            failed += 1
    assert failed > 0, name
