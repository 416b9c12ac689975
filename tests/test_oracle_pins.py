"""Pins of the fp64 oracle (CPU only).

The oracle is checked against what the pages and mathematics fix, never
against a retyped copy of itself: the printed closed-form expansion, the
latent-loss gradient (by autodiff), the beta = 0 and mu = 0 reductions, the
printed eigenvalues of the momentum system, a hand-worked example, and the
chunkwise restatement (chunk-size invariance).  ``test_oracle_mutants.py``
shows that planted mistakes in the oracle fail these pins.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import chunk_ref
from tests import pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_closed_form_expansion_with_eta():
    assert pins.check_closed_form(oracle.fwd) < 1e-12


def test_closed_form_without_eta_does_not_hold():
    # The printed expansion (summary, step 2) omits eta; the recurrence of
    # step 1 only matches it with eta_i on each rank-1 term.
    assert pins.check_closed_form(oracle.fwd, use_eta=False) > 1e-2


def test_momentum_follows_latent_loss_gradient():
    assert pins.check_latent_gradient(oracle.fwd) < 1e-12


def test_beta_zero_reduction():
    assert pins.check_beta_zero(oracle.fwd) < 1e-12


def test_mu_zero_is_gated_delta_rule():
    assert pins.check_mu_zero_gdn(oracle.fwd) < 1e-12


@pytest.mark.parametrize("gates", [
    dict(alpha=0.6, mu=0.7, beta=0.35, eta=1.5),      # complex pair (damped oscillation)
    dict(alpha=0.9, mu=0.2, beta=0.1, eta=1.9),       # real pair
    dict(alpha=0.3, mu=0.95, beta=0.6, eta=0.4),
])
def test_second_order_eigenvalues(gates):
    assert pins.check_second_order_scalar(oracle.fwd, **gates) < 1e-12


def test_complex_pair_exists_for_some_gates():
    lp, lm = pins.eigen_pair(0.6, 0.7, 0.35, 1.5, 1.0)
    assert abs(lp.imag) > 0.1 and abs(lp) < 1.0


def test_block_spectrum_alpha_mu():
    assert pins.check_second_order_block(oracle.fwd) < 1e-12


def test_step_matches_fwd():
    assert pins.check_step_matches_fwd(oracle.fwd, oracle.step) < 1e-13


def test_inplace_step_equals_copying_step():
    rng = np.random.default_rng(8)
    B, H, d = 3, 2, 8
    S = rng.standard_normal((B, H, d, d))
    M = rng.standard_normal((B, H, d, d))
    args = [rng.standard_normal((B, H, d)) for _ in range(3)] + [rng.uniform(0.2, 1.0, (B, H)) for _ in range(4)]
    o, S1, M1, vt = oracle.step(*args, S, M)
    S2, M2 = S.copy(), M.copy()
    o2, S3, M3, vt2 = oracle.step(*args, S2, M2, inplace=True)
    assert S3 is S2 and M3 is M2
    assert np.array_equal(o, o2) and np.array_equal(vt, vt2)
    assert np.array_equal(S1, S2) and np.array_equal(M1, M2)
    with pytest.raises(ValueError):
        oracle.step(*args, S.astype(np.float32), M, inplace=True)


def test_hand_worked_example():
    with open(os.path.join(GOLDEN, "hand_worked_d1.json")) as f:
        g = json.load(f)
    col = lambda x: np.array(x, dtype=np.float64)[:, None]
    O, ST, MT, Vt = oracle.fwd(col(g["q"]), col(g["k"]), col(g["v"]), np.array(g["alpha"]),
                               np.array(g["mu"]), np.array(g["beta"]), np.array(g["eta"]),
                               np.array([[g["S0"]]]), np.array([[g["M0"]]]))
    fr = lambda s: float(Fraction(s))
    assert O[:, 0].tolist() == [fr(s) for s in g["expect_o"]]
    assert Vt[:, 0].tolist() == [fr(s) for s in g["expect_vtilde"]]
    assert ST[0, 0] == fr(g["expect_S_T"]) and MT[0, 0] == fr(g["expect_M_T"])


@pytest.mark.parametrize("C", [1, 2, 4, 8, 16, 32, 64, 24])
def test_chunk_restatement_matches_recurrence(C):
    # Summary, novelty point 1: the chunkwise algorithm is an exact (strictly
    # causal) reformulation, so any chunk size -- including one that leaves a
    # ragged last chunk (24 does not divide 100) -- reproduces the recurrence.
    rng = np.random.default_rng(7)
    p = pins.rng_problem(11, T=100, dk=8, dv=5)
    S0 = rng.standard_normal((8, 5)) * 0.1
    M0 = rng.standard_normal((8, 5)) * 0.1
    ref = oracle.fwd(p["q"], p["k"], p["v"], p["alpha"], p["mu"], p["beta"], p["eta"], S0, M0)
    got = chunk_ref.chunk_fwd(p["q"], p["k"], p["v"], p["alpha"], p["mu"], p["beta"], p["eta"],
                              S0, M0, C=C)
    for a, b in zip(ref, got):
        assert np.abs(a - b).max() <= 1e-12 * max(1.0, np.abs(a).max())


def test_chunk_restatement_strong_momentum_gates():
    # Long-context regime: log mu ~ U[-2,-1.5], alpha near cos^2(theta).
    from linear_attention_sequence_mdn_amd import inputs
    x = inputs.make_chunk_inputs(1, 2, 192, 16, C=64, dtype="f32", seed=5,
                                 mu_range=(-2.0, -1.5), a_range=(5.0, 10.0))
    ref = oracle.fwd(x.q, x.k, x.v, x.alpha, x.mu, x.beta, x.eta)
    got = chunk_ref.chunk_fwd(x.q, x.k, x.v, x.alpha, x.mu, x.beta, x.eta, C=64)
    for a, b in zip(ref, got):
        assert np.abs(a - b).max() <= 1e-12 * max(1.0, np.abs(a).max())


def test_coefficients_products_vs_logdomain():
    # Summary, steps 2 and 5: the log-domain route (cumsum, logcumsumexp) and
    # the printed closed forms give the same coefficients as direct products.
    p = pins.rng_problem(3, T=16)
    d = chunk_ref.coefficients(p["alpha"], p["mu"], p["beta"], p["eta"])
    lg = chunk_ref.coefficients_logdomain(p["alpha"], p["mu"], p["beta"], p["eta"])
    for key in ("abar", "mubar", "b", "gamma", "Gamma"):
        assert np.abs(d[key] - lg[key]).max() <= 1e-12 * np.abs(d[key]).max(), key
    assert np.allclose(np.diag(d["gamma"]), p["beta"], rtol=0, atol=1e-15)
    assert np.all(np.triu(d["gamma"], 1) == 0)


def test_coefficients_with_zero_gates_are_finite():
    # Direct products stay exact when a gate is exactly zero (mu = 0 is the
    # GDN ablation); the log-domain route would form log(0).
    p = pins.rng_problem(4, T=12)
    mu = p["mu"].copy()
    mu[5] = 0.0
    d = chunk_ref.coefficients(p["alpha"], mu, p["beta"], p["eta"])
    assert np.all(np.isfinite(d["Gamma"])) and np.all(np.isfinite(d["b"]))
    # after the zero, tokens before it no longer feed the momentum
    assert np.all(d["gM"][:5] == 0.0)


def test_geometric_reordering_identity():
    # Summary, step 3: sum_i sum_{j<=i} a_i b_j == sum_i sum_{j>=i} a_j b_i.
    rng = np.random.default_rng(0)
    a, b = rng.standard_normal(37), rng.standard_normal(37)
    row = sum(a[i] * b[j] for i in range(37) for j in range(i + 1))
    colscan = sum(a[j] * b[i] for i in range(37) for j in range(i, 37))
    assert abs(row - colscan) < 1e-12
    # and the gamma double sum taken in both orders
    p = pins.rng_problem(5, T=9)
    La = chunk_ref._decay_matrix(p["alpha"])
    Lm = chunk_ref._decay_matrix(p["mu"])
    g1 = np.zeros((9, 9))
    g2 = np.zeros((9, 9))
    for r in range(9):
        for j in range(r + 1):          # row scan over j, inner over i <= j
            for i in range(j + 1):
                g1[r, i] += La[r, j] * p["beta"][j] * Lm[j, i]
        for i in range(r + 1):          # column scan over i, inner over j >= i
            for j in range(i, r + 1):
                g2[r, i] += La[r, j] * p["beta"][j] * Lm[j, i]
    assert np.abs(g1 - g2).max() < 1e-14
    assert np.abs(g1 - chunk_ref.coefficients(p["alpha"], p["mu"], p["beta"], p["eta"])["gamma"]).max() < 1e-14


def test_split_resume():
    p = pins.rng_problem(6, T=20)
    full = oracle.fwd(p["q"], p["k"], p["v"], p["alpha"], p["mu"], p["beta"], p["eta"], p["S0"], p["M0"])
    a = oracle.fwd(*(p[n][:9] for n in ("q", "k", "v", "alpha", "mu", "beta", "eta")), p["S0"], p["M0"])
    b = oracle.fwd(*(p[n][9:] for n in ("q", "k", "v", "alpha", "mu", "beta", "eta")), a[1], a[2])
    assert np.array_equal(full[0], np.concatenate([a[0], b[0]]))
    assert np.array_equal(full[1], b[1]) and np.array_equal(full[2], b[2])


def test_empty_sequence_returns_initial_state():
    p = pins.rng_problem(8, T=3)
    O, ST, MT, Vt = oracle.fwd(p["q"][:0], p["k"][:0], p["v"][:0], p["alpha"][:0], p["mu"][:0],
                               p["beta"][:0], p["eta"][:0], p["S0"], p["M0"])
    assert O.shape == (0, 2) and np.array_equal(ST, p["S0"]) and np.array_equal(MT, p["M0"])


def test_batched_heads_are_independent():
    p = pins.rng_problem(9, T=11)
    stack = lambda x: np.stack([x, 0.5 * x])
    out = oracle.fwd(*(stack(p[n]) for n in ("q", "k", "v")), *(stack(p[n]) for n in ("alpha", "mu", "beta", "eta")))
    single = oracle.fwd(*(0.5 * p[n] for n in ("q", "k", "v")), *(0.5 * p[n] for n in ("alpha", "mu", "beta", "eta")))
    for a, b in zip(out, single):
        assert np.array_equal(a[1], b)
