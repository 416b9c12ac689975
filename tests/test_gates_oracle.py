"""Pins of the fp64 gate oracle (oracle/gates_ref.py) to what the pages and
the mathematics fix, independently of the oracle's own formulas.  Each check
takes the functions it pins, so that planted mistakes in a copy of the
oracle can be shown to fail at least one of them."""
import inspect
import textwrap

import numpy as np
import pytest

from oracle import gates_ref


def _tanh_by_exp(x):
    e = np.exp(2.0 * np.asarray(x, dtype=np.float64))
    return (e - 1.0) / (e + 1.0)


def check_gate_maxima_are_the_arctan_closed_forms(gates=gates_ref.gates):
    # cos^2(arctan u) = 1/(1+u^2), sin^2(arctan u) = u^2/(1+u^2); with the
    # sigmoid inputs saturated (a, b = 40) the gates equal their maxima.
    rng = np.random.default_rng(0)
    x = rng.standard_normal(1000) * 2
    big = np.full_like(x, 40.0)
    for s in (1.0, 0.5, 2.0):
        alpha, mu, beta, eta = gates(x, big, big, np.zeros_like(x), s=s)
        u = s * (_tanh_by_exp(x) + 1.0)
        np.testing.assert_allclose(eta, _tanh_by_exp(x) + 1.0, rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(alpha, 1.0 / (1.0 + u * u), rtol=1e-12, atol=1e-15)
        np.testing.assert_allclose(beta, u * u / (1.0 + u * u), rtol=1e-12, atol=1e-15)


def check_each_gate_follows_its_own_input(gates=gates_ref.gates):
    # alpha = alpha_max sigmoid(a), beta = beta_max sigmoid(b): one input
    # saturated open and the other shut, then the other way round, and a
    # sigmoid at zero (one half) beside a saturated one
    rng = np.random.default_rng(4)
    x = rng.standard_normal(500)
    hi, lo, zero = np.full_like(x, 40.0), np.full_like(x, -40.0), np.zeros_like(x)
    u2 = (_tanh_by_exp(x) + 1.0) ** 2
    amax, bmax = 1.0 / (1.0 + u2), u2 / (1.0 + u2)
    alpha, _, beta, _ = gates(x, hi, lo, zero)
    np.testing.assert_allclose(alpha, amax, rtol=1e-12)
    assert np.all(beta < 1e-15)
    alpha, _, beta, _ = gates(x, lo, hi, zero)
    np.testing.assert_allclose(beta, bmax, rtol=1e-12)
    assert np.all(alpha < 1e-15)
    alpha, _, beta, _ = gates(x, zero, hi, zero)
    np.testing.assert_allclose(alpha, 0.5 * amax, rtol=1e-12)
    np.testing.assert_allclose(beta, bmax, rtol=1e-12)


def check_gates_respect_the_stability_bound(gates=gates_ref.gates):
    # alpha_max + beta_max = cos^2 + sin^2 = 1, so alpha + beta <= 1 and
    # eta in (0, 2) (summary, step 6; article, section 5)
    rng = np.random.default_rng(1)
    x, a, b = (rng.standard_normal(200000) * 3 for _ in range(3))
    alpha, mu, beta, eta = gates(x, a, b, rng.uniform(-3, 0.5, x.shape))
    assert np.all(alpha + beta <= 1.0 + 1e-15)
    assert np.all((eta > 0) & (eta < 2)) and np.all((alpha > 0) & (beta > 0))


def check_gates_special_values(gates=gates_ref.gates):
    # x = 0: eta = 1, theta = pi/4, alpha_max = beta_max = 1/2; a = b = 0: sigmoid = 1/2
    alpha, mu, beta, eta = gates([0.0], [0.0], [0.0], [-0.5])
    assert eta[0] == 1.0
    assert abs(alpha[0] - 0.25) < 1e-15 and abs(beta[0] - 0.25) < 1e-15
    assert abs(mu[0] - np.exp(-0.5)) < 1e-15


def check_mu_clamp(gates=gates_ref.gates):
    ml = np.array([-3.0, -2.0, -1.0, 0.0, 0.7])
    _, mu, _, _ = gates(np.zeros(5), np.zeros(5), np.zeros(5), ml, mu_log_min=-2.0)
    np.testing.assert_allclose(mu, np.exp([-2.0, -2.0, -1.0, 0.0, 0.0]), rtol=1e-15)
    _, mu, _, _ = gates(np.zeros(5), np.zeros(5), np.zeros(5), ml, mu_log_min=-1.0)
    np.testing.assert_allclose(mu, np.exp([-1.0, -1.0, -1.0, 0.0, 0.0]), rtol=1e-15)


def _trace(alpha, mu, beta, eta, k2=1.0):
    # trace of the 2x2 block [[alpha (1 - beta eta |k|^2), -beta mu], [alpha eta |k|^2, mu]]
    # of the second-order system (summary, step 6); its determinant is
    # alpha mu > 0, so both eigenvalues have positive real part iff the trace does
    return alpha * (1.0 - beta * eta * k2) + mu


def check_clamp_keeps_the_eigenvalues_in_the_right_half_plane(gates=gates_ref.gates):
    # worst corner: eta -> 2, sigmoid(a), sigmoid(b) -> 1, mu at its clamp.
    # With log mu >= -2 the trace stays positive (eigenvalues in the right
    # half plane, as the pages state); with a clamp at -3 it does not, which
    # is why the pages need the bound.
    x = np.linspace(-1, 20, 4000)
    big = np.full_like(x, 40.0)
    for lo, sign in ((-2.0, 1), (-3.0, -1)):
        alpha, mu, beta, eta = gates(x, big, big, np.full_like(x, -10.0), mu_log_min=lo)
        tr = _trace(alpha, mu, beta, eta)
        assert (tr.min() > 0) == (sign > 0), (lo, tr.min())
    # random gates of the synthetic recipe: trace well above zero
    rng = np.random.default_rng(2)
    x, a, b = (rng.standard_normal(100000) for _ in range(3))
    alpha, mu, beta, eta = gates(x, a, b, rng.uniform(-1, 0, x.shape))
    assert _trace(alpha, mu, beta, eta).min() > 0.2


def check_query_correction(query_correction=gates_ref.query_correction):
    rng = np.random.default_rng(3)
    q = rng.standard_normal((2, 3, 5, 8))
    k = rng.standard_normal((2, 3, 5, 8))
    np.testing.assert_array_equal(query_correction(q, k, np.zeros(3)), q)
    np.testing.assert_array_equal(query_correction(q, q, np.ones(3)), np.zeros_like(q))
    d = np.array([0.5, 0.0, 2.0])
    out = query_correction(q, k, d)
    np.testing.assert_array_equal(out[:, 1], q[:, 1])
    np.testing.assert_allclose(out[:, 2], q[:, 2] - 2.0 * k[:, 2], rtol=0, atol=1e-15)


GATE_CHECKS = (check_gate_maxima_are_the_arctan_closed_forms, check_each_gate_follows_its_own_input,
               check_gates_respect_the_stability_bound, check_gates_special_values, check_mu_clamp,
               check_clamp_keeps_the_eigenvalues_in_the_right_half_plane)


@pytest.mark.parametrize("check", GATE_CHECKS + (check_query_correction,), ids=lambda c: c.__name__[6:])
def test_pin(check):
    check()


# Planted mistakes in a copy of the oracle, each a plausible slip; every one
# must fail at least one pin above.
GATE_MUTANTS = {
    "alpha_from_sin": ("alpha = np.cos(theta) ** 2", "alpha = np.sin(theta) ** 2"),
    "eta_as_two_sigmoid": ("eta = np.tanh(x) + 1.0", "eta = 2.0 / (1.0 + np.exp(-x))"),
    "s_divides": ("theta = np.arctan(eta * s)", "theta = np.arctan(eta / s)"),
    "beta_from_a": ("beta = np.sin(theta) ** 2 / (1.0 + np.exp(-b))",
                    "beta = np.sin(theta) ** 2 / (1.0 + np.exp(-a))"),
    "mu_clamp_open_above": ("mu = np.exp(np.clip(mu_log, mu_log_min, 0.0))",
                            "mu = np.exp(np.maximum(mu_log, mu_log_min))"),
    "mu_clamp_one_lower": ("mu = np.exp(np.clip(mu_log, mu_log_min, 0.0))",
                           "mu = np.exp(np.clip(mu_log, mu_log_min - 1.0, 0.0))"),
}
QC_MUTANTS = {
    "correction_added": ("return q - d[None, :, None, None] * k", "return q + d[None, :, None, None] * k"),
    "d_per_batch": ("return q - d[None, :, None, None] * k", "return q - d.mean() * k"),
}


def _mutant(fn, old, new):
    src = textwrap.dedent(inspect.getsource(fn))
    assert src.count(old) == 1, old
    ns = dict(vars(gates_ref))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    return ns[fn.__name__]


def _caught(checks, fn):
    failed = 0
    for check in checks:
        try:
            check(fn)
        except AssertionError:
            failed += 1
    return failed


@pytest.mark.parametrize("name", sorted(GATE_MUTANTS))
def test_gate_mutant_is_caught(name):
    assert _caught(GATE_CHECKS, _mutant(gates_ref.gates, *GATE_MUTANTS[name])) > 0, name


@pytest.mark.parametrize("name", sorted(QC_MUTANTS))
def test_query_correction_mutant_is_caught(name):
    assert _caught((check_query_correction,), _mutant(gates_ref.query_correction, *QC_MUTANTS[name])) > 0, name
