"""Checks that pin the fp64 oracle to the pages and to mathematics.

Each check takes a ``fwd`` callable with the signature of ``oracle.fwd`` so the
same checks can run against deliberately broken copies of the oracle
(``test_oracle_mutants.py``).  Each returns the worst error it saw; the caller
asserts on it.  None of them re-states the recurrence: they compare the
oracle's outputs with closed forms, reductions, an autodiff gradient or
eigen-structure that the pages give.

Sources (pages about "MDN: Parallelizing Stepwise Momentum for Delta Linear
Attention"):
  [S] paper summary at paper.rainbus.top: method walk-through steps 1-6 and
      the novelty paragraph (second point: block state space, spectrum,
      stability interval).
  [A] ijyty.com article on MDN: section 3 (the two update equations),
      section 6 (recurrent generation), section 8 (mu = 0 ablation: GDN).
"""
from __future__ import annotations

import numpy as np


def rng_problem(seed, T=10, dk=3, dv=2, states=True, mu_range=(-1.0, 0.0)):
    rng = np.random.default_rng(1000 + seed)
    q = rng.standard_normal((T, dk))
    k = rng.standard_normal((T, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, dv))
    eta = np.tanh(rng.standard_normal(T)) + 1.0
    th = np.arctan(eta)
    alpha = np.cos(th) ** 2 / (1 + np.exp(-rng.standard_normal(T)))
    beta = np.sin(th) ** 2 / (1 + np.exp(-rng.standard_normal(T)))
    mu = np.exp(rng.uniform(mu_range[0], mu_range[1], T))
    S0 = rng.standard_normal((dk, dv)) if states else np.zeros((dk, dv))
    M0 = rng.standard_normal((dk, dv)) if states else np.zeros((dk, dv))
    return dict(q=q, k=k, v=v, alpha=alpha, mu=mu, beta=beta, eta=eta, S0=S0, M0=M0)


def prefix_states(fwd, p):
    """S_t, M_t for t = 0..T from runs on each prefix (S_0 = S0)."""
    T = p["q"].shape[0]
    Ss, Ms = [p["S0"]], [p["M0"]]
    for t in range(1, T + 1):
        _, S, M, _ = fwd(p["q"][:t], p["k"][:t], p["v"][:t], p["alpha"][:t], p["mu"][:t],
                         p["beta"][:t], p["eta"][:t], p["S0"], p["M0"])
        Ss.append(S)
        Ms.append(M)
    return Ss, Ms


def check_closed_form(fwd, seed=0, use_eta=True):
    """[S] step 2: M_t and S_t against the printed expansion, with eta_i on
    each rank-1 term (reading: the printed expansion omits it).

    c_t = sum_{i<=t} beta_i mubar_i / abar_i, b_t = abar_t c_t,
    gamma_{t,i} = (abar_t / mubar_i)(c_t - c_{i-1}).
    """
    p = rng_problem(seed)
    O, ST, MT, Vt = fwd(p["q"], p["k"], p["v"], p["alpha"], p["mu"], p["beta"], p["eta"],
                        p["S0"], p["M0"])
    Ss, Ms = prefix_states(fwd, p)
    T = p["q"].shape[0]
    abar = np.cumprod(p["alpha"])
    mubar = np.cumprod(p["mu"])
    c = np.cumsum(p["beta"] * mubar / abar)
    cp = np.concatenate([[0.0], c])       # cp[i] = c_{i} with c_0 = 0 (1-based)
    e = p["eta"] if use_eta else np.ones(T)
    worst = 0.0
    for t in range(1, T + 1):
        Mcf = mubar[t - 1] * p["M0"]
        Scf = abar[t - 1] * p["S0"] - abar[t - 1] * c[t - 1] * p["M0"]
        for i in range(1, t + 1):
            outer = np.outer(p["k"][i - 1], Vt[i - 1])
            Mcf = Mcf - (mubar[t - 1] / mubar[i - 1]) * e[i - 1] * outer
            gam = (abar[t - 1] / mubar[i - 1]) * (c[t - 1] - cp[i - 1])
            Scf = Scf + gam * e[i - 1] * outer
        scale = max(1.0, np.abs(Ss[t]).max(), np.abs(Ms[t]).max())
        worst = max(worst, np.abs(Scf - Ss[t]).max() / scale, np.abs(Mcf - Ms[t]).max() / scale)
        # read-out after the update of token t
        worst = max(worst, np.abs(O[t - 1] - Ss[t].T @ p["q"][t - 1]).max() / scale)
    return worst


def check_latent_gradient(fwd, seed=1):
    """[S] step 1: M_t - mu_t M_{t-1} = eta_t * grad of the latent loss
    L(St) = 1/2 ||v_t - St^T k_t||^2 taken at St = alpha_t S_{t-1}
    (gradient by torch autograd in fp64, not by formula)."""
    import torch

    p = rng_problem(seed)
    Ss, Ms = prefix_states(fwd, p)
    T = p["q"].shape[0]
    worst = 0.0
    for t in range(1, T + 1):
        St = torch.tensor(p["alpha"][t - 1] * Ss[t - 1], dtype=torch.float64, requires_grad=True)
        kt = torch.tensor(p["k"][t - 1], dtype=torch.float64)
        vt = torch.tensor(p["v"][t - 1], dtype=torch.float64)
        L = 0.5 * torch.sum((vt - St.T @ kt) ** 2)
        (g,) = torch.autograd.grad(L, St)
        lhs = Ms[t] - p["mu"][t - 1] * Ms[t - 1]
        rhs = p["eta"][t - 1] * g.numpy()
        worst = max(worst, np.abs(lhs - rhs).max() / max(1.0, np.abs(rhs).max()))
    return worst


def check_beta_zero(fwd, seed=2):
    """beta = 0: S_t = abar_t S_0 and o_t = abar_t S_0^T q_t; the momentum then
    integrates the errors against the decayed initial state:
    M_t = mubar_t M_0 - sum_i (mubar_t/mubar_i) eta_i k_i (v_i - abar_i S_0^T k_i)^T."""
    p = rng_problem(seed)
    p["beta"] = np.zeros_like(p["beta"])
    O, ST, MT, Vt = fwd(p["q"], p["k"], p["v"], p["alpha"], p["mu"], p["beta"], p["eta"],
                        p["S0"], p["M0"])
    T = p["q"].shape[0]
    abar = np.cumprod(p["alpha"])
    mubar = np.cumprod(p["mu"])
    worst = np.abs(ST - abar[-1] * p["S0"]).max()
    for t in range(T):
        worst = max(worst, np.abs(O[t] - abar[t] * (p["S0"].T @ p["q"][t])).max())
    Mcf = mubar[-1] * p["M0"]
    for i in range(T):
        err_i = p["v"][i] - abar[i] * (p["S0"].T @ p["k"][i])
        Mcf = Mcf - (mubar[-1] / mubar[i]) * p["eta"][i] * np.outer(p["k"][i], err_i)
    worst = max(worst, np.abs(Mcf - MT).max())
    return worst


def gated_delta_rule(q, k, v, alpha, beta_hat, S0):
    """Gated delta rule (GDN): S_t = alpha_t (I - beta_t k k^T) S_{t-1} + beta_t k v^T,
    o_t = S_t^T q_t."""
    S = S0.copy()
    dk = S.shape[0]
    O = []
    for t in range(q.shape[0]):
        kk = k[t]
        S = alpha[t] * (np.eye(dk) - beta_hat[t] * np.outer(kk, kk)) @ S + beta_hat[t] * np.outer(kk, v[t])
        O.append(S.T @ q[t])
    return np.array(O), S


def check_mu_zero_gdn(fwd, seed=3):
    """[A] section 8: with mu = 0 MDN degenerates to GDN.  The momentum then
    holds only the current error, and the fast weight follows the gated delta
    rule with step size beta_t * eta_t (M_0 = 0)."""
    p = rng_problem(seed)
    p["mu"] = np.zeros_like(p["mu"])
    O, ST, MT, Vt = fwd(p["q"], p["k"], p["v"], p["alpha"], p["mu"], p["beta"], p["eta"],
                        p["S0"], np.zeros_like(p["M0"]))
    Og, Sg = gated_delta_rule(p["q"], p["k"], p["v"], p["alpha"], p["beta"] * p["eta"], p["S0"])
    return max(np.abs(O - Og).max(), np.abs(ST - Sg).max())


def eigen_pair(alpha, mu, beta, eta, knorm2):
    """[S] step 6: lambda_pm printed for the momentum system."""
    tr = alpha + mu - alpha * beta * eta * knorm2
    disc = complex(tr * tr - 4 * alpha * mu)
    r = np.sqrt(disc)
    return (tr + r) / 2, (tr - r) / 2


def check_second_order_scalar(fwd, alpha=0.6, mu=0.7, beta=0.35, eta=1.5, T=40):
    """[S] step 6 and novelty point 2: with dk = dv = 1, constant gates,
    |k| = 1 and v = 0, [S_t; M_t] is a 2-dim linear system whose eigenvalues
    are lambda_pm, so S_t obeys S_{t+2} = (l+ + l-) S_{t+1} - l+ l- S_t."""
    q = np.ones((T, 1))
    k = np.ones((T, 1))
    v = np.zeros((T, 1))
    g = lambda x: np.full(T, x)
    S0 = np.array([[1.0]])
    M0 = np.array([[-0.5]])
    O, _, _, _ = fwd(q, k, v, g(alpha), g(mu), g(beta), g(eta), S0, M0)
    s = np.concatenate([[S0[0, 0]], O[:, 0]])   # o_t = S_t (q = 1)
    lp, lm = eigen_pair(alpha, mu, beta, eta, 1.0)
    tr, det = (lp + lm).real, (lp * lm).real
    res = s[2:] - tr * s[1:-1] + det * s[:-2]
    return np.abs(res).max() / np.abs(s).max()


def check_second_order_block(fwd, alpha=0.55, mu=0.8, beta=0.3, eta=1.2, T=30):
    """[S] novelty point 2: the block system has spectrum {alpha, mu, l+, l-}.
    With dk = 2 and k = e_1, the e_2 row never meets a key, so (S, M) on that
    row evolve with eigenvalues {alpha, mu}: M decays as mu^t and S obeys
    S_{t+2} = (alpha + mu) S_{t+1} - alpha mu S_t."""
    q = np.tile([0.0, 1.0], (T, 1))
    k = np.tile([1.0, 0.0], (T, 1))
    v = np.zeros((T, 1))
    g = lambda x: np.full(T, x)
    S0 = np.array([[0.7], [1.0]])
    M0 = np.array([[0.2], [-0.4]])
    O, ST, MT, _ = fwd(q, k, v, g(alpha), g(mu), g(beta), g(eta), S0, M0)
    s = np.concatenate([[S0[1, 0]], O[:, 0]])   # q = e_2 reads row 2
    res = s[2:] - (alpha + mu) * s[1:-1] + alpha * mu * s[:-2]
    err = np.abs(res).max() / np.abs(s).max()
    err = max(err, abs(MT[1, 0] - mu ** T * M0[1, 0]) / abs(M0[1, 0]))
    return err


def check_step_matches_fwd(fwd, step, seed=4):
    """[A] section 6: generation runs the recurrence one token at a time and
    matches the training-time forward."""
    p = rng_problem(seed, T=7)
    O, ST, MT, Vt = fwd(p["q"], p["k"], p["v"], p["alpha"], p["mu"], p["beta"], p["eta"],
                        p["S0"], p["M0"])
    S, M = p["S0"], p["M0"]
    worst = 0.0
    for t in range(7):
        o, S, M, vt = step(p["q"][t], p["k"][t], p["v"][t], p["alpha"][t], p["mu"][t],
                           p["beta"][t], p["eta"][t], S, M)
        worst = max(worst, np.abs(o - O[t]).max(), np.abs(vt - Vt[t]).max())
    return max(worst, np.abs(S - ST).max(), np.abs(M - MT).max())
