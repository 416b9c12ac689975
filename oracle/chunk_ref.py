"""NumPy fp64 restatement of MDN's chunkwise algorithm (oracle side).

TEST INFRASTRUCTURE ONLY (see the ``oracle`` package docstring).

The recurrence oracle (``oracle.fwd``) is the definition of the outputs.  This
module restates the chunkwise algorithm of the MDN summary at
paper.rainbus.top (method walk-through, steps 2-5) in the pages' own notation,
so that

* the chunk equations can be checked against the recurrence (chunk-size
  invariance, C = 1 reducing to the token form), and
* the per-chunk intermediates the GPU path produces (the coefficient vectors,
  Gamma, T) have a definition of their own to be compared with.

Indexing: a chunk holds tokens r = 1..C (arrays are 0-based, so array row r-1
is token r).  All cumulative quantities restart at every chunk; S and M below
are the states at the start of the chunk.

Readings of the pages used here:

* eta_i multiplies every rank-1 term of the expansion in step 2; the printed
  expansion omits it, and without it the expansion does not reproduce the
  recurrence of step 1.
* Gamma_{r,i} = eta_i * gamma_{r,i} for i <= r, and the strictly lower
  "Gamma^-" of step 4 is Gamma shifted down one row: Gamma^-_{r,i} =
  Gamma_{r-1,i} for i < r.
* "alpha_bar_{0->C-1}" and "b_{0->C-1}" in Y and Z (step 4) are the exclusive
  prefixes alpha_bar_{r-1}, b_{r-1}, with alpha_bar_0 = 1 and b_0 = 0.
* The chunk output and end-of-chunk state update, which the pages do not
  print, are the closed form of step 2 evaluated at r (output, o_r = S_r^T q_r)
  and at r = C (state).
"""
from __future__ import annotations

import numpy as np


def _decay_matrix(g):
    """L[r, j] = prod_{s=j+1..r} g_s for j <= r (1 on the diagonal), else 0.

    Built row by row from the plain product definition (L[r, :r] = L[r-1, :r]
    times g_r); no division, so zeros in g are exact.
    """
    C = g.shape[0]
    L = np.zeros((C, C))
    for r in range(C):
        if r > 0:
            L[r, :r] = L[r - 1, :r] * g[r]
        L[r, r] = 1.0
    return L


def coefficients(alpha, mu, beta, eta):
    """Per-chunk coefficients from direct products (MDN summary, step 2).

    Definitions (tokens 1..C of one chunk):
      abar_r  = prod_{s<=r} alpha_s            mubar_r = prod_{s<=r} mu_s
      b_r     = sum_{j<=r} beta_j (abar_r/abar_j) mubar_j
      gamma_{r,i} = sum_{j=i..r} beta_j (abar_r/abar_j)(mubar_j/mubar_i)
      Gamma_{r,i} = eta_i gamma_{r,i}  (i <= r)
      gS_i = Gamma_{C,i},  gM_i = eta_i mubar_C / mubar_i
    Every ratio above is a product over a contiguous range of gates, so it is
    formed as such (``_decay_matrix``) and stays exact for zero gates.
    The closed forms on the page (b_t = abar_t c_t and
    gamma_{t,i} = (abar_t/mubar_i)(c_t - c_{i-1})) are the same numbers; the
    pins compare the two.
    """
    alpha, mu, beta, eta = (np.asarray(x, dtype=np.float64) for x in (alpha, mu, beta, eta))
    La = _decay_matrix(alpha)          # abar_r / abar_j
    Lm = _decay_matrix(mu)             # mubar_j / mubar_i
    abar = np.cumprod(alpha)
    mubar = np.cumprod(mu)
    gamma = La @ np.diag(beta) @ Lm    # sum over i <= j <= r; zero above the diagonal
    b = La @ (beta * mubar)
    Gamma = gamma * eta[None, :]
    gS = Gamma[-1, :].copy()
    gM = eta * Lm[-1, :]
    return dict(abar=abar, mubar=mubar, b=b, gamma=gamma, Gamma=Gamma, gS=gS, gM=gM)


def coefficients_logdomain(alpha, mu, beta, eta):
    """The page's log-domain route to abar, mubar, c and b (summary, step 5).

    Lambda_a = cumsum(log alpha), Lambda_m = cumsum(log mu),
    log c = logcumsumexp(log beta + Lambda_m - Lambda_a), b = exp(Lambda_a + log c),
    and gamma_{t,i} = (abar_t / mubar_i)(c_t - c_{i-1}) as printed in step 2.
    Valid for gates in (0, 1]; the difference c_t - c_{i-1} loses precision
    when mu << alpha, so it is only compared on gates where it is benign.
    """
    alpha, mu, beta, eta = (np.asarray(x, dtype=np.float64) for x in (alpha, mu, beta, eta))
    La = np.cumsum(np.log(alpha))
    Lm = np.cumsum(np.log(mu))
    x = np.log(beta) + Lm - La
    logc = np.logaddexp.accumulate(x)
    b = np.exp(La + logc)
    c = np.exp(logc)
    c_prev = np.concatenate([[0.0], c[:-1]])
    C = alpha.shape[0]
    gamma = np.zeros((C, C))
    for t in range(C):
        for i in range(t + 1):
            gamma[t, i] = np.exp(La[t] - Lm[i]) * (c[t] - c_prev[i])
    return dict(abar=np.exp(La), mubar=np.exp(Lm), logc=logc, b=b, gamma=gamma,
                Gamma=gamma * eta[None, :])


def chunk_matrices(k, alpha, mu, beta, eta, q=None):
    """T, A and (if q is given) the masked score matrix of one chunk.

    MDN summary, steps 3-4: P = Diag(alpha) K, A = (P K^T) o Gamma^-,
    T = Tril(I + A)^{-1}; the intra-chunk read-out uses (Q K^T) o Gamma.
    Returns dict(T, A, Aqk, coef).
    """
    k = np.asarray(k, dtype=np.float64)
    coef = coefficients(alpha, mu, beta, eta)
    C = k.shape[0]
    Gamma = coef["Gamma"]
    Gm = np.zeros((C, C))
    Gm[1:, :] = Gamma[:-1, :]
    Gm = np.tril(Gm, -1)
    P = np.asarray(alpha, dtype=np.float64)[:, None] * k
    A = (P @ k.T) * Gm
    T = np.linalg.solve(np.eye(C) + A, np.eye(C))
    T = np.tril(T)
    out = dict(T=T, A=A, coef=coef)
    if q is not None:
        out["Aqk"] = (np.asarray(q, dtype=np.float64) @ k.T) * np.tril(Gamma)
    return out


def chunk_fwd_head(q, k, v, alpha, mu, beta, eta, S0, M0, C):
    """Chunkwise forward of one head (summary, steps 2-4), fp64.

    q, k: [T, dk]; v: [T, dv]; gates: [T]; S0, M0: [dk, dv].
    Returns (O, S_T, M_T, Vtilde).  The last chunk may be shorter than C.
    """
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    alpha, mu, beta, eta = (np.asarray(x, dtype=np.float64) for x in (alpha, mu, beta, eta))
    T_len, dk = k.shape
    dv = v.shape[1]
    S = np.array(S0, dtype=np.float64).reshape(dk, dv)
    M = np.array(M0, dtype=np.float64).reshape(dk, dv)
    O = np.zeros((T_len, dv))
    Vt = np.zeros((T_len, dv))
    for s in range(0, T_len, C):
        e = min(s + C, T_len)
        sl = slice(s, e)
        Kc, Qc, Vc = k[sl], q[sl], v[sl]
        a, m, bt, et = alpha[sl], mu[sl], beta[sl], eta[sl]
        mats = chunk_matrices(Kc, a, m, bt, et, q=Qc)
        coef, Tm = mats["coef"], mats["T"]
        abar, b = coef["abar"], coef["b"]
        abar_prev = np.concatenate([[1.0], abar[:-1]])
        b_prev = np.concatenate([[0.0], b[:-1]])
        P = a[:, None] * Kc
        U = Tm @ Vc
        Y = Tm @ (abar_prev[:, None] * P)
        Z = Tm @ (b_prev[:, None] * P)
        Vtil = U - Y @ S + Z @ M
        Oc = abar[:, None] * (Qc @ S) - b[:, None] * (Qc @ M) + mats["Aqk"] @ Vtil
        S_new = abar[-1] * S - b[-1] * M + Kc.T @ (coef["gS"][:, None] * Vtil)
        M_new = coef["mubar"][-1] * M - Kc.T @ (coef["gM"][:, None] * Vtil)
        O[sl] = Oc
        Vt[sl] = Vtil
        S, M = S_new, M_new
    return O, S, M, Vt


def chunk_fwd(q, k, v, alpha, mu, beta, eta, S0=None, M0=None, C=64):
    """Batched wrapper of :func:`chunk_fwd_head` over leading dims."""
    q = np.asarray(q, dtype=np.float64)
    lead = q.shape[:-2]
    T_len, dk = q.shape[-2:]
    dv = np.shape(v)[-1]
    n = int(np.prod(lead)) if lead else 1
    qf = q.reshape(n, T_len, dk)
    kf = np.asarray(k, dtype=np.float64).reshape(n, T_len, dk)
    vf = np.asarray(v, dtype=np.float64).reshape(n, T_len, dv)
    gates = [np.asarray(g, dtype=np.float64).reshape(n, T_len) for g in (alpha, mu, beta, eta)]
    S0f = np.zeros((n, dk, dv)) if S0 is None else np.broadcast_to(S0, lead + (dk, dv)).reshape(n, dk, dv)
    M0f = np.zeros((n, dk, dv)) if M0 is None else np.broadcast_to(M0, lead + (dk, dv)).reshape(n, dk, dv)
    outs = [chunk_fwd_head(qf[h], kf[h], vf[h], *(g[h] for g in gates), S0f[h], M0f[h], C)
            for h in range(n)]
    O = np.stack([o[0] for o in outs]).reshape(lead + (T_len, dv))
    ST = np.stack([o[1] for o in outs]).reshape(lead + (dk, dv))
    MT = np.stack([o[2] for o in outs]).reshape(lead + (dk, dv))
    Vt = np.stack([o[3] for o in outs]).reshape(lead + (T_len, dv))
    return O, ST, MT, Vt
