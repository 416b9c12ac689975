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


def chunk_bwd_head(q, k, v, alpha, mu, beta, eta, S0, M0, dO, dST, dMT, C):
    """Chunkwise reverse mode of one head, fp64 (the gradients of
    L = sum(dO*O) + sum(dST*S_T) + sum(dMT*M_T), like ``oracle.bwd``).

    The pages give no backward; this is the chain rule applied to the chunk
    equations of :func:`chunk_fwd_head` in the form
    W = V - Diag(abar) K S + Diag(alpha b_prev) K M, Vtilde = T W (the same
    numbers as U - Y S + Z M).  Three parts:

    1. chunk-start states S[n], M[n] replayed forward from Vtilde (only the
       state update, no T);
    2. a reverse pass that carries dS, dM (adjoints of the chunk-end states)
       to the chunk start:
         dVt = Aqk^T dO + Diag(gS) K dS' - Diag(gM) K dM',   dW = T^T dVt,
         dS  = abar_L dS' + Q^T Diag(abar) dO - K^T Diag(abar) dW,
         dM  = mubar_L dM' - b_L dS' - Q^T Diag(b) dO + K^T Diag(alpha b_prev) dW;
    3. per chunk, the gradients of Q, K, V and of the coefficients, then of
       the gates through the coefficient definitions.  With
       E[r,j] = abar_r/abar_j, F[j,i] = mubar_j/mubar_i, Psi = E Diag(beta) F
       (so Gamma = Psi Diag(eta)) and b = E (beta mubar), the adjoints of
       Gamma and b give
         dbeta_j = Z_j = sum_{r>=j, i<=j} E[r,j] DPsi[r,i] F[j,i] + sum_{r>=j} E[r,j] Db_r mubar_j,
         d Lambda_alpha_m += rowsum(DPsi o Psi)_m + Db_m b_m - beta_m Z_m,
         d Lambda_mu_m    += beta_m Z_m - colsum(DPsi o Psi)_m,
       and dalpha_s = sum_{r>=s} d Lambda_alpha_r / alpha_s (likewise mu),
       where Lambda are the inclusive cumulative logs of the chunk.
    Gates must be positive (the logs).  The last chunk may be shorter than C.
    Returns the same dict as ``oracle.bwd``.
    """
    q, k, v, dO = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dO))
    alpha, mu, beta, eta = (np.asarray(x, dtype=np.float64) for x in (alpha, mu, beta, eta))
    T_len, dk = k.shape
    dv = v.shape[1]
    starts = list(range(0, T_len, C))
    # 1. forward replay of the chunk-start states, keeping each chunk's matrices
    S = np.array(S0, dtype=np.float64).reshape(dk, dv)
    M = np.array(M0, dtype=np.float64).reshape(dk, dv)
    saved = []
    for s in starts:
        sl = slice(s, min(s + C, T_len))
        Kc, Qc, Vc = k[sl], q[sl], v[sl]
        a, m, bt, et = alpha[sl], mu[sl], beta[sl], eta[sl]
        n = a.shape[0]
        la, lm = np.cumsum(np.log(a)), np.cumsum(np.log(m))
        E = np.tril(np.exp(np.minimum(la[:, None] - la[None, :], 0.0)))
        F = np.tril(np.exp(np.minimum(lm[:, None] - lm[None, :], 0.0)))
        abar, mubar = np.exp(la), np.exp(lm)
        Psi = E @ np.diag(bt) @ F
        Gam = Psi * et[None, :]
        b = E @ (bt * mubar)
        bprev = np.concatenate([[0.0], b[:-1]])
        ab = a * bprev
        Gm = np.zeros((n, n))
        Gm[1:, :] = Gam[:-1, :]
        Gm = np.tril(Gm, -1)
        P = a[:, None] * Kc
        PK = P @ Kc.T
        A = PK * Gm
        Tm = np.linalg.inv(np.eye(n) + A)
        QK = Qc @ Kc.T
        Aqk = QK * Gam
        W = Vc - abar[:, None] * (Kc @ S) + ab[:, None] * (Kc @ M)
        Vt = Tm @ W
        gS, gM = Gam[-1, :].copy(), et * F[-1, :]
        saved.append(dict(sl=sl, S=S, M=M, E=E, F=F, abar=abar, mubar=mubar, Psi=Psi, Gam=Gam, b=b,
                          bprev=bprev, ab=ab, Gm=Gm, P=P, PK=PK, Tm=Tm, QK=QK, Aqk=Aqk, Vt=Vt, gS=gS, gM=gM))
        S = abar[-1] * S - b[-1] * M + Kc.T @ (gS[:, None] * Vt)
        M = mubar[-1] * M - Kc.T @ (gM[:, None] * Vt)
    out = dict(dq=np.zeros((T_len, dk)), dk=np.zeros((T_len, dk)), dv=np.zeros((T_len, dv)),
               dalpha=np.zeros(T_len), dmu=np.zeros(T_len), dbeta=np.zeros(T_len), deta=np.zeros(T_len))
    dS = np.zeros((dk, dv)) if dST is None else np.array(dST, dtype=np.float64).reshape(dk, dv)
    dM = np.zeros((dk, dv)) if dMT is None else np.array(dMT, dtype=np.float64).reshape(dk, dv)
    # 2 + 3. reverse over chunks
    for c in reversed(saved):
        sl = c["sl"]
        Kc, Qc = k[sl], q[sl]
        a, m, bt, et = alpha[sl], mu[sl], beta[sl], eta[sl]
        dOc = dO[sl]
        S, M, Vt = c["S"], c["M"], c["Vt"]
        dVt = c["Aqk"].T @ dOc + c["gS"][:, None] * (Kc @ dS) - c["gM"][:, None] * (Kc @ dM)
        dW = c["Tm"].T @ dVt
        dAqk = np.tril(dOc @ Vt.T)
        dA = -np.tril(dW @ Vt.T, -1)
        dOS, dOM, dWS, dWM = dOc @ S.T, dOc @ M.T, dW @ S.T, dW @ M.T
        # Q, K, V
        X1 = dAqk * c["Gam"]
        X2 = dA * c["Gm"]
        dP = X2 @ Kc
        out["dq"][sl] = c["abar"][:, None] * dOS - c["b"][:, None] * dOM + X1 @ Kc
        out["dk"][sl] = (X1.T @ Qc + X2.T @ c["P"] + a[:, None] * dP - c["abar"][:, None] * dWS
                         + c["ab"][:, None] * dWM + c["gS"][:, None] * (Vt @ dS.T) - c["gM"][:, None] * (Vt @ dM.T))
        out["dv"][sl] = dW
        # coefficient adjoints
        L = a.shape[0] - 1
        Dabar = (Qc * dOS).sum(1) - (Kc * dWS).sum(1)
        Dabar[L] += (S * dS).sum()
        Dab = (Kc * dWM).sum(1)
        Db = -(Qc * dOM).sum(1)
        Db[L] -= (M * dS).sum()
        Db[:-1] += Dab[1:] * a[1:]
        dalpha_direct = (Kc * dP).sum(1) + Dab * c["bprev"]
        DGam = dAqk * c["QK"]
        DGam[:-1, :] += np.tril(dA * c["PK"], -1)[1:, :]
        DgS = ((Vt @ dS.T) * Kc).sum(1)
        DgM = -((Vt @ dM.T) * Kc).sum(1)
        DGam[L, :] += DgS
        Dmubar_L = (M * dM).sum()
        # gates through the coefficient definitions
        E, F, Psi, b, mubar, abar = c["E"], c["F"], c["Psi"], c["b"], c["mubar"], c["abar"]
        DPsi = np.tril(DGam) * et[None, :]
        deta = (np.tril(DGam) * Psi).sum(0) + DgM * F[L, :]
        Z = ((E.T @ DPsi) * F).sum(1) + (E.T @ Db) * mubar
        dla = (DPsi * Psi).sum(1) + Db * b - bt * Z + Dabar * abar
        dlm = bt * Z - (DPsi * Psi).sum(0) - DgM * c["gM"]
        dlm[L] += (DgM * c["gM"]).sum() + Dmubar_L * mubar[L]
        rev = lambda x: np.cumsum(x[::-1])[::-1]
        out["dalpha"][sl] = rev(dla) / a + dalpha_direct
        out["dmu"][sl] = rev(dlm) / m
        out["dbeta"][sl] = Z
        out["deta"][sl] = deta
        # chunk-start adjoints
        dS, dM = (abar[L] * dS + Qc.T @ (abar[:, None] * dOc) - Kc.T @ (abar[:, None] * dW),
                  mubar[L] * dM - b[L] * dS + (-Qc.T @ (b[:, None] * dOc)) + Kc.T @ (c["ab"][:, None] * dW))
    out["dS0"], out["dM0"] = dS, dM
    return out
