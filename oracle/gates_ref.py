"""NumPy fp64 gate pre-operation and query correction (oracle side).

TEST INFRASTRUCTURE ONLY (see the ``oracle`` package docstring).

The elementwise step between a layer's projections and the recurrence, in the
order the pages give it:

* stable gating (MDN summary at paper.rainbus.top, method walk-through step 6;
  ijyty.com article on MDN, section 5): an angle theta = arctan(eta * s)
  bounds the two gates, alpha_max = cos^2(theta) and beta_max = sin^2(theta),
  and log mu is clamped from below (at -2 on the pages);
* the eta activation tanh(.) + 1 (article, section 8, where replacing it by
  2 sigmoid(.) is the ablation);
* the query correction q - d k taken from Comba (summary, step 7; article,
  section 8).

Readings (the pages name the bounds but not how a projection output reaches
a gate): alpha = alpha_max * sigmoid(a) and beta = beta_max * sigmoid(b), the
plain reading of "maximum" with a sigmoid gate, which is also the recipe of
the synthetic workloads; mu = exp(clamp(mu_log, mu_log_min, 0)); d is one
scalar per head.
"""
from __future__ import annotations

import numpy as np


def gates(x, a, b, mu_log, s=1.0, mu_log_min=-2.0):
    """(alpha, mu, beta, eta) from the projection outputs, fp64 (summary,
    step 6; article, sections 5 and 8)."""
    x, a, b, mu_log = (np.asarray(t, dtype=np.float64) for t in (x, a, b, mu_log))
    eta = np.tanh(x) + 1.0
    theta = np.arctan(eta * s)
    alpha = np.cos(theta) ** 2 / (1.0 + np.exp(-a))
    beta = np.sin(theta) ** 2 / (1.0 + np.exp(-b))
    mu = np.exp(np.clip(mu_log, mu_log_min, 0.0))
    return alpha, mu, beta, eta


def query_correction(q, k, d):
    """q - d_h k for q, k of shape [B, H, T, dk] and d of shape [H], fp64
    (summary, step 7)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    d = np.asarray(d, dtype=np.float64)
    return q - d[None, :, None, None] * k
