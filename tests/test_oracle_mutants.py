"""Planted mistakes in the oracle (on the CPU) must fail at least one pin.

Each mutant is a one-line change to a copy of ``oracle/mdn_oracle.c`` that a
plausible slip would produce: a flipped sign, the wrong state in the error
term, the old momentum in the fast-weight update, a dropped eta, a dropped
alpha in p_t, the read-out before the update, a transposed read.  The copy is
compiled into a temporary library; the real oracle is untouched.
"""
import ctypes
import os
import subprocess
import tempfile

import numpy as np
import pytest

from tests import pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "mdn_oracle.c")

MUTANTS = {
    "flip_momentum_sign": ("mu * M[i * dv + j] - eta * k[i] * vtilde[j]",
                           "mu * M[i * dv + j] + eta * k[i] * vtilde[j]"),
    "drop_eta": ("mu * M[i * dv + j] - eta * k[i] * vtilde[j]",
                 "mu * M[i * dv + j] - k[i] * vtilde[j]"),
    "old_momentum_in_S": ("S[i * dv + j] = alpha * S[i * dv + j] - beta * m;",
                          "S[i * dv + j] = alpha * S[i * dv + j] - beta * M[i * dv + j] * 0.0 - beta * (m + eta * k[i] * vtilde[j]);"),
    "drop_alpha_in_p": ("acc += S[i * dv + j] * (alpha * k[i]);",
                        "acc += S[i * dv + j] * k[i];"),
    "plus_beta": ("alpha * S[i * dv + j] - beta * m",
                  "alpha * S[i * dv + j] + beta * m"),
    "transposed_read": ("for (long i = 0; i < dk; ++i) acc += S[i * dv + j] * q[i];",
                        "for (long i = 0; i < dk; ++i) acc += S[j * dv + i] * q[i];"),
    "mu_on_update": ("double m = mu * M[i * dv + j] - eta * k[i] * vtilde[j];",
                     "double m = mu * (M[i * dv + j] - eta * k[i] * vtilde[j]);"),
}


def _build_mutant(name, old, new, tmpdir):
    src = open(SRC).read()
    assert src.count(old) == 1, name
    path_c = os.path.join(tmpdir, name + ".c")
    path_so = os.path.join(tmpdir, name + ".so")
    with open(path_c, "w") as f:
        f.write(src.replace(old, new))
    subprocess.check_call(["gcc", "-O1", "-fPIC", "-shared", "-std=c99", "-o", path_so, path_c])
    lib = ctypes.CDLL(path_so)
    d = ctypes.POINTER(ctypes.c_double)
    L = ctypes.c_long
    lib.mdn_oracle_fwd.argtypes = [L, L, L, L] + [d] * 7 + [ctypes.c_void_p, ctypes.c_void_p] + [d] * 4
    lib.mdn_oracle_step.argtypes = [L, L, L] + [d] * 7 + [d] * 4
    return lib


def _fwd_from(lib):
    P = lambda a: a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))

    def fwd(q, k, v, alpha, mu, beta, eta, S0=None, M0=None):
        f = lambda x: np.ascontiguousarray(np.asarray(x, dtype=np.float64))
        q, k, v, alpha, mu, beta, eta = map(f, (q, k, v, alpha, mu, beta, eta))
        T, dk = q.shape
        dv = v.shape[1]
        O, Vt = np.zeros((T, dv)), np.zeros((T, dv))
        ST, MT = np.zeros((dk, dv)), np.zeros((dk, dv))
        S0 = f(S0) if S0 is not None else np.zeros((dk, dv))
        M0 = f(M0) if M0 is not None else np.zeros((dk, dv))
        lib.mdn_oracle_fwd(1, T, dk, dv, P(q), P(k), P(v), P(alpha), P(mu), P(beta), P(eta),
                           S0.ctypes.data, M0.ctypes.data, P(O), P(ST), P(MT), P(Vt))
        return O, ST, MT, Vt
    return fwd


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    with tempfile.TemporaryDirectory() as tmp:
        fwd = _fwd_from(_build_mutant(name, old, new, tmp))
        errs = {
            "closed_form": pins.check_closed_form(fwd),
            "latent_gradient": pins.check_latent_gradient(fwd),
            "beta_zero": pins.check_beta_zero(fwd),
            "mu_zero_gdn": pins.check_mu_zero_gdn(fwd),
            "second_order": pins.check_second_order_scalar(fwd),
            "block_spectrum": pins.check_second_order_block(fwd),
        }
    caught = [k for k, e in errs.items() if not (e < 1e-9)]
    assert caught, f"mutant {name} passed every pin: {errs}"
