"""fp64 CPU oracle for the Momentum DeltaNet (MDN) hot path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``linear_attention_sequence_mdn_amd``) never imports it, and the two share no
code: the only module both sides use is the seeded input generator, which holds
none of the method's arithmetic.

Contents
--------
* ``fwd`` / ``step``: the token-by-token recurrence, in C (``mdn_oracle.c``),
  fp64, OpenMP over heads.  ``fwd_varlen`` runs ``fwd`` per sequence of a
  packed batch.  ``bwd``: reverse mode of the same recurrence (C), the
  gradients of every input for given output gradients.  This is the plain definition of what the chunkwise
  forward and the decode step compute (MDN paper summary at paper.rainbus.top,
  method walk-through step 1; ijyty.com article on MDN, sections 3 and 6).
* ``chunk_ref``: a NumPy fp64 restatement of the chunkwise algorithm (same
  summary, steps 2-5), used to pin the oracle and to give the per-chunk
  intermediates (coefficients, Gamma, T) a definition of their own.
* ``gates_ref``: the gate pre-operation and query correction (same summary,
  steps 6-7; article, sections 5 and 8) in NumPy fp64.

Every function cites the passage it follows; the pins that tie the oracle to
the pages live in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mdn_oracle.c")
_LIB = os.path.join(_HERE, "libmdn_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the C oracle with gcc (-O2, no fast-math, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
               "-Wall", "-o", tmp, _SRC]
        subprocess.check_call(cmd)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        d = ctypes.POINTER(ctypes.c_double)
        L = ctypes.c_long
        lib.mdn_oracle_fwd.argtypes = [L, L, L, L] + [d] * 7 + [ctypes.c_void_p, ctypes.c_void_p] + [d] * 4
        lib.mdn_oracle_fwd.restype = None
        lib.mdn_oracle_step.argtypes = [L, L, L] + [d] * 7 + [d] * 4
        lib.mdn_oracle_step.restype = None
        lib.mdn_oracle_bwd.argtypes = ([L, L, L, L] + [d] * 7 + [ctypes.c_void_p] * 2 + [d]
                                       + [ctypes.c_void_p] * 2 + [d] * 9)
        lib.mdn_oracle_bwd.restype = None
        lib.mdn_oracle_threads.argtypes = []
        lib.mdn_oracle_threads.restype = ctypes.c_int
        lib.mdn_oracle_set_threads.argtypes = [ctypes.c_int]
        lib.mdn_oracle_set_threads.restype = None
        _lib = lib
    return _lib


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def threads() -> int:
    """OpenMP threads the C oracle uses."""
    return int(_load().mdn_oracle_threads())


def set_threads(n: int) -> None:
    """Use n OpenMP threads in the following oracle calls."""
    _load().mdn_oracle_set_threads(int(n))


def fwd(q, k, v, alpha, mu, beta, eta, S0=None, M0=None):
    """Token-by-token MDN forward in fp64.

    Shapes: q, k ``[..., T, dk]``; v ``[..., T, dv]``; gates ``[..., T]``;
    S0, M0 ``[..., dk, dv]`` or None (zero).  Leading dims are flattened into
    independent heads.  Returns ``(O, S_T, M_T, Vtilde)`` as float64 arrays
    with ``O, Vtilde: [..., T, dv]`` and ``S_T, M_T: [..., dk, dv]``.

    Follows the recurrence of the MDN summary (paper.rainbus.top), method
    walk-through step 1, with the read-out o_t = S_t^T q_t taken after the
    update of token t.
    """
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    alpha, mu, beta, eta = _f64(alpha), _f64(mu), _f64(beta), _f64(eta)
    lead = q.shape[:-2]
    T, dk = q.shape[-2], q.shape[-1]
    dv = v.shape[-1]
    assert k.shape == q.shape and v.shape[:-1] == q.shape[:-1]
    assert alpha.shape == lead + (T,) and mu.shape == alpha.shape
    assert beta.shape == alpha.shape and eta.shape == alpha.shape
    BH = int(np.prod(lead)) if lead else 1
    O = np.zeros(lead + (T, dv))
    Vt = np.zeros(lead + (T, dv))
    ST = np.zeros(lead + (dk, dv))
    MT = np.zeros(lead + (dk, dv))
    s0p = None
    m0p = None
    if S0 is not None:
        S0 = _f64(np.broadcast_to(S0, lead + (dk, dv)))
        s0p = S0.ctypes.data
    if M0 is not None:
        M0 = _f64(np.broadcast_to(M0, lead + (dk, dv)))
        m0p = M0.ctypes.data
    lib.mdn_oracle_fwd(BH, T, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(mu),
                       _ptr(beta), _ptr(eta), s0p, m0p, _ptr(O), _ptr(ST), _ptr(MT), _ptr(Vt))
    return O, ST, MT, Vt


def bwd(q, k, v, alpha, mu, beta, eta, S0=None, M0=None, dO=None, dST=None, dMT=None):
    """Gradients of L = sum(dO*O) + sum(dST*S_T) + sum(dMT*M_T) in fp64.

    Same shapes as :func:`fwd`; dO like O, dST/dMT like S_T (None = zero).
    Returns a dict with dq, dk, dv, dalpha, dmu, dbeta, deta, dS0, dM0 (the
    gradient with respect to the initial states, zero or not).

    Reverse mode of the recurrence of the MDN summary (paper.rainbus.top,
    method walk-through step 1), one token at a time, last token first: the
    chain rule applied to the four update equations (the C source lists each
    term).  The states are replayed from checkpoints every 64 tokens.
    """
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    alpha, mu, beta, eta = _f64(alpha), _f64(mu), _f64(beta), _f64(eta)
    lead = q.shape[:-2]
    T, dk = q.shape[-2], q.shape[-1]
    dv = v.shape[-1]
    BH = int(np.prod(lead)) if lead else 1
    dO = np.zeros(lead + (T, dv)) if dO is None else _f64(np.broadcast_to(dO, lead + (T, dv)))
    keep = []

    def opt(x):
        if x is None:
            return None
        a = _f64(np.broadcast_to(x, lead + (dk, dv)))
        keep.append(a)
        return a.ctypes.data

    out = dict(dq=np.zeros(lead + (T, dk)), dk=np.zeros(lead + (T, dk)), dv=np.zeros(lead + (T, dv)),
               dalpha=np.zeros(lead + (T,)), dmu=np.zeros(lead + (T,)), dbeta=np.zeros(lead + (T,)),
               deta=np.zeros(lead + (T,)), dS0=np.zeros(lead + (dk, dv)), dM0=np.zeros(lead + (dk, dv)))
    lib.mdn_oracle_bwd(BH, T, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(mu), _ptr(beta),
                       _ptr(eta), opt(S0), opt(M0), _ptr(dO), opt(dST), opt(dMT),
                       *(_ptr(out[n]) for n in ("dq", "dk", "dv", "dalpha", "dmu", "dbeta", "deta",
                                                "dS0", "dM0")))
    return out


def fwd_varlen(q, k, v, alpha, mu, beta, eta, cu, S0=None, M0=None):
    """Packed variable-length forward in fp64: each sequence runs the
    recurrence of :func:`fwd` on its own tokens from its own initial state.

    q, k ``[H, T, dk]``; v ``[H, T, dv]``; gates ``[H, T]``; ``cu`` the
    ``nseq + 1`` sequence starts (sequence i is tokens ``cu[i]:cu[i+1]`` of
    every head); S0, M0 ``[nseq, H, dk, dv]`` or None (zero).  Returns
    ``(O [H,T,dv], S_T [nseq,H,dk,dv], M_T, Vtilde [H,T,dv])``.

    The recurrence is the MDN summary's (paper.rainbus.top, method
    walk-through step 1); a sequence start resets the state to that
    sequence's initial state, so no token of one sequence reaches another.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    alpha, mu, beta, eta = _f64(alpha), _f64(mu), _f64(beta), _f64(eta)
    cu = np.asarray(cu, dtype=np.int64)
    H, T, dk = q.shape
    dv = v.shape[-1]
    nseq = len(cu) - 1
    assert cu[0] == 0 and cu[-1] == T and np.all(np.diff(cu) >= 0)
    O = np.zeros((H, T, dv))
    Vt = np.zeros((H, T, dv))
    ST = np.zeros((nseq, H, dk, dv))
    MT = np.zeros((nseq, H, dk, dv))
    for i in range(nseq):
        a, b = int(cu[i]), int(cu[i + 1])
        s0 = None if S0 is None else S0[i]
        m0 = None if M0 is None else M0[i]
        if a == b:
            ST[i] = 0.0 if s0 is None else s0
            MT[i] = 0.0 if m0 is None else m0
            continue
        o, st, mt, vt = fwd(q[:, a:b], k[:, a:b], v[:, a:b], alpha[:, a:b], mu[:, a:b],
                            beta[:, a:b], eta[:, a:b], s0, m0)
        O[:, a:b], Vt[:, a:b], ST[i], MT[i] = o, vt, st, mt
    return O, ST, MT, Vt


def step(q, k, v, alpha, mu, beta, eta, S, M, inplace=False):
    """One decode step of the recurrence for every head, fp64.

    q, k ``[..., dk]``; v ``[..., dv]``; gates ``[...]``; S, M ``[..., dk, dv]``.
    Returns ``(o, S_new, M_new, vtilde)``.  The inputs S and M are not
    modified, unless ``inplace`` is set: then they must be C-contiguous fp64
    arrays of the full shape, are updated in place and returned as S_new,
    M_new (which saves two copies of the states per step on large batches).
    Same equations as :func:`fwd` (one token): the recurrent form the MDN
    article (ijyty.com, section 6) says generation uses.
    """
    lib = _load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    alpha, mu, beta, eta = _f64(alpha), _f64(mu), _f64(beta), _f64(eta)
    lead = q.shape[:-1]
    dk, dv = q.shape[-1], v.shape[-1]
    BH = int(np.prod(lead)) if lead else 1
    if inplace:
        for name, a in (("S", S), ("M", M)):
            if not (isinstance(a, np.ndarray) and a.dtype == np.float64 and a.flags.c_contiguous
                    and a.shape == lead + (dk, dv)):
                raise ValueError(f"inplace step: {name} must be a C-contiguous float64 array of shape "
                                 f"{lead + (dk, dv)}")
        S2, M2 = S, M
    else:
        S2 = np.array(np.broadcast_to(S, lead + (dk, dv)), dtype=np.float64, order="C", copy=True)
        M2 = np.array(np.broadcast_to(M, lead + (dk, dv)), dtype=np.float64, order="C", copy=True)
    o = np.zeros(lead + (dv,))
    vt = np.zeros(lead + (dv,))
    lib.mdn_oracle_step(BH, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(mu),
                        _ptr(beta), _ptr(eta), _ptr(S2), _ptr(M2), _ptr(o), _ptr(vt))
    return o, S2, M2, vt


from . import chunk_ref  # noqa: E402,F401
