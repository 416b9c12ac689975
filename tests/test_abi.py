"""C-ABI checks that need no GPU: the library loads, exports every function
``include/mdn.h`` declares, and rejects bad arguments on the host before any
HIP call (fake device addresses are never dereferenced by validation)."""
import ctypes
import os
import re
import subprocess

import pytest

import linear_attention_sequence_mdn_amd as mdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mdn.h")

OK, NULL_ARG, BAD_SHAPE, UNSUPPORTED, ALIAS, WORKSPACE, ALIGN, TOO_LARGE = 0, 1, 2, 3, 4, 5, 6, 8


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(mdn.LIB_PATH):
        pytest.fail("libmdn.so not built: run __graft_entry__.build() first")
    return mdn.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mdn_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    names = declared_functions()
    for n in ("mdn_chunk_fwd", "mdn_step", "mdn_chunk_fwd_workspace_bytes", "mdn_chunk_intra",
              "mdn_chunk_inter", "mdn_chunk_coef", "mdn_gates", "mdn_chunk_fwd_varlen",
              "mdn_chunk_fwd_varlen_workspace_bytes", "mdn_chunk_bwd", "mdn_chunk_bwd_workspace_bytes",
              "mdn_chunk_fwd_fused", "mdn_chunk_fwd_noalloc", "mdn_stream_rw",
              "mdn_chunk_fwd_split", "mdn_chunk_fwd_split_workspace_bytes",
              "mdn_status_string", "mdn_abi_version"):
        assert n in names


def test_every_declared_symbol_is_exported(L):
    out = subprocess.run(["nm", "-D", "--defined-only", mdn.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    for n in declared_functions():
        getattr(L, n)   # resolvable through the loader too


def test_abi_version(L):
    assert L.mdn_abi_version() == 8


def test_status_strings(L):
    for s in range(9):
        assert L.mdn_status_string(s).startswith(b"MDN_")
    assert L.mdn_status_string(99) == b"unknown mdn status"


def test_workspace_bytes(L):
    # T matrices + (QK^T) o Gamma (bf16, C x C per chunk) + 8 coefficient rows (fp32)
    B, H, T, d, C = 8, 8, 4096, 128, 64
    tiles = B * H * (T // C)
    expect = 2 * tiles * C * C * 2 + tiles * 8 * C * 4
    assert mdn.chunk_fwd_workspace_bytes(B, H, T, d, d, C, mdn.MDN_BF16) == expect
    assert L.mdn_chunk_fwd_workspace_bytes(1, 1, 0, 16, 16, 16, 0) == 0
    bad = ctypes.c_size_t(-1).value
    assert L.mdn_chunk_fwd_workspace_bytes(1, 1, 64, 48, 48, 16, 0) == bad
    # bf16 at d = 16 or C = 16 runs the fp32 kernels on widened copies: the
    # fp32 workspace, then fp32 q, k, v, O and vtilde
    f32 = L.mdn_chunk_fwd_workspace_bytes(1, 1, 64, 16, 16, 16, 0)
    assert L.mdn_chunk_fwd_workspace_bytes(1, 1, 64, 16, 16, 16, 1) == f32 + 5 * 64 * 16 * 4
    f32 = L.mdn_chunk_fwd_workspace_bytes(2, 3, 100, 128, 128, 16, 0)
    assert L.mdn_chunk_fwd_workspace_bytes(2, 3, 100, 128, 128, 16, 1) == f32 + 5 * 600 * 128 * 4
    assert L.mdn_chunk_fwd_workspace_bytes(-1, 1, 64, 16, 16, 16, 0) == bad


# fake, 256-byte aligned, non-overlapping device addresses
BASE = 1 << 40


def addrs(n, stride=1 << 32):
    return [ctypes.c_void_p(BASE + i * stride) for i in range(n)]


def chunk_call(L, B=1, H=1, T=64, d=16, C=16, dt=0, ptrs=None, ws_bytes=None, S0=None, M0=None):
    p = addrs(14) if ptrs is None else ptrs
    q, k, v, a, m, b, e, s0, m0, O, ST, MT, Vt, ws = p
    if S0 is not None:
        s0 = S0
    if M0 is not None:
        m0 = M0
    n = L.mdn_chunk_fwd_workspace_bytes(B, H, T, d, d, C, dt) if ws_bytes is None else ws_bytes
    return L.mdn_chunk_fwd(B, H, T, d, d, C, dt, q, k, v, a, m, b, e, s0, m0, O, ST, MT, Vt,
                           ws, n, None)


def test_chunk_unsupported(L):
    assert chunk_call(L, d=48) == UNSUPPORTED
    assert chunk_call(L, C=128) == UNSUPPORTED
    assert chunk_call(L, d=16, C=128, dt=1) == UNSUPPORTED
    # the widened bf16 shapes need the widened workspace
    assert chunk_call(L, d=16, dt=1, ws_bytes=L.mdn_chunk_fwd_workspace_bytes(1, 1, 64, 16, 16, 16, 0)) == WORKSPACE
    assert chunk_call(L, dt=7) == UNSUPPORTED
    p = addrs(14)
    assert L.mdn_chunk_fwd(1, 1, 64, 32, 64, 32, 1, *p[:13], p[13], 1 << 20, None) == UNSUPPORTED


def test_chunk_bad_shape(L):
    assert chunk_call(L, B=-1) == BAD_SHAPE
    assert chunk_call(L, T=-5) == BAD_SHAPE
    assert chunk_call(L, B=1 << 30, H=1 << 30, T=1 << 20) == BAD_SHAPE


def test_chunk_empty_batch_is_noop(L):
    assert chunk_call(L, B=0) == OK
    assert chunk_call(L, H=0, ptrs=[None] * 14) == OK


def test_chunk_null_args(L):
    p = addrs(14)
    for i in (0, 1, 2, 3, 4, 5, 6, 9, 10, 11, 12):
        q = list(p)
        q[i] = None
        assert chunk_call(L, ptrs=q) == NULL_ARG, i
    q = list(p)
    q[7] = q[8] = None          # S0, M0 may be NULL (zero state)
    assert chunk_call(L, ptrs=q, ws_bytes=0) == WORKSPACE


def test_chunk_workspace(L):
    need = L.mdn_chunk_fwd_workspace_bytes(1, 1, 64, 16, 16, 16, 0)
    assert chunk_call(L, ws_bytes=need - 1) == WORKSPACE
    q = addrs(14)
    q[13] = None
    assert chunk_call(L, ptrs=q) == WORKSPACE


def test_chunk_alignment(L):
    q = addrs(14)
    q[4] = ctypes.c_void_p(q[4].value + 4)
    assert chunk_call(L, ptrs=q) == ALIGN


def test_chunk_alias(L):
    p = addrs(14)
    q = list(p)
    q[9] = q[0]                 # O on top of q
    assert chunk_call(L, ptrs=q) == ALIAS
    q = list(p)
    q[12] = ctypes.c_void_p(p[9].value + 256)   # Vtilde overlapping O
    assert chunk_call(L, ptrs=q) == ALIAS
    q = list(p)
    q[13] = q[3]                # workspace on alpha
    assert chunk_call(L, ptrs=q) == ALIAS
    q = list(p)
    q[10] = ctypes.c_void_p(p[7].value + 256)   # S_T overlapping S0 but not equal
    assert chunk_call(L, ptrs=q) == ALIAS


def step_call(L, B=2, H=2, d=16, dt=0, ptrs=None):
    p = addrs(10) if ptrs is None else ptrs
    return L.mdn_step(B, H, d, d, dt, *p, None)


def test_step_validation(L):
    assert step_call(L, d=8) == UNSUPPORTED
    assert step_call(L, dt=5) == UNSUPPORTED
    assert step_call(L, B=-2) == BAD_SHAPE
    assert step_call(L, B=0) == OK
    p = addrs(10)
    for i in range(10):
        q = list(p)
        q[i] = None
        assert step_call(L, ptrs=q) == NULL_ARG, i
    q = list(p)
    q[8] = q[7]                 # M on top of S
    assert step_call(L, ptrs=q) == ALIAS
    q = list(p)
    q[9] = q[0]                 # o on top of q
    assert step_call(L, ptrs=q) == ALIAS
    q = list(p)
    q[7] = ctypes.c_void_p(p[7].value + 8)
    assert step_call(L, ptrs=q) == ALIGN


def test_noalloc_validation(L):
    # host-side checks, made before the scratch is looked up (no device needed)
    p = addrs(13)
    f = lambda B, H, T, d, C, dt, ptrs=p: L.mdn_chunk_fwd_noalloc(B, H, T, d, d, C, dt, *ptrs, None)
    assert f(8, 8, 4672, 128, 64, 1) == TOO_LARGE       # 4672 tiles of 18 KiB: beyond the 80 MiB scratch
    assert f(8, 8, 4096, 48, 64, 1) == UNSUPPORTED
    assert f(-1, 8, 4096, 128, 64, 1) == BAD_SHAPE
    assert f(0, 8, 4096, 128, 64, 1) == OK               # empty: no workspace, nothing to do


def test_stream_rw_validation(L):
    p = addrs(1)[0]
    assert L.mdn_stream_rw(p, -16, 1.0, None) == BAD_SHAPE
    assert L.mdn_stream_rw(p, 24, 1.0, None) == BAD_SHAPE
    assert L.mdn_stream_rw(p, 1 << 48, 1.0, None) == BAD_SHAPE
    assert L.mdn_stream_rw(None, 0, 1.0, None) == OK
    assert L.mdn_stream_rw(None, 64, 1.0, None) == NULL_ARG
    assert L.mdn_stream_rw(ctypes.c_void_p(p.value + 4), 64, 1.0, None) == ALIGN


def test_coef_validation(L):
    p = addrs(6)
    assert L.mdn_chunk_coef(1, 1, 64, 48, *p, None) == UNSUPPORTED
    assert L.mdn_chunk_coef(1, 1, -1, 16, *p, None) == BAD_SHAPE
    assert L.mdn_chunk_coef(1, 1, 0, 16, *p, None) == OK
    q = list(p)
    q[4] = None
    assert L.mdn_chunk_coef(1, 1, 64, 16, *q, None) == NULL_ARG
    q = list(p)
    q[5] = q[4]
    assert L.mdn_chunk_coef(1, 1, 64, 16, *q, None) == ALIAS


def test_binding_raises_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(mdn, "_lib", None)
    monkeypatch.setattr(mdn, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="missing"):
        mdn.lib()


def test_stage_entry_points_validate(L):
    p = addrs(14)
    q, k, v, a, m, b, e, s0, m0, O, ST, MT, Vt, ws = p
    need = L.mdn_chunk_fwd_workspace_bytes(1, 1, 64, 16, 16, 16, 0)
    assert L.mdn_chunk_intra(1, 1, 64, 16, 16, 16, 0, q, k, a, m, b, e, ws, need - 1, None) == WORKSPACE
    assert L.mdn_chunk_intra(1, 1, 64, 16, 16, 16, 0, None, k, a, m, b, e, ws, need, None) == NULL_ARG
    assert L.mdn_chunk_intra(1, 1, 64, 48, 48, 16, 0, q, k, a, m, b, e, ws, need, None) == UNSUPPORTED
    # the stage entry points expose the workspace in the element type: they
    # take the natively compiled shapes only
    assert L.mdn_chunk_intra(1, 1, 64, 16, 16, 16, 1, q, k, a, m, b, e, ws, need, None) == UNSUPPORTED
    assert L.mdn_chunk_intra(1, 1, 64, 16, 16, 16, 0, q, k, a, m, b, e, q, need, None) == ALIAS
    assert L.mdn_chunk_inter(1, 1, 64, 16, 16, 16, 0, q, k, v, a, m, b, e, s0, m0, O, ST, MT, None,
                             ws, need, None) == NULL_ARG
    assert L.mdn_chunk_inter(1, 1, 64, 16, 16, 16, 0, q, k, v, a, m, b, e, s0, m0, O, ST, MT, O,
                             ws, need, None) == ALIAS


def test_gates_validation(L):
    p = addrs(12)
    x, a, b, ml, al, mu, be, et, q, k, d, qo = p
    f = ctypes.c_float
    args = lambda **kw: [kw.get(n, v) for n, v in zip(
        ("x", "a", "b", "ml", "al", "mu", "be", "et", "q", "k", "d", "qo"), p)]
    call = lambda B=1, H=2, T=64, dk=16, dt=1, s=1.0, lo=-2.0, **kw: L.mdn_gates(
        B, H, T, dk, dt, f(s), f(lo), *args(**kw), None)
    assert call(T=-1) == BAD_SHAPE
    assert call(s=0.0) == BAD_SHAPE and call(s=float("inf")) == BAD_SHAPE
    assert call(lo=0.5) == BAD_SHAPE and call(lo=float("nan")) == BAD_SHAPE
    assert call(dt=7) == UNSUPPORTED
    assert call(dk=48) == UNSUPPORTED
    assert call(d=None) == NULL_ARG                      # correction half given
    assert call(T=0) == OK                               # nothing to do
    assert call(x=None) == NULL_ARG
    assert call(al=ctypes.c_void_p(al.value + 4)) == ALIGN
    assert call(al=x) == ALIAS                           # output on an input
    assert call(mu=al) == ALIAS                          # two outputs on each other
    assert call(qo=k) == ALIAS
    # no correction at all: q, k, d, q_out all NULL and dk is not checked
    assert L.mdn_gates(1, 2, 0, 48, 1, f(1.0), f(-2.0), x, a, b, ml, al, mu, be, et,
                       None, None, None, None, None) == OK


def varlen_call(L, H=2, T=100, nseq=3, d=32, C=32, dt=1, cu=None, ptrs=None, ws_bytes=None):
    p = addrs(14) if ptrs is None else ptrs
    cu = ctypes.c_void_p(BASE - (1 << 20)) if cu is None else cu
    n = L.mdn_chunk_fwd_varlen_workspace_bytes(H, T, nseq, d, d, C, dt) if ws_bytes is None else ws_bytes
    return L.mdn_chunk_fwd_varlen(H, T, nseq, cu, d, d, C, dt, *p[:13], p[13], n, None)


def test_varlen_workspace_bytes(L):
    # tile slots T // C + nseq per head; T, Aqk (bf16), coefficients, the slot table, the order
    H, T, nseq, d, C = 8, 32768, 19, 128, 64
    slots = H * (T // C + nseq)
    a256 = lambda x: (x + 255) // 256 * 256
    expect = (2 * a256(slots * C * C * 2) + a256(slots * 8 * C * 4) + a256((T // C + nseq) * 8)
              + a256(nseq * 4))
    assert mdn.chunk_fwd_varlen_workspace_bytes(H, T, nseq, d, d, C, mdn.MDN_BF16) == expect
    bad = ctypes.c_size_t(-1).value
    assert L.mdn_chunk_fwd_varlen_workspace_bytes(1, 1 << 31, 1, 32, 32, 32, 1) == bad   # beyond int32
    assert L.mdn_chunk_fwd_varlen_workspace_bytes(1, 64, -1, 32, 32, 32, 1) == bad
    assert L.mdn_chunk_fwd_varlen_workspace_bytes(1, 64, 2, 48, 48, 32, 1) == bad


def test_varlen_validation(L):
    assert varlen_call(L, nseq=-1) == BAD_SHAPE
    assert varlen_call(L, T=1 << 31) == BAD_SHAPE
    assert varlen_call(L, d=48) == UNSUPPORTED
    assert varlen_call(L, nseq=0, ptrs=[None] * 14, cu=ctypes.c_void_p(0)) == OK   # nothing to do
    assert varlen_call(L, H=0, ptrs=[None] * 14) == OK
    assert varlen_call(L, cu=ctypes.c_void_p(0)) == NULL_ARG
    assert varlen_call(L, cu=ctypes.c_void_p(BASE - (1 << 20) + 2)) == ALIGN
    p = addrs(14)
    for i in (0, 1, 2, 3, 9, 10, 11, 12):
        q = list(p)
        q[i] = None
        assert varlen_call(L, ptrs=q) == NULL_ARG, i
    assert varlen_call(L, ws_bytes=1) == WORKSPACE
    q = list(p)
    q[9] = q[0]                                          # O on top of q
    assert varlen_call(L, ptrs=q) == ALIAS
    assert varlen_call(L, cu=p[13]) == ALIAS             # sequence bounds inside the workspace


def bwd_call(L, B=1, H=2, T=64, d=32, C=32, dt=1, ptrs=None, ws_bytes=None):
    p = addrs(22) if ptrs is None else ptrs
    n = L.mdn_chunk_bwd_workspace_bytes(B, H, T, d, d, C, dt) if ws_bytes is None else ws_bytes
    return L.mdn_chunk_bwd(B, H, T, d, d, C, dt, *p[:21], p[21], n, None)


def test_bwd_workspace_bytes(L):
    # T^T, Aqk^T (bf16 C x C per chunk), 8 coefficient rows, four d x d states
    # and two C x d partial gradients (bf16), and 8 rows of coefficient adjoints
    B, H, T, d, C = 8, 8, 4096, 128, 64
    tiles = B * H * (T // C)
    expect = (2 * tiles * C * C * 2 + tiles * 8 * C * 4 + 4 * tiles * d * d * 2 + 2 * tiles * C * d * 2
              + tiles * 8 * C * 4)
    assert mdn.chunk_bwd_workspace_bytes(B, H, T, d, d, C, mdn.MDN_BF16) == expect
    bad = ctypes.c_size_t(-1).value
    assert L.mdn_chunk_bwd_workspace_bytes(1, 1, 64, 48, 48, 16, 0) == bad
    # widened bf16 shapes: the fp32 workspace, then fp32 q, k, vtilde, dO, dq, dk, dv
    for d, C in ((16, 32), (128, 16)):
        f32 = L.mdn_chunk_bwd_workspace_bytes(1, 1, 64, d, d, C, 0)
        assert L.mdn_chunk_bwd_workspace_bytes(1, 1, 64, d, d, C, 1) == f32 + 7 * 64 * d * 4


def test_bwd_validation(L):
    assert bwd_call(L, d=48) == UNSUPPORTED
    assert bwd_call(L, dt=1, d=16, C=128) == UNSUPPORTED
    assert bwd_call(L, dt=1, d=16, C=32, ws_bytes=L.mdn_chunk_bwd_workspace_bytes(1, 2, 64, 16, 16, 32, 0)) == WORKSPACE
    assert bwd_call(L, T=-1) == BAD_SHAPE
    assert bwd_call(L, B=0, ptrs=[None] * 22) == OK
    p = addrs(22)
    for i in (0, 1, 2, 3, 4, 5, 8, 9, 12, 13, 14, 15, 16, 17, 18, 19, 20):
        q = list(p)
        q[i] = None
        assert bwd_call(L, ptrs=q) == NULL_ARG, i
    q = list(p)
    q[6] = q[7] = q[10] = q[11] = None       # S0, M0, dS_T, dM_T may be NULL
    assert bwd_call(L, ptrs=q, ws_bytes=0) == WORKSPACE
    assert bwd_call(L, ws_bytes=1) == WORKSPACE
    q = list(p)
    q[2] = ctypes.c_void_p(p[2].value + 4)
    assert bwd_call(L, ptrs=q) == ALIGN
    q = list(p)
    q[12] = q[0]                               # dq on top of q
    assert bwd_call(L, ptrs=q) == ALIAS
    q = list(p)
    q[21] = q[8]                               # workspace on Vtilde
    assert bwd_call(L, ptrs=q) == ALIAS


def test_fused_forward_validation(L):
    p = addrs(13)
    f = lambda B=1, H=2, T=64, d=128, C=64, dt=1, ptrs=p: L.mdn_chunk_fwd_fused(B, H, T, d, d, C, dt, *ptrs, None)
    assert f(dt=0) == UNSUPPORTED                 # fp32
    assert f(C=32) == UNSUPPORTED
    assert f(d=32) == UNSUPPORTED
    assert L.mdn_chunk_fwd_fused(1, 2, 64, 128, 64, 64, 1, *p, None) == UNSUPPORTED   # dk != dv
    assert f(B=-1) == BAD_SHAPE
    assert f(B=0, ptrs=[None] * 13) == OK
    for i in (0, 1, 2, 3, 4, 5, 6, 9, 10, 11, 12):
        q = list(p)
        q[i] = None
        assert f(ptrs=q) == NULL_ARG, i
    q = list(p)
    q[9] = q[0]                                   # O over q
    assert f(ptrs=q) == ALIAS
    q = list(p)
    q[12] = ctypes.c_void_p(BASE + 8)             # misaligned vtilde
    assert f(ptrs=q) == ALIGN


def test_split_forward_validation(L):
    """mdn_chunk_fwd_split: the forward's workspace plus 2 * BH (1 + 4 (nseg - 2))
    fp32 state slots; native sizes and 2 <= nseg <= 64 only; the state slots
    count in the workspace and alias checks."""
    bad = ctypes.c_size_t(-1).value
    B, H, T, d, C = 1, 16, 16384, 128, 64
    base = 2 * B * H * (T // C) * C * C * 2 + B * H * (T // C) * 8 * C * 4     # the single pass's workspace
    for nseg in (2, 3, 5):
        slots = B * H * (1 + 4 * (nseg - 2)) * d * d * 4
        assert L.mdn_chunk_fwd_split_workspace_bytes(B, H, T, d, d, C, 1, nseg) == base + 2 * slots
    assert L.mdn_chunk_fwd_split_workspace_bytes(B, H, T, d, d, C, 1, 1) == bad
    assert L.mdn_chunk_fwd_split_workspace_bytes(B, H, T, d, d, C, 1, 65) == bad
    assert L.mdn_chunk_fwd_split_workspace_bytes(1, 1, 64, 16, 16, 16, 1, 3) == bad     # widened bf16 shape
    # mdn_chunk_fwd sizes its workspace for the sequence split where it
    # takes it (few heads of bf16 d = 128, C = 64, long sequences; the head
    # range depends on the device's compute units), else for one pass
    assert L.mdn_chunk_fwd_workspace_bytes(B, H, T, d, d, C, 1) in (
        base, L.mdn_chunk_fwd_split_workspace_bytes(B, H, T, d, d, C, 1, 3))
    one_pass = 2 * 64 * 64 * 64 * 64 * 2 + 64 * 64 * 8 * 64 * 4
    assert L.mdn_chunk_fwd_workspace_bytes(8, 8, 4096, 128, 128, 64, 1) == one_pass
    assert L.mdn_chunk_fwd_workspace_bytes(1, 16, 1024, 128, 128, 64, 1) == 2 * 16 * 16 * 64 * 64 * 2 + 16 * 16 * 8 * 64 * 4
    p = addrs(14)

    def f(B=1, H=2, T=640, d=64, C=64, dt=1, nseg=3, ptrs=p, ws=None):
        n = L.mdn_chunk_fwd_split_workspace_bytes(B, H, T, d, d, C, dt, nseg) if ws is None else ws
        return L.mdn_chunk_fwd_split(B, H, T, d, d, C, dt, nseg, *ptrs[:13], ptrs[13], n, None)
    assert f(nseg=1, ws=1 << 30) == UNSUPPORTED
    assert f(nseg=65, ws=1 << 30) == UNSUPPORTED
    assert f(d=16) == UNSUPPORTED and f(C=16, ws=1 << 30) == UNSUPPORTED
    assert f(d=48, ws=1 << 30) == UNSUPPORTED
    assert f(B=-1, ws=1 << 30) == BAD_SHAPE
    assert f(B=0, ptrs=[None] * 14, ws=0) == OK
    # the forward's own workspace is not enough
    assert f(ws=L.mdn_chunk_fwd_workspace_bytes(1, 2, 640, 64, 64, 64, 1)) == WORKSPACE
    for i in (0, 1, 2, 3, 4, 5, 6, 9, 10, 11, 12, 13):
        q = list(p)
        q[i] = None
        assert f(ptrs=q) == (WORKSPACE if i == 13 else NULL_ARG), i
    # an output inside the state slots at the end of the workspace
    q = list(p)
    q[10] = ctypes.c_void_p(p[13].value + L.mdn_chunk_fwd_split_workspace_bytes(1, 2, 640, 64, 64, 64, 1, 3) - 256)
    assert f(ptrs=q) == ALIAS
    q = list(p)
    q[12] = ctypes.c_void_p(BASE + 8)             # misaligned vtilde
    assert f(ptrs=q) == ALIGN
