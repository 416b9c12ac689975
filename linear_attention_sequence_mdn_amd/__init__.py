"""MI355X-native Momentum DeltaNet hot path: thin binding over ``libmdn.so``.

Every step of the computation runs in the HIP kernels behind the C ABI
(``include/mdn.h``).  This module only marshals torch tensors into pointers,
sizes and the current HIP stream, allocates outputs and workspace with torch,
and turns nonzero status codes into :class:`MdnError`.  There is no CPU or
PyTorch fallback: if the library is missing, every call raises.

Entry points (same names as the C ABI):
    chunk_fwd(q, k, v, alpha, mu, beta, eta, S0=None, M0=None, C=64)
        -> (O, S_T, M_T, Vtilde)
    chunk_fwd_noalloc(q, k, v, alpha, mu, beta, eta, S0, M0, C, out=(O, Vt), S_T=, M_T=)
        -> (O, S_T, M_T, Vtilde)   workspace in the library's static scratch
    chunk_fwd_fused(q, k, v, alpha, mu, beta, eta, S0=None, M0=None, C=64)
        -> (O, S_T, M_T, Vtilde)   the forward in one kernel, no workspace
                                   (bf16, C = 64, d in {64, 128})
    chunk_fwd_varlen(q, k, v, alpha, mu, beta, eta, cu_seqlens, S0=None, M0=None, C=64)
        -> (O, S_T, M_T, Vtilde)   packed variable-length batch
    step(q, k, v, alpha, mu, beta, eta, S, M) -> o   (S, M updated in place)
    chunk_coef(alpha, mu, beta, eta, C) -> (coef, gamma)
    gates(x, a, b, mu_log, s=1.0, mu_log_min=-2.0, q=None, k=None, d=None)
        -> (alpha, mu, beta, eta) [+ q_out]
    chunk_bwd(q, k, alpha, mu, beta, eta, Vtilde, dO, S0=None, M0=None, dS_T=None, dM_T=None, C=64)
        -> dict of dq, dk, dv, dalpha, dmu, dbeta, deta, dS0, dM0
    chunk_fwd_workspace_bytes(B, H, T, dk, dv, C, dtype) -> int
    chunk_fwd_varlen_workspace_bytes(H, T, nseq, dk, dv, C, dtype) -> int
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmdn.so")

MDN_F32 = 0
MDN_BF16 = 1
COEF_ROWS = 8
COEF_NAMES = ("abar", "abp", "b", "gS", "gM", "la", "lm", "logc")

_lib = None


class MdnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().mdn_status_string(status).decode()
        super().__init__(f"{where}: {msg} (status {status})")


def lib():
    """The loaded C library (ctypes); raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m linear_attention_sequence_mdn_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
        L.mdn_chunk_fwd_workspace_bytes.argtypes = [i64, i64, i64, i32, i32, i32, i32]
        L.mdn_chunk_fwd_workspace_bytes.restype = sz
        L.mdn_chunk_fwd.argtypes = [i64, i64, i64, i32, i32, i32, i32] + [vp] * 13 + [vp, sz, vp]
        L.mdn_chunk_fwd.restype = i32
        L.mdn_chunk_bwd_workspace_bytes.argtypes = [i64, i64, i64, i32, i32, i32, i32]
        L.mdn_chunk_bwd_workspace_bytes.restype = sz
        L.mdn_chunk_bwd.argtypes = [i64, i64, i64, i32, i32, i32, i32] + [vp] * 21 + [vp, sz, vp]
        L.mdn_chunk_bwd.restype = i32
        L.mdn_chunk_fwd_varlen_workspace_bytes.argtypes = [i64, i64, i64, i32, i32, i32, i32]
        L.mdn_chunk_fwd_varlen_workspace_bytes.restype = sz
        L.mdn_chunk_fwd_varlen.argtypes = [i64, i64, i64, vp, i32, i32, i32, i32] + [vp] * 13 + [vp, sz, vp]
        L.mdn_chunk_fwd_varlen.restype = i32
        L.mdn_chunk_fwd_noalloc.argtypes = [i64, i64, i64, i32, i32, i32, i32] + [vp] * 13 + [vp]
        L.mdn_chunk_fwd_noalloc.restype = i32
        L.mdn_chunk_fwd_split_workspace_bytes.argtypes = [i64, i64, i64, i32, i32, i32, i32, i32]
        L.mdn_chunk_fwd_split_workspace_bytes.restype = sz
        L.mdn_chunk_fwd_split.argtypes = [i64, i64, i64, i32, i32, i32, i32, i32] + [vp] * 13 + [vp, sz, vp]
        L.mdn_chunk_fwd_split.restype = i32
        L.mdn_chunk_fwd_fused.argtypes = [i64, i64, i64, i32, i32, i32, i32] + [vp] * 13 + [vp]
        L.mdn_chunk_fwd_fused.restype = i32
        L.mdn_chunk_intra.argtypes = [i64, i64, i64, i32, i32, i32, i32] + [vp] * 6 + [vp, sz, vp]
        L.mdn_chunk_intra.restype = i32
        L.mdn_chunk_inter.argtypes = [i64, i64, i64, i32, i32, i32, i32] + [vp] * 13 + [vp, sz, vp]
        L.mdn_chunk_inter.restype = i32
        L.mdn_step.argtypes = [i64, i64, i32, i32, i32] + [vp] * 10 + [vp]
        L.mdn_step.restype = i32
        L.mdn_chunk_coef.argtypes = [i64, i64, i64, i32] + [vp] * 6 + [vp]
        L.mdn_chunk_coef.restype = i32
        L.mdn_gates.argtypes = [i64, i64, i64, i32, i32, ctypes.c_float, ctypes.c_float] + [vp] * 12 + [vp]
        L.mdn_gates.restype = i32
        L.mdn_stream_rw.argtypes = [vp, i64, ctypes.c_float, vp]
        L.mdn_stream_rw.restype = i32
        L.mdn_status_string.argtypes = [i32]
        L.mdn_status_string.restype = ctypes.c_char_p
        L.mdn_abi_version.argtypes = []
        L.mdn_abi_version.restype = i32
        _lib = L
    return _lib


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return MDN_BF16
    if t.dtype == torch.float32:
        return MDN_F32
    raise TypeError(f"q/k/v must be bfloat16 or float32, got {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, owned=()):
    """The hipStream_t handle of `stream` (None = torch's current stream).

    `owned` are the tensors this binding allocated for the call (outputs,
    workspace).  They come from the caching allocator on the current stream;
    when the kernels run on another stream, each is recorded on that stream so
    that its memory is not handed out again before the kernels have finished
    with it, even if the caller drops it at once."""
    torch = _torch()
    cur = torch.cuda.current_stream()
    if stream is None:
        stream = cur
    elif stream != cur:
        for t in owned:
            if t is not None:
                t.record_stream(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status: int, where: str):
    if status != 0:
        raise MdnError(status, where)


def _need(t, name, dtype, shape, device):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name}: expected device {device}, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def chunk_fwd_workspace_bytes(B, H, T, dk, dv, C, dtype) -> int:
    n = lib().mdn_chunk_fwd_workspace_bytes(B, H, T, dk, dv, C, dtype)
    if n == ctypes.c_size_t(-1).value:
        raise MdnError(3, "mdn_chunk_fwd_workspace_bytes")
    return int(n)


_NO_WORKSPACE = object()      # ChunkCall(workspace=_NO_WORKSPACE): allocate none


class ChunkCall:
    """Validated, preallocated arguments of one chunk forward.

    Holds the output tensors and the workspace so that repeated calls (the
    benchmark, a training loop) allocate nothing; ``run()`` is
    ``mdn_chunk_fwd``, ``intra()``/``inter()`` its two stages."""

    def __init__(self, q, k, v, alpha, mu, beta, eta, S0=None, M0=None, C=64, *,
                 out=None, S_T=None, M_T=None, workspace=None):
        torch = _torch()
        B, H, T, dk = q.shape
        dv = v.shape[-1]
        self.dt = _dtype_code(q)
        dev = q.device
        _need(q, "q", q.dtype, (B, H, T, dk), dev)
        _need(k, "k", q.dtype, (B, H, T, dk), dev)
        _need(v, "v", q.dtype, (B, H, T, dv), dev)
        for name, g in (("alpha", alpha), ("mu", mu), ("beta", beta), ("eta", eta)):
            _need(g, name, torch.float32, (B, H, T), dev)
        for name, s in (("S0", S0), ("M0", M0)):
            if s is not None:
                _need(s, name, torch.float32, (B, H, dk, dv), dev)
        owned = []
        if out is None:
            O = torch.empty((B, H, T, dv), dtype=q.dtype, device=dev)
            Vt = torch.empty((B, H, T, dv), dtype=q.dtype, device=dev)
            owned += [O, Vt]
        else:
            O, Vt = out
        if S_T is None:
            S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
            owned.append(S_T)
        if M_T is None:
            M_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
            owned.append(M_T)
        if workspace is _NO_WORKSPACE:
            workspace = None
        else:
            nws = chunk_fwd_workspace_bytes(B, H, T, dk, dv, C, self.dt)
            if workspace is None and nws > 0:
                workspace = torch.empty(nws, dtype=torch.uint8, device=dev)
                owned.append(workspace)
        self._owned = owned
        self.sizes = (B, H, T, dk, dv, C, self.dt)
        self.tensors = (q, k, v, alpha, mu, beta, eta, S0, M0, O, S_T, M_T, Vt)
        self.workspace = workspace
        self.outputs = (O, S_T, M_T, Vt)
        self._ptrs = [_ptr(t) for t in self.tensors]
        self._ws = (_ptr(workspace) if workspace is not None else None,
                    workspace.numel() if workspace is not None else 0)

    def run(self, stream=None):
        _check(lib().mdn_chunk_fwd(*self.sizes, *self._ptrs, *self._ws, _stream(stream, self._owned)),
               "mdn_chunk_fwd")
        return self.outputs

    def intra(self, stream=None):
        p = self._ptrs
        _check(lib().mdn_chunk_intra(*self.sizes, p[0], p[1], p[3], p[4], p[5], p[6], *self._ws,
                                     _stream(stream, self._owned)), "mdn_chunk_intra")

    def fused(self, stream=None):
        """``mdn_chunk_fwd_fused`` on the same arguments (the workspace is
        not used)."""
        _check(lib().mdn_chunk_fwd_fused(*self.sizes, *self._ptrs, _stream(stream, self._owned)),
               "mdn_chunk_fwd_fused")
        return self.outputs

    def inter(self, stream=None):
        _check(lib().mdn_chunk_inter(*self.sizes, *self._ptrs, *self._ws, _stream(stream, self._owned)),
               "mdn_chunk_inter")
        return self.outputs

    def split(self, nseg, stream=None, workspace=None):
        """``mdn_chunk_fwd_split`` on the same arguments, each sequence cut
        into ``nseg`` segments; its workspace is ``workspace`` or one
        allocated on first use for that ``nseg`` and kept."""
        torch = _torch()
        B, H, T, dk, dv, C, dt = self.sizes
        need = chunk_fwd_split_workspace_bytes(B, H, T, dk, dv, C, dt, nseg)
        if workspace is None:
            cache = self.__dict__.setdefault("_split_ws", {})
            if nseg not in cache:
                cache[nseg] = torch.empty(max(need, 1), dtype=torch.uint8, device=self.outputs[0].device)
            workspace = cache[nseg]
        owned = list(self._owned) + [workspace]
        _check(lib().mdn_chunk_fwd_split(B, H, T, dk, dv, C, dt, int(nseg), *self._ptrs, _ptr(workspace),
                                         workspace.numel(), _stream(stream, owned)), "mdn_chunk_fwd_split")
        return self.outputs


def chunk_fwd(q, k, v, alpha, mu, beta, eta, S0=None, M0=None, C=64, *,
              out=None, S_T=None, M_T=None, workspace=None, stream=None):
    """Chunkwise forward: returns (O, S_T, M_T, Vtilde).

    q, k: [B,H,T,dk]; v: [B,H,T,dv] (bf16 or fp32, same dtype, on the GPU);
    gates [B,H,T] fp32; S0, M0 [B,H,dk,dv] fp32 or None.  ``out`` may be an
    (O, Vtilde) pair of preallocated tensors; ``S_T``/``M_T`` may alias S0/M0
    for an in-place update; ``workspace`` a uint8 tensor of at least
    ``chunk_fwd_workspace_bytes`` bytes.
    """
    call = ChunkCall(q, k, v, alpha, mu, beta, eta, S0, M0, C, out=out, S_T=S_T, M_T=M_T,
                     workspace=workspace)
    return call.run(stream)


def chunk_fwd_split_workspace_bytes(B, H, T, dk, dv, C, dtype, nseg) -> int:
    n = lib().mdn_chunk_fwd_split_workspace_bytes(B, H, T, dk, dv, C, dtype, nseg)
    if n == ctypes.c_size_t(-1).value:
        raise MdnError(3, "mdn_chunk_fwd_split_workspace_bytes")
    return int(n)


def chunk_fwd_split(q, k, v, alpha, mu, beta, eta, S0=None, M0=None, C=64, nseg=3, *,
                    out=None, S_T=None, M_T=None, workspace=None, stream=None):
    """``mdn_chunk_fwd_split``: the chunk forward with each sequence cut into
    ``nseg`` segments that run side by side (for few heads and long
    sequences); arguments and results as :func:`chunk_fwd`, ``workspace`` a
    uint8 tensor of at least ``chunk_fwd_split_workspace_bytes`` bytes."""
    call = ChunkCall(q, k, v, alpha, mu, beta, eta, S0, M0, C, out=out, S_T=S_T, M_T=M_T,
                     workspace=_NO_WORKSPACE)
    return call.split(nseg, stream, workspace)


NOALLOC_SCRATCH_BYTES = 80 << 20


def chunk_fwd_noalloc(q, k, v, alpha, mu, beta, eta, S0=None, M0=None, C=64, *, out, S_T, M_T, stream=None):
    """``mdn_chunk_fwd_noalloc``: the chunk forward with its workspace in the
    library's static device scratch, for callers that cannot allocate.  The
    caller passes every output: ``out`` = (O, Vtilde), ``S_T``, ``M_T``
    (shapes as in :func:`chunk_fwd`).  Calls that overlap in time on one GPU
    share the scratch and race."""
    call = ChunkCall(q, k, v, alpha, mu, beta, eta, S0, M0, C, out=out, S_T=S_T, M_T=M_T,
                     workspace=_NO_WORKSPACE)
    _check(lib().mdn_chunk_fwd_noalloc(*call.sizes, *call._ptrs, _stream(stream)), "mdn_chunk_fwd_noalloc")
    return call.outputs


def chunk_fwd_fused(q, k, v, alpha, mu, beta, eta, S0=None, M0=None, C=64, *, out=None, S_T=None, M_T=None,
                    stream=None):
    """``mdn_chunk_fwd_fused``: the chunk forward in one kernel, without a
    workspace (bf16, C = 64, dk = dv in {64, 128}); arguments and results as
    :func:`chunk_fwd`."""
    call = ChunkCall(q, k, v, alpha, mu, beta, eta, S0, M0, C, out=out, S_T=S_T, M_T=M_T,
                     workspace=_NO_WORKSPACE)
    return call.fused(stream)


def chunk_bwd_workspace_bytes(B, H, T, dk, dv, C, dtype) -> int:
    n = lib().mdn_chunk_bwd_workspace_bytes(B, H, T, dk, dv, C, dtype)
    if n == ctypes.c_size_t(-1).value:
        raise MdnError(3, "mdn_chunk_bwd_workspace_bytes")
    return int(n)


BWD_NAMES = ("dq", "dk", "dv", "dalpha", "dmu", "dbeta", "deta", "dS0", "dM0")


class BwdCall:
    """Validated, preallocated arguments of one ``mdn_chunk_bwd``; ``run()``
    allocates nothing and returns the dict of gradient tensors."""

    def __init__(self, q, k, alpha, mu, beta, eta, Vtilde, dO, S0=None, M0=None, dS_T=None, dM_T=None,
                 C=64, *, workspace=None):
        torch = _torch()
        B, H, T, dk = q.shape
        dv = Vtilde.shape[-1]
        self.dt = _dtype_code(q)
        dev = q.device
        _need(k, "k", q.dtype, (B, H, T, dk), dev)
        _need(Vtilde, "Vtilde", q.dtype, (B, H, T, dv), dev)
        _need(dO, "dO", q.dtype, (B, H, T, dv), dev)
        for name, g in (("alpha", alpha), ("mu", mu), ("beta", beta), ("eta", eta)):
            _need(g, name, torch.float32, (B, H, T), dev)
        for name, s in (("S0", S0), ("M0", M0), ("dS_T", dS_T), ("dM_T", dM_T)):
            if s is not None:
                _need(s, name, torch.float32, (B, H, dk, dv), dev)
        self.grads = dict(
            dq=torch.empty((B, H, T, dk), dtype=q.dtype, device=dev),
            dk=torch.empty((B, H, T, dk), dtype=q.dtype, device=dev),
            dv=torch.empty((B, H, T, dv), dtype=q.dtype, device=dev),
            dalpha=torch.empty((B, H, T), dtype=torch.float32, device=dev),
            dmu=torch.empty((B, H, T), dtype=torch.float32, device=dev),
            dbeta=torch.empty((B, H, T), dtype=torch.float32, device=dev),
            deta=torch.empty((B, H, T), dtype=torch.float32, device=dev),
            dS0=torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev),
            dM0=torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev))
        self._owned = list(self.grads.values())
        nws = chunk_bwd_workspace_bytes(B, H, T, dk, dv, C, self.dt)
        if workspace is None:
            workspace = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev)
            self._owned.append(workspace)
        self.workspace = workspace
        self.sizes = (B, H, T, dk, dv, C, self.dt)
        self.inputs = (q, k, alpha, mu, beta, eta, S0, M0, Vtilde, dO, dS_T, dM_T)
        self._ptrs = [_ptr(t) for t in self.inputs] + [_ptr(self.grads[n]) for n in BWD_NAMES]
        self._ws = (_ptr(workspace), workspace.numel())

    def run(self, stream=None):
        _check(lib().mdn_chunk_bwd(*self.sizes, *self._ptrs, *self._ws, _stream(stream, self._owned)),
               "mdn_chunk_bwd")
        return self.grads


def chunk_bwd(q, k, alpha, mu, beta, eta, Vtilde, dO, S0=None, M0=None, dS_T=None, dM_T=None, C=64, *,
              workspace=None, stream=None):
    """Backward of :func:`chunk_fwd`: gradients of a loss given dL/dO (and
    optionally dL/dS_T, dL/dM_T) for the forward's inputs.  ``Vtilde`` is the
    forward's output for the same inputs.  Returns a dict with dq, dk, dv
    ([B,H,T,d], input dtype), dalpha, dmu, dbeta, deta ([B,H,T] fp32) and
    dS0, dM0 ([B,H,dk,dv] fp32)."""
    return BwdCall(q, k, alpha, mu, beta, eta, Vtilde, dO, S0, M0, dS_T, dM_T, C, workspace=workspace).run(stream)


def chunk_fwd_varlen_workspace_bytes(H, T, nseq, dk, dv, C, dtype) -> int:
    n = lib().mdn_chunk_fwd_varlen_workspace_bytes(H, T, nseq, dk, dv, C, dtype)
    if n == ctypes.c_size_t(-1).value:
        raise MdnError(3, "mdn_chunk_fwd_varlen_workspace_bytes")
    return int(n)


class VarlenCall:
    """Validated, preallocated arguments of one packed variable-length
    forward (``mdn_chunk_fwd_varlen``); ``run()`` allocates nothing."""

    def __init__(self, q, k, v, alpha, mu, beta, eta, cu_seqlens, S0=None, M0=None, C=64, *,
                 out=None, S_T=None, M_T=None, workspace=None):
        torch = _torch()
        H, T, dk = q.shape
        dv = v.shape[-1]
        self.dt = _dtype_code(q)
        dev = q.device
        nseq = cu_seqlens.numel() - 1
        if cu_seqlens.dim() != 1 or nseq < 0:
            raise ValueError("cu_seqlens must be a 1-D tensor of nseq + 1 sequence starts")
        _need(cu_seqlens, "cu_seqlens", torch.int32, (nseq + 1,), dev)
        _need(q, "q", q.dtype, (H, T, dk), dev)
        _need(k, "k", q.dtype, (H, T, dk), dev)
        _need(v, "v", q.dtype, (H, T, dv), dev)
        for name, g in (("alpha", alpha), ("mu", mu), ("beta", beta), ("eta", eta)):
            _need(g, name, torch.float32, (H, T), dev)
        for name, s in (("S0", S0), ("M0", M0)):
            if s is not None:
                _need(s, name, torch.float32, (nseq, H, dk, dv), dev)
        owned = []
        if out is None:
            O = torch.empty((H, T, dv), dtype=q.dtype, device=dev)
            Vt = torch.empty((H, T, dv), dtype=q.dtype, device=dev)
            owned += [O, Vt]
        else:
            O, Vt = out
        if S_T is None:
            S_T = torch.empty((nseq, H, dk, dv), dtype=torch.float32, device=dev)
            owned.append(S_T)
        if M_T is None:
            M_T = torch.empty((nseq, H, dk, dv), dtype=torch.float32, device=dev)
            owned.append(M_T)
        nws = chunk_fwd_varlen_workspace_bytes(H, T, nseq, dk, dv, C, self.dt)
        if workspace is None and nws > 0:
            workspace = torch.empty(nws, dtype=torch.uint8, device=dev)
            owned.append(workspace)
        self._owned = owned
        self.sizes = (H, T, nseq)
        self.dims = (dk, dv, C, self.dt)
        self.cu = cu_seqlens
        self.tensors = (q, k, v, alpha, mu, beta, eta, S0, M0, O, S_T, M_T, Vt)
        self.workspace = workspace
        self.outputs = (O, S_T, M_T, Vt)
        self._ptrs = [_ptr(t) for t in self.tensors]
        self._ws = (_ptr(workspace) if workspace is not None else None,
                    workspace.numel() if workspace is not None else 0)

    def run(self, stream=None):
        _check(lib().mdn_chunk_fwd_varlen(*self.sizes, _ptr(self.cu), *self.dims, *self._ptrs, *self._ws,
                                          _stream(stream, self._owned)), "mdn_chunk_fwd_varlen")
        return self.outputs


def chunk_fwd_varlen(q, k, v, alpha, mu, beta, eta, cu_seqlens, S0=None, M0=None, C=64, *,
                     out=None, S_T=None, M_T=None, workspace=None, stream=None):
    """Packed variable-length forward: returns (O, S_T, M_T, Vtilde).

    q, k: [H,T,dk]; v: [H,T,dv] (bf16 or fp32); gates [H,T] fp32, where T is
    the packed length; cu_seqlens: int32 [nseq+1] on the GPU, sequence i being
    tokens [cu_seqlens[i], cu_seqlens[i+1]) (cu_seqlens[0] = 0, nondecreasing,
    cu_seqlens[-1] = T); S0, M0 [nseq,H,dk,dv] fp32 or None.  O, Vtilde are
    [H,T,dv]; S_T, M_T [nseq,H,dk,dv].
    """
    call = VarlenCall(q, k, v, alpha, mu, beta, eta, cu_seqlens, S0, M0, C, out=out, S_T=S_T,
                      M_T=M_T, workspace=workspace)
    return call.run(stream)


def step(q, k, v, alpha, mu, beta, eta, S, M, *, o=None, stream=None):
    """One decode step; S and M ([B,H,dk,dv] fp32) are updated in place.
    q, k: [B,H,dk]; v: [B,H,dv]; gates [B,H].  Returns o [B,H,dv]."""
    torch = _torch()
    B, H, dk = q.shape
    dv = v.shape[-1]
    dt = _dtype_code(q)
    dev = q.device
    _need(k, "k", q.dtype, (B, H, dk), dev)
    _need(v, "v", q.dtype, (B, H, dv), dev)
    for name, g in (("alpha", alpha), ("mu", mu), ("beta", beta), ("eta", eta)):
        _need(g, name, torch.float32, (B, H), dev)
    _need(S, "S", torch.float32, (B, H, dk, dv), dev)
    _need(M, "M", torch.float32, (B, H, dk, dv), dev)
    owned = ()
    if o is None:
        o = torch.empty((B, H, dv), dtype=q.dtype, device=dev)
        owned = (o,)
    st = lib().mdn_step(B, H, dk, dv, dt, _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(mu),
                        _ptr(beta), _ptr(eta), _ptr(S), _ptr(M), _ptr(o), _stream(stream, owned))
    _check(st, "mdn_step")
    return o


def stream_rw(buf, scale=1.0, *, stream=None):
    """Measurement reference for the decode step: every fp32 of the
    contiguous device tensor ``buf`` is read and written back times
    ``scale``, in place, with the step's access pattern (``mdn_stream_rw``)."""
    if not buf.is_contiguous():
        raise ValueError("buf must be contiguous")
    _check(lib().mdn_stream_rw(_ptr(buf), buf.numel() * buf.element_size(), float(scale), _stream(stream)),
           "mdn_stream_rw")
    return buf


def chunk_coef(alpha, mu, beta, eta, C, *, with_gamma=True, stream=None):
    """The log-domain coefficient stage alone (diagnostic).

    Returns (coef [B,H,NT,8,C], gamma [B,H,NT,C,C] or None); coefficient rows
    are named in ``COEF_NAMES``."""
    torch = _torch()
    B, H, T = alpha.shape
    dev = alpha.device
    for name, g in (("alpha", alpha), ("mu", mu), ("beta", beta), ("eta", eta)):
        _need(g, name, torch.float32, (B, H, T), dev)
    NT = (T + C - 1) // C
    coef = torch.empty((B, H, NT, COEF_ROWS, C), dtype=torch.float32, device=dev)
    gamma = torch.empty((B, H, NT, C, C), dtype=torch.float32, device=dev) if with_gamma else None
    st = lib().mdn_chunk_coef(B, H, T, C, _ptr(alpha), _ptr(mu), _ptr(beta), _ptr(eta),
                              _ptr(coef), _ptr(gamma), _stream(stream, (coef, gamma)))
    _check(st, "mdn_chunk_coef")
    return coef, gamma


def gates(x, a, b, mu_log, *, s=1.0, mu_log_min=-2.0, q=None, k=None, d=None, q_out=None,
          out=None, stream=None):
    """Gate pre-operation: (alpha, mu, beta, eta) from the projection outputs
    x, a, b, mu_log ([B,H,T] fp32).  With q, k ([B,H,T,dk], bf16 or fp32) and
    d ([H] fp32) also the query correction q - d k, returned as a fifth
    tensor (``q_out`` may be given, and may be ``q`` itself).  ``out`` may be
    a tuple of four preallocated [B,H,T] fp32 tensors."""
    torch = _torch()
    B, H, T = x.shape
    dev = x.device
    for name, t in (("x", x), ("a", a), ("b", b), ("mu_log", mu_log)):
        _need(t, name, torch.float32, (B, H, T), dev)
    corr = q is not None or k is not None or d is not None
    owned = []
    dk, dt = 16, MDN_F32
    if corr:
        if q is None or k is None or d is None:
            raise ValueError("the query correction needs q, k and d")
        dk = q.shape[-1]
        dt = _dtype_code(q)
        _need(q, "q", q.dtype, (B, H, T, dk), dev)
        _need(k, "k", q.dtype, (B, H, T, dk), dev)
        _need(d, "d", torch.float32, (H,), dev)
        if q_out is None:
            q_out = torch.empty_like(q)
            owned.append(q_out)
        _need(q_out, "q_out", q.dtype, (B, H, T, dk), dev)
    if out is None:
        out = tuple(torch.empty((B, H, T), dtype=torch.float32, device=dev) for _ in range(4))
        owned += list(out)
    for name, t in zip(("alpha", "mu", "beta", "eta"), out):
        _need(t, name, torch.float32, (B, H, T), dev)
    _check(lib().mdn_gates(B, H, T, dk, dt, float(s), float(mu_log_min),
                           _ptr(x), _ptr(a), _ptr(b), _ptr(mu_log), *[_ptr(t) for t in out],
                           _ptr(q), _ptr(k), _ptr(d), _ptr(q_out), _stream(stream, owned)), "mdn_gates")
    return (*out, q_out) if corr else tuple(out)
