"""The allocation-free chunk forward (mdn_chunk_fwd_noalloc) against
mdn_chunk_fwd, through the C ABI: the same inputs must give the same outputs
(both run the same kernels; the first with the library's static scratch as
workspace, the second with a workspace the binding allocates).  Two calls in
a row, the second with a smaller problem, so that the second runs on the
scratch the first left behind."""
import numpy as np
import pytest

from linear_attention_sequence_mdn_amd import inputs
from tests.gpu_util import TOL, dev, note, rel_err, torch_mod

pytestmark = pytest.mark.gpu

NAMES = ("O", "S_T", "M_T", "Vtilde")


def _args(x):
    S0 = None if x.S0 is None else dev(x.S0)
    M0 = None if x.M0 is None else dev(x.M0)
    return [dev(x.q, x.dtype), dev(x.k, x.dtype), dev(x.v, x.dtype), dev(x.alpha), dev(x.mu), dev(x.beta),
            dev(x.eta), S0, M0]


def _outputs(x, torch):
    tdt = torch.bfloat16 if x.dtype == "bf16" else torch.float32
    nan = lambda shape, dt: torch.full(shape, float("nan"), dtype=dt, device="cuda")
    return ((nan((x.B, x.H, x.T, x.dv), tdt), nan((x.B, x.H, x.T, x.dv), tdt)),
            nan((x.B, x.H, x.dk, x.dv), torch.float32), nan((x.B, x.H, x.dk, x.dv), torch.float32))


def test_noalloc_matches_chunk_fwd_on_two_calls():
    import linear_attention_sequence_mdn_amd as mdn
    torch = torch_mod()
    cases = [("400M-layer shape B8 H8 T4096 d128 C64 bf16 (4096 chunk tiles)", inputs.config_inputs(1)),
             ("smaller: B1 H3 T130 d64 C32 bf16, random S0 M0",
              inputs.make_chunk_inputs(1, 3, 130, 64, C=32, dtype="bf16", seed=12, state_std=0.02))]
    for label, x in cases:
        note(f"noalloc vs chunk_fwd: {label}")
        need = mdn.chunk_fwd_workspace_bytes(x.B, x.H, x.T, x.dk, x.dv, x.C,
                                             mdn.MDN_BF16 if x.dtype == "bf16" else mdn.MDN_F32)
        assert need <= mdn.NOALLOC_SCRATCH_BYTES
        args = _args(x)
        (O, Vt), ST, MT = _outputs(x, torch)
        got = mdn.chunk_fwd_noalloc(*args, C=x.C, out=(O, Vt), S_T=ST, M_T=MT)
        ref = mdn.chunk_fwd(*args, C=x.C)
        torch.cuda.synchronize()
        for n, g, r in zip(NAMES, got, ref):
            gh, rh = g.float().cpu().numpy(), r.float().cpu().numpy()
            e = rel_err(gh, rh)
            note(f"  {n}: rel err {e:.1e}, identical {bool(np.array_equal(gh, rh))}")
            assert np.all(np.isfinite(gh)), n
            assert e <= TOL[x.dtype], (label, n, e)
            assert np.array_equal(gh, rh), (label, n)


def test_noalloc_rejects_a_problem_beyond_the_scratch():
    import linear_attention_sequence_mdn_amd as mdn
    torch = torch_mod()
    # 4672 chunk tiles of 18 KiB (d = 128, C = 64, bf16): more workspace than
    # the scratch holds
    B, H, T, d = 8, 8, 4672, 128
    need = mdn.chunk_fwd_workspace_bytes(B, H, T, d, d, 64, mdn.MDN_BF16)
    assert need > mdn.NOALLOC_SCRATCH_BYTES
    z = torch.zeros((B, H, T, d), dtype=torch.bfloat16, device="cuda")
    g = torch.full((B, H, T), 0.5, dtype=torch.float32, device="cuda")
    O = torch.full((B, H, T, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    ST = torch.full((B, H, d, d), float("nan"), device="cuda")
    with pytest.raises(mdn.MdnError, match="TOO_LARGE"):
        mdn.chunk_fwd_noalloc(z, z, z, g, g, g, g, None, None, C=64, out=(O, O.clone()), S_T=ST,
                              M_T=ST.clone())
    torch.cuda.synchronize()
    assert torch.isnan(O.float()).all() and torch.isnan(ST).all()   # nothing was enqueued
