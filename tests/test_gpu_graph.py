"""The allocation-free chunk forward under HIP graph capture.

mdn_chunk_fwd_noalloc exists for callers that cannot allocate, code under
graph capture among them: its workspace is the library's static scratch, so
a captured call holds no allocation of its own.  The call is captured once
and replayed several times; between replays the outputs are overwritten with
NaN and an eager call on another problem reuses the scratch, with
synchronisations in between.  Every replay must reproduce the eager
mdn_chunk_fwd result bit for bit (the same kernels on the same inputs), and
that result is itself compared with the oracle."""
import numpy as np
import pytest

import oracle
from linear_attention_sequence_mdn_amd import inputs
from tests.gpu_util import TOL, dev, note, rel_err, torch_mod

pytestmark = pytest.mark.gpu

NAMES = ("O", "S_T", "M_T", "Vtilde")


def _args(x):
    S0 = None if x.S0 is None else dev(x.S0)
    M0 = None if x.M0 is None else dev(x.M0)
    return [dev(x.q, x.dtype), dev(x.k, x.dtype), dev(x.v, x.dtype), dev(x.alpha), dev(x.mu), dev(x.beta),
            dev(x.eta), S0, M0]


@pytest.mark.parametrize("dtype,d,C,T", [("bf16", 128, 64, 300), ("f32", 64, 32, 130), ("bf16", 16, 16, 70)])
def test_noalloc_forward_replays_in_a_hip_graph(dtype, d, C, T):
    import linear_attention_sequence_mdn_amd as mdn
    torch = torch_mod()
    x = inputs.make_chunk_inputs(2, 3, T, d, C=C, dtype=dtype, seed=3 * d + C + T,
                                 state_std=0.02 if dtype == "bf16" else 0.3)
    note(f"graph capture of mdn_chunk_fwd_noalloc: {dtype} d={d} C={C} T={T}")
    args = _args(x)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    O = torch.empty((x.B, x.H, x.T, x.dv), dtype=tdt, device="cuda")
    Vt = torch.empty_like(O)
    ST = torch.empty((x.B, x.H, x.dk, x.dv), dtype=torch.float32, device="cuda")
    MT = torch.empty_like(ST)
    outs = (O, ST, MT, Vt)

    ref = [t.float().cpu().numpy() for t in mdn.chunk_fwd(*args, C=C)]
    want = oracle.fwd(x.q, x.k, x.v, x.alpha, x.mu, x.beta, x.eta, x.S0, x.M0)
    for n, r, w in zip(NAMES, ref, want):
        assert rel_err(r, w) <= TOL[dtype], n

    # eager first: the scratch's device address is looked up outside capture
    mdn.chunk_fwd_noalloc(*args, C=C, out=(O, Vt), S_T=ST, M_T=MT)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        mdn.chunk_fwd_noalloc(*args, C=C, out=(O, Vt), S_T=ST, M_T=MT)
    torch.cuda.synchronize()

    other = inputs.make_chunk_inputs(1, 2, 97, d, C=C, dtype=dtype, seed=77, state_std=0.02)
    oargs = _args(other)
    oo = torch.empty((1, 2, 97, d), dtype=tdt, device="cuda")
    ost = torch.empty((1, 2, d, d), dtype=torch.float32, device="cuda")
    for replay in range(3):
        for t in outs:
            t.fill_(float("nan"))
        mdn.chunk_fwd_noalloc(*oargs, C=C, out=(oo, oo.clone()), S_T=ost, M_T=ost.clone())
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n, g, r in zip(NAMES, outs, ref):
            gh = g.float().cpu().numpy()
            assert np.array_equal(gh, r), (replay, n, rel_err(gh, r))
        note(f"  replay {replay}: every output identical to the eager call")
