"""GPU parity of mdn_gates (gate pre-operation and query correction) against
the fp64 gate oracle."""
import numpy as np
import pytest

from oracle import gates_ref
from linear_attention_sequence_mdn_amd import inputs
from tests.gpu_util import dev, host, note, torch_mod

pytestmark = pytest.mark.gpu


def _run(x, s, lo, correction=True, in_place=False):
    import linear_attention_sequence_mdn_amd as mdn
    torch = torch_mod()
    args = [dev(t) for t in (x.x, x.a, x.b, x.mu_log)]
    kw = dict(s=s, mu_log_min=lo)
    if correction:
        q = dev(x.q, x.dtype)
        kw.update(q=q, k=dev(x.k, x.dtype), d=dev(x.d))
        if in_place:
            kw["q_out"] = q
    out = mdn.gates(*args, **kw)
    torch.cuda.synchronize()
    return [host(t) for t in out]


def _check_gates(got, x, s, lo, label):
    ref = gates_ref.gates(x.x, x.a, x.b, x.mu_log, s=s, mu_log_min=lo)
    worst = 0.0
    for name, g, r in zip(("alpha", "mu", "beta", "eta"), got, ref):
        # fp32 arithmetic: a few ulps of relative error per element
        err = float(np.max(np.abs(g - r) / np.maximum(np.abs(r), 1e-30)))
        worst = max(worst, err)
        assert err <= 2e-6, (label, name, err)
    note(f"  {label}: gates max relative error {worst:.2e}")


def _check_correction(got, x, label):
    ref = gates_ref.query_correction(x.q, x.k, x.d)
    # fp32 arithmetic (rounding of the order of 2^-24 of the operands), then
    # for bf16 one rounding to nearest of the result (half an ulp, 2^-9 of it)
    scale = np.abs(x.q) + np.abs(x.d[None, :, None, None] * x.k)
    tol = scale * 2.0 ** -22 + (np.abs(ref) * 2.0 ** -8 if x.dtype == "bf16" else 0.0)
    bad = np.abs(got - ref) > tol
    assert not bad.any(), (label, int(bad.sum()))
    note(f"  {label}: query correction max |err| {np.max(np.abs(got - ref)):.2e}")


@pytest.mark.parametrize("B,H,T,dk,dtype", [(1, 1, 1, 16, "f32"), (2, 3, 37, 16, "f32"),
                                            (1, 2, 130, 128, "bf16"), (3, 2, 7, 64, "bf16")])
def test_gates_small_ragged(B, H, T, dk, dtype):
    x = inputs.make_gate_inputs(B, H, T, dk, dtype=dtype, seed=B * 100 + T)
    got = _run(x, 1.0, -2.0)
    _check_gates(got[:4], x, 1.0, -2.0, f"B{B} H{H} T{T} d{dk} {dtype}")
    _check_correction(got[4], x, f"B{B} H{H} T{T} d{dk} {dtype}")


@pytest.mark.parametrize("s,lo", [(0.7, -1.0), (2.0, -2.5)])
def test_gates_other_scale_and_clamp(s, lo):
    x = inputs.make_gate_inputs(2, 4, 257, 32, dtype="bf16", seed=7)
    got = _run(x, s, lo, correction=False)
    assert len(got) == 4
    _check_gates(got, x, s, lo, f"s={s} clamp={lo}")


def test_gates_in_place_correction():
    x = inputs.make_gate_inputs(2, 2, 64, 128, dtype="bf16", seed=11)
    got = _run(x, 1.0, -2.0, in_place=True)
    _check_correction(got[4], x, "in place")


def test_gates_full_layer_shape():
    # the 400M-layer shape: B8 H8 T4096, dk = 128, bf16
    x = inputs.make_gate_inputs(8, 8, 4096, 128, dtype="bf16", seed=1)
    got = _run(x, 1.0, -2.0)
    _check_gates(got[:4], x, 1.0, -2.0, "B8 H8 T4096 d128 bf16")
    _check_correction(got[4], x, "B8 H8 T4096 d128 bf16")
    alpha, mu, beta, eta = got[:4]
    assert np.all(alpha + beta <= 1.0 + 1e-6)
