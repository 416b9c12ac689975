"""Properties of the seeded input generator (CPU only)."""
import numpy as np
import torch

from linear_attention_sequence_mdn_amd import inputs


def test_deterministic():
    a = inputs.make_chunk_inputs(2, 3, 40, 16, C=16, seed=9)
    b = inputs.make_chunk_inputs(2, 3, 40, 16, C=16, seed=9)
    for n in ("q", "k", "v", "alpha", "mu", "beta", "eta"):
        assert np.array_equal(getattr(a, n), getattr(b, n))


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(100000) * np.exp(rng.uniform(-20, 20, 100000))).astype(np.float32)
    ours = inputs.round_to_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(ours, ref)


def test_values_exact_in_dtype():
    x = inputs.make_chunk_inputs(1, 2, 64, 32, C=32, dtype="bf16", seed=1)
    for n in ("q", "k", "v"):
        a = getattr(x, n)
        assert np.array_equal(a, inputs.round_to_bf16(a))


def test_keys_unit_norm_before_cast():
    x = inputs.make_chunk_inputs(1, 2, 64, 32, C=32, dtype="f32", seed=1)
    n = np.linalg.norm(x.k.astype(np.float64), axis=-1)
    assert np.abs(n - 1).max() < 1e-6


def test_gate_ranges_and_stability_interval():
    # MDN summary (paper.rainbus.top), novelty point 2: the momentum system is
    # stable for -(1-a)(1-m) <= a*b*e*|k|^2 <= (1+a)(1+m); the parametrisation
    # of step 6 keeps alpha + beta <= 1 and eta in (0, 2).
    for kw in (dict(), dict(mu_range=(-2.0, -1.5), a_range=(5.0, 10.0))):
        x = inputs.make_chunk_inputs(4, 4, 4096, 16, C=64, dtype="f32", seed=2, **kw)
        a, m, b, e = (getattr(x, n).astype(np.float64) for n in ("alpha", "mu", "beta", "eta"))
        assert np.all((a > 0) & (a < 1) & (m > 0) & (m <= 1) & (b > 0) & (b < 1) & (e > 0) & (e < 2))
        assert np.all(a + b <= 1 + 1e-6)
        k2 = np.sum(x.k.astype(np.float64) ** 2, axis=-1)
        s = a * b * e * k2
        assert np.all(s >= -(1 - a) * (1 - m)) and np.all(s <= (1 + a) * (1 + m))
        lo = kw.get("mu_range", (-1.0, 0.0))
        assert np.all(np.log(m) >= lo[0] - 1e-6) and np.all(np.log(m) <= lo[1] + 1e-6)


def test_long_context_alpha_near_bound():
    x = inputs.make_chunk_inputs(1, 2, 1024, 16, C=64, dtype="f32", seed=4,
                                 mu_range=(-2.0, -1.5), a_range=(5.0, 10.0))
    amax = 1.0 / (1.0 + x.eta.astype(np.float64) ** 2)      # cos^2(arctan(eta))
    r = x.alpha / amax
    assert r.min() > 0.993 and r.max() <= 1.0 + 1e-6


def test_decode_steps_shapes():
    it = inputs.decode_steps(2, 3, 16, steps=4, dtype="bf16", seed=3)
    steps = list(it)
    assert len(steps) == 4 and steps[0].q.shape == (2, 3, 16) and steps[0].alpha.shape == (2, 3)
    assert not np.array_equal(steps[0].q, steps[1].q)
