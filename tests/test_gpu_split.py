"""GPU parity of mdn_chunk_fwd_split (the forward with each sequence cut into
segments that run side by side) against the fp64 oracle, whole tensors."""
import numpy as np
import pytest

import oracle
from linear_attention_sequence_mdn_amd import inputs
from tests.gpu_util import TOL, dev, host, note, rel_err, run_chunk, torch_mod

pytestmark = pytest.mark.gpu

NAMES = ("O", "S_T", "M_T", "Vtilde")


def run_split(x, nseg, ws_fill=None):
    import linear_attention_sequence_mdn_amd as mdn
    torch = torch_mod()
    args = [dev(x.q, x.dtype), dev(x.k, x.dtype), dev(x.v, x.dtype), dev(x.alpha), dev(x.mu),
            dev(x.beta), dev(x.eta), None if x.S0 is None else dev(x.S0), None if x.M0 is None else dev(x.M0)]
    ws = None
    if ws_fill is not None:
        dt = mdn.MDN_BF16 if x.dtype == "bf16" else mdn.MDN_F32
        n = mdn.chunk_fwd_split_workspace_bytes(x.B, x.H, x.T, x.dk, x.dv, x.C, dt, nseg)
        ws = torch.full((max(n, 1),), ws_fill, dtype=torch.uint8, device="cuda")
    out = mdn.chunk_fwd_split(*args, C=x.C, nseg=nseg, workspace=ws)
    torch.cuda.synchronize()
    return tuple(host(t) for t in out)


def oracle_of(x):
    return oracle.fwd(x.q, x.k, x.v, x.alpha, x.mu, x.beta, x.eta, x.S0, x.M0)


def check_all(got, ref, tol, label):
    errs = {n: rel_err(g, r) for n, g, r in zip(NAMES, got, ref)}
    note(f"  {label}: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    for n, e in errs.items():
        assert e <= tol, (label, n, e)


# Segment counts 2 (two passes, no combine step), 3 and more (combine steps
# in order), more segments than chunks (empty segments), ragged last chunk,
# both dtypes, every natively compiled (d, C) family, few and many heads.
CASES = [
    # dtype, B, H, T, d, C, nseg, state_std
    ("bf16", 1, 2, 64 * 9 + 17, 128, 64, 3, 0.02),
    ("bf16", 1, 1, 64 * 7, 128, 64, 2, None),
    ("bf16", 2, 2, 64 * 12, 128, 64, 5, 0.02),
    ("bf16", 1, 3, 32 * 11 + 9, 64, 32, 4, 0.02),
    ("bf16", 1, 2, 64 * 5 + 1, 64, 64, 3, None),
    ("bf16", 2, 1, 32 * 6, 32, 32, 3, 0.02),
    ("bf16", 1, 1, 100, 64, 64, 5, 0.02),          # 2 chunks, 5 segments: empty segments
    ("f32", 1, 2, 16 * 20 + 3, 16, 16, 5, 0.3),
    ("f32", 2, 1, 32 * 13 + 5, 32, 32, 4, 0.3),
    ("f32", 1, 2, 64 * 6, 128, 64, 3, 0.3),
    ("f32", 1, 1, 32 * 9, 64, 32, 3, None),
    ("f32", 1, 3, 64 * 4 + 63, 64, 64, 2, 0.3),
    ("bf16", 1, 1, 64 * 30 + 7, 128, 64, 12, 0.02),     # ten combine steps in order
    ("f32", 1, 2, 32 * 40 + 3, 32, 32, 23, 0.3),
]


@pytest.mark.parametrize("dtype,B,H,T,d,C,nseg,sd", CASES)
def test_split_small(dtype, B, H, T, d, C, nseg, sd):
    x = inputs.make_chunk_inputs(B, H, T, d, C=C, dtype=dtype, seed=T + 3 * d + nseg, state_std=sd)
    note(f"split {dtype} B{B} H{H} T{T} d{d} C{C} nseg={nseg} S0={'random' if sd else 'zero'}")
    got = run_split(x, nseg)
    check_all(got, oracle_of(x), TOL[dtype], f"split {dtype} d{d} C{C} T{T} nseg{nseg}")
    # and the plain forward on the same inputs
    check_all(got, run_chunk(x), TOL[dtype], "split vs mdn_chunk_fwd")


def long_memory(x, seed):
    """Gates that keep the state over many chunks (alpha, mu within 1% of 1,
    small beta and eta: the gate map at eta near 0, where alpha = cos^2(theta)
    sigma(a) can approach 1).  With the workloads' own gates a chunk of 64
    tokens scales the state by about e^-30, so a segment's map of the start
    state is far below fp32 resolution and a wrong map would go unseen."""
    rng = np.random.default_rng(seed)
    shp = x.alpha.shape
    x.alpha = np.exp(-rng.uniform(0.0, 0.01, shp)).astype(np.float32)
    x.mu = np.exp(-rng.uniform(0.0, 0.02, shp)).astype(np.float32)
    x.beta = rng.uniform(0.0, 0.02, shp).astype(np.float32)
    x.eta = rng.uniform(0.0, 0.2, shp).astype(np.float32)
    return x


def start_state_matters(x, nseg, tol):
    """On the CPU: the last segment's outputs from a zero start state differ
    from the true ones by far more than the tolerance, so the case checks
    the combine step (the oracle alone, no GPU result)."""
    import copy
    NT = -(-x.T // x.C)
    c0 = (nseg - 1) * NT // nseg * x.C
    ref = oracle_of(x)
    y = copy.copy(x)
    for n in ("q", "k", "v", "alpha", "mu", "beta", "eta"):
        setattr(y, n, np.ascontiguousarray(getattr(x, n)[:, :, c0:]))
    y.T = x.T - c0
    y.S0 = y.M0 = None
    cold = oracle_of(y)
    d = rel_err(cold[0], ref[0][:, :, c0:])
    note(f"    last segment from a zero state: O differs by {d:.2e} of max |O|")
    assert d > 20 * tol


@pytest.mark.parametrize("dtype,d,C,T,nseg", [("bf16", 128, 64, 64 * 12 + 5, 3), ("bf16", 64, 32, 32 * 17, 5),
                                              ("f32", 128, 64, 64 * 9, 3), ("f32", 32, 32, 32 * 14 + 7, 4),
                                              ("bf16", 128, 64, 64 * 26, 12)])
def test_split_long_memory_gates(dtype, d, C, T, nseg):
    x = long_memory(inputs.make_chunk_inputs(1, 2, T, d, C=C, dtype=dtype, seed=808 + d + nseg,
                                             state_std=0.3), 909 + T)
    note(f"split long-memory gates {dtype} d{d} C{C} T{T} nseg={nseg}")
    start_state_matters(x, nseg, TOL[dtype])
    got = run_split(x, nseg)
    check_all(got, oracle_of(x), TOL[dtype], f"split long memory {dtype} d{d} nseg{nseg}")
    check_all(run_chunk(x), oracle_of(x), TOL[dtype], "mdn_chunk_fwd long memory")


def test_split_strong_momentum_gates():
    """The long-context gate regime (log mu ~ U[-2, -1.5], alpha near its
    bound), where the segment maps carry the slowest-decaying state."""
    x = inputs.make_chunk_inputs(1, 2, 64 * 12 + 30, 128, C=64, dtype="bf16", seed=404,
                                 mu_range=(-2.0, -1.5), a_range=(5.0, 10.0), state_std=0.02)
    note("split bf16 strong-momentum gates T798 nseg=3")
    check_all(run_split(x, 3), oracle_of(x), TOL["bf16"], "split strong momentum")


def test_split_empty_sequence_copies_states():
    x = inputs.make_chunk_inputs(1, 2, 0, 64, C=64, dtype="bf16", seed=5, state_std=0.3)
    note("split T=0 nseg=3")
    got = run_split(x, 3)
    assert np.array_equal(got[1], x.S0.astype(np.float64)) and np.array_equal(got[2], x.M0.astype(np.float64))


@pytest.mark.parametrize("dtype,d,C", [("bf16", 128, 64), ("f32", 64, 32)])
def test_split_on_nan_workspace(dtype, d, C):
    """Every workspace byte starts as 0xFF: the state slots are all written
    before they are read."""
    x = inputs.make_chunk_inputs(1, 2, 7 * C + 3, d, C=C, dtype=dtype, seed=606 + d, state_std=0.02)
    note(f"split nan workspace {dtype} d{d} C{C} nseg=4")
    check_all(run_split(x, 4, ws_fill=0xFF), oracle_of(x), TOL[dtype], f"split nan-ws {dtype}")


def test_split_in_place_states():
    """S_T, M_T given as S0, M0 (the in-place update): the first pass reads the
    start state before the second pass writes the end state."""
    import linear_attention_sequence_mdn_amd as mdn
    torch = torch_mod()
    x = long_memory(inputs.make_chunk_inputs(1, 2, 64 * 10 + 3, 128, C=64, dtype="bf16", seed=515,
                                             state_std=0.3), 516)
    note("split in-place states bf16 T643 nseg=4")
    args = [dev(x.q, "bf16"), dev(x.k, "bf16"), dev(x.v, "bf16"), dev(x.alpha), dev(x.mu), dev(x.beta), dev(x.eta)]
    S, M = dev(x.S0), dev(x.M0)
    O, ST, MT, Vt = mdn.chunk_fwd_split(*args, S, M, C=64, nseg=4, S_T=S, M_T=M)
    torch.cuda.synchronize()
    assert ST.data_ptr() == S.data_ptr() and MT.data_ptr() == M.data_ptr()
    check_all((host(O), host(S), host(M), host(Vt)), oracle_of(x), TOL["bf16"], "split in place")


def test_split_deterministic():
    x = inputs.make_chunk_inputs(1, 2, 64 * 10, 128, C=64, dtype="bf16", seed=707, state_std=0.02)
    a, b = run_split(x, 3), run_split(x, 3)
    for n, u, v in zip(NAMES, a, b):
        assert np.array_equal(u, v), n


def test_split_long_context_full_size():
    """The long-context workload (B1 H16 T16384 d128 C64 bf16) in three
    segments, every head against the oracle, whole tensors."""
    x = inputs.config_inputs(4)
    note(f"split nseg=3 on {inputs.CONFIG_NAMES[4]}")
    got = run_split(x, 3)
    ref = oracle_of(x)
    check_all(got, ref, TOL["bf16"], "long context split, all 16 heads")
    for n, g, r in zip(NAMES, got, ref):
        per = np.abs(g - r).reshape(x.B * x.H, -1).max(axis=1) / np.abs(r).max()
        note(f"    {n}: worst head {int(per.argmax())} err {per.max():.2e}, median head {np.median(per):.2e}")


def auto_segments(BH, T, cus, d=128):
    """The segment count mdn_chunk_fwd takes for bf16, C = 64, d in {64, 128}
    (0: the single pass): the largest P whose first pass, 1 + 3 (P - 2) units
    of d / 32 workgroups per head, fits the compute units in one round, with
    at least 32 chunks per segment (64 where the three-segment first pass
    fills more than half of the device), at most 12, and at least 3."""
    w = d // 32
    units = cus // (w * BH)
    P = (units - 1) // 3 + 2 if units >= 1 else 0
    floor_chunks = 64 if 2 * 4 * w * BH > cus else 32
    P = min(P, (-(-T // 64)) // floor_chunks, 12)
    return P if P >= 3 else 0


@pytest.mark.parametrize("B,H,T,d", [(1, 16, 16384, 128), (1, 4, 32768, 128), (1, 16, 8192, 128),
                                     (1, 16, 8192, 64), (1, 32, 8192, 64)])
def test_forward_takes_the_split_on_few_long_heads(B, H, T, d):
    """mdn_chunk_fwd with the workspace its query returns takes the sequence
    split where the rule above chooses it: bit for bit the outputs of
    mdn_chunk_fwd_split with that segment count (and the single pass where it
    chooses none: the query then returns the single pass's size)."""
    import linear_attention_sequence_mdn_amd as mdn
    torch = torch_mod()
    x = inputs.config_inputs(4) if (B, H, T, d) == (1, 16, 16384, 128) else \
        inputs.make_chunk_inputs(B, H, T, d, C=64, dtype="bf16", seed=T + H + d)
    args = [dev(x.q, "bf16"), dev(x.k, "bf16"), dev(x.v, "bf16"), dev(x.alpha), dev(x.mu), dev(x.beta),
            dev(x.eta), None, None]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    P = auto_segments(B * H, T, cus, d)
    n_auto = mdn.chunk_fwd_workspace_bytes(B, H, T, d, d, 64, mdn.MDN_BF16)
    note(f"B{B} H{H} T{T} d{d}: {cus} compute units, rule: {P or 'single pass'}; workspace query {n_auto} bytes")
    if P == 0:
        single = 2 * B * H * (T // 64) * 64 * 64 * 2 + B * H * (T // 64) * 8 * 64 * 4
        assert n_auto == single
        return
    assert n_auto == mdn.chunk_fwd_split_workspace_bytes(B, H, T, d, d, 64, mdn.MDN_BF16, P)
    auto = [t.clone() for t in mdn.chunk_fwd(*args, C=64)]
    split = [t.clone() for t in mdn.chunk_fwd_split(*args, C=64, nseg=P)]
    torch.cuda.synchronize()
    for n, a, b in zip(NAMES, auto, split):
        assert torch.equal(a, b), n
