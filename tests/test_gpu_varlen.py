"""GPU parity of the packed variable-length forward (mdn_chunk_fwd_varlen)
against the fp64 oracle, and its agreement with the fixed-length layout."""
import numpy as np
import pytest

import oracle
from linear_attention_sequence_mdn_amd import inputs
from tests.gpu_util import TOL, dev, host, note, rel_err, torch_mod

pytestmark = pytest.mark.gpu

NAMES = ("O", "S_T", "M_T", "Vtilde")


def check_all(got, ref, tol, label):
    errs = {n: rel_err(g, r) for n, g, r in zip(NAMES, got, ref)}
    note(f"  {label}: " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    for n, e in errs.items():
        assert e <= tol, (label, n, e)


def device_args(x):
    torch = torch_mod()
    return ([dev(x.q, x.dtype), dev(x.k, x.dtype), dev(x.v, x.dtype), dev(x.alpha), dev(x.mu),
             dev(x.beta), dev(x.eta), torch.from_numpy(x.cu).cuda()],
            [None if x.S0 is None else dev(x.S0), None if x.M0 is None else dev(x.M0)])


def run_varlen(x, **kw):
    import linear_attention_sequence_mdn_amd as mdn
    torch = torch_mod()
    a, s = device_args(x)
    out = mdn.chunk_fwd_varlen(*a, *s, C=x.C, **kw)
    torch.cuda.synchronize()
    return tuple(host(t) for t in out)


def oracle_of(x):
    return oracle.fwd_varlen(x.q, x.k, x.v, x.alpha, x.mu, x.beta, x.eta, x.cu, x.S0, x.M0)


# Length mixes: empty sequences, one token, C - 1, C, C + 1 and several
# chunks with a ragged end, packed so that sequence starts fall at every
# offset within a chunk.
CASES = [
    ("bf16", 128, 64, 3, [0, 1, 63, 64, 65, 200, 7, 130, 0, 300]),
    ("bf16", 64, 32, 2, [33, 0, 97, 32, 5]),
    ("bf16", 32, 32, 2, [31, 1, 64, 40]),
    ("f32", 16, 16, 2, [1, 15, 16, 17, 50, 0, 3]),
    ("f32", 32, 32, 2, [70, 0, 31]),
    ("f32", 128, 64, 2, [65, 130, 1]),
    ("bf16", 16, 16, 2, [1, 15, 17, 0, 40]),       # widened to the fp32 kernels
    ("bf16", 64, 16, 2, [33, 16, 2]),
]


@pytest.mark.parametrize("dtype,d,C,H,lengths", CASES)
def test_varlen_matches_oracle(dtype, d, C, H, lengths):
    x = inputs.make_varlen_inputs(H, lengths, d, C=C, dtype=dtype, seed=d + C + len(lengths),
                                  state_std=0.02 if dtype == "bf16" else 0.3)
    note(f"varlen {dtype} d={d} C={C} H={H} lengths={lengths}")
    check_all(run_varlen(x), oracle_of(x), TOL[dtype], f"varlen {dtype} d{d} C{C}")


def test_varlen_zero_state():
    x = inputs.make_varlen_inputs(2, [100, 3, 64], 128, C=64, dtype="bf16", seed=5)
    note("varlen bf16 d128 C64, S0 = M0 = NULL")
    check_all(run_varlen(x), oracle_of(x), TOL["bf16"], "varlen zero state")


def test_equal_lengths_match_fixed_layout():
    # B sequences of one length T, packed per head, give bit for bit the
    # outputs of the [B,H,T,.] layout: the same tiles and the same carry.
    import linear_attention_sequence_mdn_amd as mdn
    torch = torch_mod()
    B, H, T, d = 3, 2, 200, 128
    x = inputs.make_chunk_inputs(B, H, T, d, C=64, dtype="bf16", seed=31, state_std=0.02)
    note(f"varlen vs fixed layout: B{B} H{H} T{T} d{d} bf16")
    pack = lambda a: np.ascontiguousarray(np.swapaxes(a, 0, 1).reshape((H, B * T) + a.shape[3:]))
    fixed = mdn.chunk_fwd(dev(x.q, "bf16"), dev(x.k, "bf16"), dev(x.v, "bf16"), dev(x.alpha), dev(x.mu),
                          dev(x.beta), dev(x.eta), dev(x.S0), dev(x.M0), C=64)
    cu = torch.tensor([0, T, 2 * T, 3 * T], dtype=torch.int32, device="cuda")
    packed = mdn.chunk_fwd_varlen(dev(pack(x.q), "bf16"), dev(pack(x.k), "bf16"), dev(pack(x.v), "bf16"),
                                  dev(pack(x.alpha)), dev(pack(x.mu)), dev(pack(x.beta)), dev(pack(x.eta)),
                                  cu, dev(x.S0), dev(x.M0), C=64)
    torch.cuda.synchronize()
    unpack = lambda t: t.reshape(H, B, T, -1).transpose(0, 1)
    assert torch.equal(unpack(packed[0]), fixed[0])
    assert torch.equal(unpack(packed[3]), fixed[3])
    assert torch.equal(packed[1], fixed[1]) and torch.equal(packed[2], fixed[2])


def test_all_sequences_empty_copy_states():
    x = inputs.make_varlen_inputs(2, [0, 0, 0], 64, C=32, dtype="bf16", seed=6, state_std=0.5)
    note("varlen: three empty sequences")
    O, ST, MT, Vt = run_varlen(x)
    assert O.shape == (2, 0, 64)
    assert np.array_equal(ST, x.S0) and np.array_equal(MT, x.M0)


def test_no_sequences_is_a_no_op():
    import linear_attention_sequence_mdn_amd as mdn
    torch = torch_mod()
    q = torch.zeros((2, 0, 64), dtype=torch.bfloat16, device="cuda")
    g = torch.zeros((2, 0), device="cuda")
    cu = torch.zeros(1, dtype=torch.int32, device="cuda")
    O, ST, MT, Vt = mdn.chunk_fwd_varlen(q, q, q, g, g, g, g, cu, C=64)
    torch.cuda.synchronize()
    assert ST.shape == (0, 2, 64, 64) and O.shape == (2, 0, 64)


def test_in_place_state_update():
    import linear_attention_sequence_mdn_amd as mdn
    torch = torch_mod()
    x = inputs.make_varlen_inputs(2, [70, 0, 129], 128, C=64, dtype="bf16", seed=7, state_std=0.02)
    a, (S0, M0) = device_args(x)
    ref = run_varlen(x)
    mdn.chunk_fwd_varlen(*a, S0, M0, C=64, S_T=S0, M_T=M0)
    torch.cuda.synchronize()
    assert np.array_equal(host(S0), ref[1]) and np.array_equal(host(M0), ref[2])


def test_deterministic_and_every_output_written():
    import linear_attention_sequence_mdn_amd as mdn
    torch = torch_mod()
    x = inputs.make_varlen_inputs(4, [5, 200, 64, 1, 0, 77], 128, C=64, dtype="bf16", seed=8, state_std=0.02)
    a, s = device_args(x)
    res = []
    for _ in range(2):
        O = torch.full((4, x.T, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
        Vt = torch.full_like(O, float("nan"))
        ST = torch.full((6, 4, 128, 128), float("nan"), device="cuda")
        MT = torch.full_like(ST, float("nan"))
        mdn.chunk_fwd_varlen(*a, *s, C=64, out=(O, Vt), S_T=ST, M_T=MT)
        torch.cuda.synchronize()
        for t in (O, Vt, ST, MT):
            assert bool(torch.isfinite(t).all())
        res.append([t.clone() for t in (O, Vt, ST, MT)])
    for p, q in zip(*res):
        assert torch.equal(p, q)


def test_prefill_then_decode_steps():
    # S_T, M_T of a packed prefill feed mdn_step; the steps continue every
    # sequence as the oracle does on the unsplit sequences
    import linear_attention_sequence_mdn_amd as mdn
    torch = torch_mod()
    lengths, extra, H, d = [90, 64, 3], 4, 2, 128
    full = inputs.make_varlen_inputs(H, [n + extra for n in lengths], d, C=64, dtype="bf16", seed=9,
                                     state_std=0.02)
    ends = full.cu[1:]
    keep = np.concatenate([np.arange(a, b - extra) for a, b in zip(full.cu[:-1], ends)])
    pre = inputs.VarlenInputs(H, int(sum(lengths)), d, d, 64, "bf16", np.asarray(lengths),
                              np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32),
                              *(np.ascontiguousarray(getattr(full, n)[:, keep])
                                for n in ("q", "k", "v", "alpha", "mu", "beta", "eta")),
                              full.S0, full.M0)
    a, (S0, M0) = device_args(pre)
    _, S, M, _ = mdn.chunk_fwd_varlen(*a, S0, M0, C=64)      # [nseq, H, d, d]: the step's [B, H] layout
    ref = oracle_of(full)
    outs = []
    for j in range(extra):
        t = ends - extra + j                                  # token j of each continuation
        sel = lambda n: np.ascontiguousarray(np.swapaxes(getattr(full, n)[:, t], 0, 1))
        o = mdn.step(dev(sel("q"), "bf16"), dev(sel("k"), "bf16"), dev(sel("v"), "bf16"),
                     dev(sel("alpha")), dev(sel("mu")), dev(sel("beta")), dev(sel("eta")), S, M)
        outs.append(host(o).reshape(len(lengths), H, d))
    torch.cuda.synchronize()
    got_o = np.stack(outs, axis=2)                            # [nseq, H, extra, d]
    ref_o = np.stack([ref[0][:, e - extra:e] for e in ends])  # [nseq, H, extra, d]
    check_all((got_o, host(S), host(M), got_o),
              (ref_o, ref[1], ref[2], ref_o), TOL["bf16"], "prefill + decode")


def test_serving_mix_sampled():
    # a packed prefill batch: 32768 tokens of sequences with lengths ~ U{1..4096},
    # 8 heads of d = 128; every head of four sequences against the oracle
    lengths = inputs.serving_lengths(32768, 1, 4096, seed=11)
    x = inputs.make_varlen_inputs(8, lengths, 128, C=64, dtype="bf16", seed=11)
    note(f"varlen serving mix: {len(lengths)} sequences, T={x.T}, H=8, d=128 bf16")
    got = run_varlen(x)
    for g in got:
        assert np.all(np.isfinite(g))
    picks = sorted({0, len(lengths) // 2, len(lengths) - 1, int(np.argmax(lengths))})
    for i in picks:
        a, b = int(x.cu[i]), int(x.cu[i + 1])
        ref = oracle.fwd(x.q[:, a:b], x.k[:, a:b], x.v[:, a:b], x.alpha[:, a:b], x.mu[:, a:b],
                         x.beta[:, a:b], x.eta[:, a:b])
        check_all((got[0][:, a:b], got[1][i], got[2][i], got[3][:, a:b]), ref, TOL["bf16"],
                  f"sequence {i} (length {b - a})")


def test_slot_table_and_dispatch_order():
    # index work, compared bit for bit with the definitions in include/mdn.h:
    # sequence i owns slots [cu[i] // C + i, cu[i+1] // C + i + 1), its chunks
    # first; the order lists the sequences by length, longest first, ties by index
    import linear_attention_sequence_mdn_amd as mdn
    torch = torch_mod()
    lengths = [0, 1, 63, 64, 65, 200, 7, 130, 0, 300, 64, 1]
    H, d, C = 2, 64, 32
    x = inputs.make_varlen_inputs(H, lengths, d, C=C, dtype="bf16", seed=12)
    a, s = device_args(x)
    call = mdn.VarlenCall(*a, *s, C)
    call.run()
    torch.cuda.synchronize()
    nseq, T = len(lengths), x.T
    NT = T // C + nseq
    a256 = lambda n: (n + 255) // 256 * 256
    off = 2 * a256(H * NT * C * C * 2) + a256(H * NT * 8 * C * 4)
    ws = call.workspace.cpu().numpy()
    tab = ws[off:off + NT * 8].view(np.int32).reshape(NT, 2)
    order = ws[off + a256(NT * 8):off + a256(NT * 8) + nseq * 4].view(np.int32)
    want = np.zeros((NT, 2), dtype=np.int32)
    cu = x.cu.astype(np.int64)
    for i in range(nseq):
        base, n_chunks = cu[i] // C + i, -(-(cu[i + 1] - cu[i]) // C)
        for n in range(n_chunks):
            want[base + n] = (cu[i] + n * C, min(C, cu[i + 1] - cu[i] - n * C))
    assert np.array_equal(tab, want)
    assert np.array_equal(order, np.argsort(-np.asarray(lengths), kind="stable"))
