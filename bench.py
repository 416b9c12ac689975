"""Benchmark of the MDN hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

A *step* is one ``mdn_chunk_fwd`` call (coefficients + intra-chunk kernel,
then the inter-chunk kernel: the whole chunkwise forward) over one batch of
the 400M-layer workload: B=8, H=8, T=4096, dk=dv=128, C=64, bf16 q/k/v,
fp32 gates, zero initial state.  Inputs are synthetic (seeded generator) and
resident in HBM before the timed region.  W untimed warm-up steps, then K
steps timed with HIP events on the stream the kernels run on, bracketed by
device synchronisation.  Before the warm-up steps of each timed section the
device is held for ``--settle-ms`` (200 ms) under a neutral load (a bf16
matrix product from torch, not the measured path): from idle the clocks ramp
up over tens of milliseconds, and a few warm-up steps alone would time the
ramp.  ``value`` = B*T / time per step (tokens/s).  Each
kernel's average launch duration comes from K back-to-back launches of its
stage entry point, timed the same way right after.

The same run also reports, each measured live with HIP events:
  * the median of the K per-call durations;
  * per-kernel average durations (K launches of each stage) and the roofline
    of the dominant kernel: the path's algorithmic bytes (q, k, v, gates, O
    and vtilde per token-head, the states per head) over that kernel's
    average launch duration, against the HBM peak; the same over the whole
    call; and how much more the kernels move (their own algorithmic bytes,
    and the counted traffic from the committed counter summaries when they
    match the sources);
  * the decode workload (B=256, H=16, d=128, 128 consecutive ``mdn_step``
    calls, median of 5 repetitions) as GB/s of algorithmic HBM traffic,
    beside an in-place read-write stream over the same bytes;
  * the gate pre-operation with the query correction (``mdn_gates``) on the
    400M-layer shape, as GB/s of algorithmic HBM traffic;
  * a packed prefill batch (``mdn_chunk_fwd_varlen``): 32768 tokens of 8
    heads in sequences of lengths ~U{1..4096}, as tokens/s;
  * the backward (``mdn_chunk_bwd``) on the 400M-layer workload, as tokens/s;
  * the fp64 CPU oracle on a bounded sample of the chunk workload, with all of
    the host's threads and with one.
Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MDN chunk-fwd tokens/s at 400M layer shape (% bf16 MFMA peak); decode GB/s"
PEAK_BF16_TFLOPS = 2500.0        # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0            # MI355X HBM3E
# FLOP per token*head of the whole chunk forward (d = 128, C = 64), counting
# only the causal triangles: 12 d^2 + 6 C d + (2/3) C^2.
F_TOKEN_HEAD = 248_491
F_TOKEN_HEAD_FULL = 297_643       # the same work counting full C x C tiles


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-decode", action="store_true")
    p.add_argument("--no-gates", action="store_true")
    p.add_argument("--no-varlen", action="store_true")
    p.add_argument("--no-bwd", action="store_true")
    p.add_argument("--no-chunk", action="store_true")
    p.add_argument("--settle-ms", type=float, default=200.0,
                   help="device settling before each section's warm-up: ms of in-place stream load (0 = none)")
    p.add_argument("--settle-kind", choices=("gemm", "stream"), default="gemm")
    p.add_argument("--sustained-ms", type=float, default=150.0,
                   help="after the chunk section, ms of back-to-back calls before the sustained-load window")
    p.add_argument("--decode-reps", type=int, default=5)
    p.add_argument("--decode-steps", type=int, default=128)
    p.add_argument("--calibration-copy", action="store_true",
                   help="run one 1 GiB device copy first (HBM counter calibration)")
    p.add_argument("--cpu-seconds", type=float, default=8.0)
    p.add_argument("--cpu-threads", type=int, default=0,
                   help="threads of the CPU-baseline oracle (0 = all the host's OpenMP threads)")
    p.add_argument("--workload", type=int, default=1, choices=(1, 2, 4),
                   help="chunk workload: 1 = 400M layer (the headline line), 2 = 1.3B layer, 4 = long context")
    return p.parse_args()


def kernel_sources_sha(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "linear_attention_sequence_mdn_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(summary, sha):
    """Counter-derived HBM bytes per launch from a committed rocprofv3 summary,
    or None when the summary is missing or was taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    m = re.search(r"^traffic_json:\s*(\{.*\})\s*$", open(path).read(), flags=re.M)
    if not m:
        return None
    d = json.loads(m.group(1))
    if d.get("source_sha") != sha:
        return None
    return d.get("traffic_bytes_per_launch")


def settle_device(args, torch, mdn):
    """Hold the device under a neutral load, not the measured path, for
    ``--settle-ms`` of wall time, so that the warm-up steps that follow start
    from running clocks rather than from the idle state: a bf16 matrix
    product of two 8192 x 8192 operands (``--settle-kind gemm``) or an
    in-place read-write stream over 256 MiB (``stream``).  Returns what was
    run."""
    if args.settle_ms <= 0:
        return None
    if args.settle_kind == "gemm":
        a = torch.ones((8192, 8192), dtype=torch.bfloat16, device="cuda")
        b = torch.ones((8192, 8192), dtype=torch.bfloat16, device="cuda")
        c = torch.empty((8192, 8192), dtype=torch.bfloat16, device="cuda")
        work, kind = (lambda: torch.mm(a, b, out=c)), "torch.mm bf16 8192 x 8192 x 8192"
    else:
        buf = torch.ones(64 * 1024 * 1024, dtype=torch.float32, device="cuda")
        work, kind = (lambda: mdn.stream_rw(buf, 1.0)), "mdn_stream_rw, 256 MiB in place"
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while (time.perf_counter() - t0) * 1e3 < args.settle_ms:
        for _ in range(4):
            work()
        torch.cuda.synchronize()
        n += 4
    return {"kind": kind, "ms": round((time.perf_counter() - t0) * 1e3, 1), "launches": n}


WORKLOAD_NAMES = {
    1: "400M-layer chunk forward B8 H8 T4096 dk=dv=128 C64 bf16, zero initial state",
    2: "1.3B-layer chunk forward B4 H16 T4096 dk=dv=128 C64 bf16, S0/M0 ~ N(0, 0.02^2)",
    4: "long-context chunk forward B1 H16 T16384 dk=dv=128 C64 bf16, log mu ~ U[-2,-1.5]",
}


def chunk_bench(args, torch, mdn, inputs):
    cfg = inputs.CONFIGS[args.workload]
    x = inputs.config_inputs(args.workload)
    B, H, T, d, C = x.B, x.H, x.T, x.dk, x.C
    to = lambda a, bf=False: (torch.from_numpy(np.ascontiguousarray(a)).cuda().to(torch.bfloat16)
                              if bf else torch.from_numpy(np.ascontiguousarray(a)).cuda())
    q, k, v = to(x.q, True), to(x.k, True), to(x.v, True)
    gates = [to(x.alpha), to(x.mu), to(x.beta), to(x.eta)]
    S0 = None if x.S0 is None else to(x.S0)
    M0 = None if x.M0 is None else to(x.M0)
    call = mdn.ChunkCall(q, k, v, *gates, S0, M0, C)
    torch.cuda.synchronize()

    settle = settle_device(args, torch, mdn)
    for _ in range(args.warmup):
        call.run()
    torch.cuda.synchronize()

    def timed(fn, per_call=False):
        """Average duration (ms) of K back-to-back launches of fn, HIP events
        on the stream the kernels run on (torch's current stream); with
        per_call, also the median of the K per-call durations (an event
        between consecutive calls)."""
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1 if per_call else 2)]
        torch.cuda.synchronize()
        ev[0].record()
        for i in range(args.steps):
            fn()
            if per_call:
                ev[i + 1].record()
        ev[-1].record()
        torch.cuda.synchronize()
        avg = ev[0].elapsed_time(ev[-1]) / args.steps
        if not per_call:
            return avg
        return avg, float(np.median([ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)]))

    # the timed region: K whole steps (plain mdn_chunk_fwd calls)
    ms_step, ms_call_median = timed(call.run, per_call=True)
    # each kernel's average launch duration: K launches of its stage alone
    # (repeating either stage recomputes the same result)
    ms_intra = timed(call.intra)
    ms_inter = timed(call.inter)

    O, ST, MT, Vt = call.outputs
    finite = bool(torch.isfinite(O.float()).all() and torch.isfinite(ST).all())

    tokens = B * T
    tok_head = B * H * T
    es = 2
    # algorithmic bytes / FLOP per launch of each kernel: what the kernel must
    # read and write (each input once, each output once) and its causal-triangle
    # matrix work
    # T and Aqk without their all-zero upper-right quadrant (C = 64 in bf16),
    # which the intra kernel does not write and the inter kernel does not read
    tq = 2 * C * es * 3 // 4 if C == 64 else 2 * C * es
    intra_bytes = tok_head * (2 * 2 * d + 16 + tq + 8 * 4)
    nstate = 2 if x.S0 is None else 4                 # S_T, M_T written (and S0, M0 read when given)
    inter_bytes = tok_head * (es * 3 * d + es * 2 * d + tq + 8 * 4) + B * H * nstate * d * d * 4
    intra_flop = tok_head * (2 * C * d + (2 * C * C) // 3)
    inter_flop = tok_head * (12 * d * d + 2 * C * d)
    kernels = {
        "mdn_intra_kernel": {"ms": ms_intra, "alg_bytes": intra_bytes, "alg_flop": intra_flop},
        "mdn_inter_kernel": {"ms": ms_inter, "alg_bytes": inter_bytes, "alg_flop": inter_flop},
    }
    for kd in kernels.values():
        s = kd["ms"] / 1e3
        kd["GBps"] = kd["alg_bytes"] / s / 1e9
        kd["TFLOPs"] = kd["alg_flop"] / s / 1e12
        t_hbm = kd["alg_bytes"] / (PEAK_HBM_GBS * 1e9)
        t_mfma = kd["alg_flop"] / (PEAK_BF16_TFLOPS * 1e12)
        kd["bound"] = "hbm" if t_hbm >= t_mfma else "mfma"
    srcs = {"mdn_intra_kernel": ["mdn_intra.hip", "mdn_lds.h", "mdn_device.h"],
            "mdn_inter_kernel": ["mdn_chunk.hip", "mdn_lds.h", "mdn_device.h"]}
    for name, kd in kernels.items():
        kd["source_sha"] = kernel_sources_sha(srcs[name])
        kd["traffic"] = (load_traffic(f"traffic_{name}_400M_layer.md", kd["source_sha"])
                         if args.workload == 1 else None)
    dom_name = max(kernels, key=lambda n: kernels[n]["ms"])
    dom = kernels[dom_name]
    tps = tokens / (ms_step / 1e3)
    mfma_frac = tps * H * F_TOKEN_HEAD / (PEAK_BF16_TFLOPS * 1e12)
    # The path's algorithmic HBM bytes: per token-head q, k, v, the four
    # gates, O and vtilde (1,296 B at d = 128 in bf16), per head the final
    # states (and the initial ones when given).  Intermediates that one
    # kernel hands to the next through HBM are not algorithmic: they are
    # reported as the workspace overhead below.
    call_bytes = tok_head * (3 * d * es + 16 + 2 * d * es) + B * H * nstate * d * d * 4
    call_flop = tok_head * F_TOKEN_HEAD
    hbm_cap = tokens / (call_bytes / (PEAK_HBM_GBS * 1e9))
    # The roofline of the dominant kernel: the path's algorithmic bytes over
    # that kernel's average launch duration.  Its intensity (FLOP per byte)
    # is below the chip's ridge, so HBM bounds it.
    bound = "hbm" if call_flop / call_bytes < PEAK_BF16_TFLOPS / PEAK_HBM_GBS else "mfma"
    achieved = call_bytes / (dom["ms"] / 1e3) / 1e9
    roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": achieved / PEAK_HBM_GBS, "traffic": dom["traffic"], "kernel": dom_name, "ms": dom["ms"],
            "alg_bytes_per_launch": call_bytes, "intensity_flop_per_byte": call_flop / call_bytes,
            "intensity_bound": bound, "source_sha": dom["source_sha"],
            "call": {"ms": ms_step, "GBps": call_bytes / (ms_step / 1e3) / 1e9,
                     "frac": call_bytes / (ms_step / 1e3) / 1e9 / PEAK_HBM_GBS}}
    # what the kernels move beyond the path's bytes: their own algorithmic
    # bytes (each input read once per kernel, the workspace they hand on)
    # and, when the committed counter summaries match the sources, the
    # counted traffic
    kern_bytes = sum(kd["alg_bytes"] for kd in kernels.values())
    roof["workspace_overhead"] = kern_bytes / call_bytes
    trs = [kd["traffic"] for kd in kernels.values()]
    roof["counted_traffic_over_alg"] = (sum(trs) / call_bytes) if all(t is not None for t in trs) else None
    # the optional single-kernel forward (mdn_chunk_fwd_fused) on the same
    # inputs, where it applies: K launches, same events and stream
    fused = None
    if x.dtype == "bf16" and C == 64 and d in (64, 128) and x.dk == x.dv:
        for _ in range(args.warmup):
            call.fused()
        ms_fused = timed(call.fused)
        fused = {"kernel": "mdn_fwd_kernel", "ms": ms_fused, "tokens_per_s": tokens / (ms_fused / 1e3),
                 "GBps": call_bytes / (ms_fused / 1e3) / 1e9,
                 "frac": call_bytes / (ms_fused / 1e3) / 1e9 / PEAK_HBM_GBS,
                 "source_sha": kernel_sources_sha(["mdn_fwd.hip", "mdn_lds.h", "mdn_device.h"]),
                 "note": "mdn_chunk_fwd_fused: the whole forward in one kernel without a workspace; "
                         "value and roofline above are for mdn_chunk_fwd"}
    # a side figure, not the value: K calls timed after --sustained-ms of
    # back-to-back calls, where the clocks have settled under this load
    sustained = None
    if args.sustained_ms > 0:
        t0 = time.perf_counter()
        while (time.perf_counter() - t0) * 1e3 < args.sustained_ms:
            for _ in range(8):
                call.run()
            torch.cuda.synchronize()
        ms_sus = timed(call.run)
        sustained = {"ms_per_call": ms_sus, "tokens_per_s": tokens / (ms_sus / 1e3),
                     "after_ms_of_calls": args.sustained_ms}
    # which forward mdn_chunk_fwd ran: with few long heads it cuts each
    # sequence into segments (mdn_chunk_fwd_split), and its workspace query
    # then returns the split's size; `kernels` above are the single pass's
    # stage entry points either way
    dt = mdn.MDN_BF16 if x.dtype == "bf16" else mdn.MDN_F32
    n_ws = mdn.chunk_fwd_workspace_bytes(B, H, T, d, d, C, dt)
    path = {"kind": "single pass", "segments": 1}
    if x.dk == x.dv:
        for nseg in range(3, 65):
            try:
                if n_ws == mdn.chunk_fwd_split_workspace_bytes(B, H, T, d, d, C, dt, nseg):
                    path = {"kind": "sequence split", "segments": nseg,
                            "single_pass_stages_ms": ms_intra + ms_inter}
                    break
            except mdn.MdnError:
                break
    return dict(ms_step=ms_step, ms_call_median=ms_call_median, tokens_per_s=tps, mfma_frac=mfma_frac,
                kernels=kernels, roofline=roof, finite=finite, x=x, cfg=cfg, call=call, call_bytes=call_bytes,
                hbm_cap=hbm_cap, fused=fused, settle=settle, sustained=sustained, path=path)


def decode_bench(args, torch, mdn, inputs):
    c = inputs.CONFIGS[3]
    B, H, d, n = c["B"], c["H"], c["dk"], args.decode_steps
    qs, ks, vs, gs = [], [], [], []
    for st in inputs.decode_steps(B, H, d, steps=n, dtype="bf16", seed=c["seed"]):
        qs.append(st.q); ks.append(st.k); vs.append(st.v)
        gs.append(np.stack([st.alpha, st.mu, st.beta, st.eta]))
    bf = lambda a: torch.from_numpy(np.stack(a)).cuda().to(torch.bfloat16)
    Q, K, V = bf(qs), bf(ks), bf(vs)
    G = torch.from_numpy(np.stack(gs)).cuda()          # [n, 4, B, H]
    S = torch.zeros((B, H, d, d), dtype=torch.float32, device="cuda")
    M = torch.zeros_like(S)
    o = torch.empty((n, B, H, d), dtype=torch.bfloat16, device="cuda")
    L = mdn.lib()
    import ctypes
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    argv = [(P(Q[i]), P(K[i]), P(V[i]), P(G[i, 0]), P(G[i, 1]), P(G[i, 2]), P(G[i, 3]), P(S), P(M), P(o[i]))
            for i in range(n)]

    def run_all():
        for a in argv:
            st = L.mdn_step(B, H, d, d, mdn.MDN_BF16, *a, stream)
            if st != 0:
                raise mdn.MdnError(st, "mdn_step")

    settle_device(args, torch, mdn)
    run_all()                                           # warm-up pass
    times = []
    for _ in range(args.decode_reps):
        S.zero_(); M.zero_()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        run_all()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = float(np.median(times))
    bytes_step = B * H * (16 * d * d + 2 * (2 * d + d) + 16 + 2 * d)
    gbs = n * bytes_step / (ms / 1e3) / 1e9
    # The attainable-bandwidth reference: the library's in-place stream over
    # a buffer of the states' size (read, scale by 1, write back, with the
    # step's non-temporal 16-byte accesses), 128 passes timed the same way.
    buf = torch.ones(2 * B * H * d * d, dtype=torch.float32, device="cuda")
    mdn.stream_rw(buf, 1.0)
    torch.cuda.synchronize()
    rw_times = []
    for _ in range(args.decode_reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            mdn.stream_rw(buf, 1.0)
        e1.record()
        torch.cuda.synchronize()
        rw_times.append(e0.elapsed_time(e1))
    rw_gbs = n * 2 * buf.numel() * 4 / (float(np.median(rw_times)) / 1e3) / 1e9
    del buf
    sha = kernel_sources_sha(["mdn_step.hip", "mdn_device.h"])
    traffic = load_traffic("traffic_mdn_step_kernel_decode.md", sha)
    return {"metric": "decode GB/s", "value": gbs, "unit": "GB/s",
            "workload": f"decode B{B} H{H} d{d} bf16, {n} consecutive mdn_step calls",
            "ms_per_decode_step": ms / n, "reps": args.decode_reps,
            "alg_bytes_per_step": bytes_step, "stream_rw_GBps": rw_gbs, "frac_of_stream_rw": gbs / rw_gbs,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gbs / PEAK_HBM_GBS, "traffic": traffic, "kernel": "mdn_step_kernel",
                         "source_sha": sha}}


# algorithmic FLOP per token-head of the backward at d = 128, C = 64: the
# state products of the reverse carry (12 d^2) and of the per-chunk state
# gradients (12 d^2), the replay's state update (4 d^2), the in-chunk
# products (about 12 C d over the causal halves) and the recomputed intra
# stage (2 C d + 2 C^2 / 3)
def bwd_flop_per_token_head(d, C):
    return 28 * d * d + 12 * C * d + 2 * C * d + (2 * C * C) // 3


def bwd_bench(args, torch, mdn, inputs, ch):
    """The backward (``mdn_chunk_bwd``) on the 400M-layer workload, from the
    forward's vtilde with a seeded bf16 dL/dO: tokens/s of whole calls."""
    x = ch["x"]
    call = ch["call"]
    q, k, v, alpha, mu, beta, eta, S0, M0 = call.tensors[:9]
    O, ST, MT, Vt = call.run()
    rng = np.random.default_rng(901)
    dO = torch.from_numpy(rng.standard_normal(O.shape).astype(np.float32)).cuda().to(torch.bfloat16)
    bc = mdn.BwdCall(q, k, alpha, mu, beta, eta, Vt, dO, S0, M0, None, None, x.C)
    settle_device(args, torch, mdn)
    for _ in range(args.warmup):
        bc.run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        bc.run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    tokens = x.B * x.T
    f = bwd_flop_per_token_head(x.dk, x.C)
    tflops = tokens * x.H * f / (ms / 1e3) / 1e12
    finite = all(bool(torch.isfinite(t.float()).all()) for t in bc.grads.values())
    return {"metric": "backward tokens/s", "value": tokens / (ms / 1e3), "unit": "tokens/s", "ms_per_call": ms,
            "workload": WORKLOAD_NAMES[1] + ", dL/dO ~ N(0,1) bf16, dL/dS_T = dL/dM_T = 0",
            "flop_per_token_head": f, "TFLOPs": tflops, "mfma_frac_of_bf16_peak": tflops / PEAK_BF16_TFLOPS,
            "grads_finite": finite}


def varlen_bench(args, torch, mdn, inputs):
    """Packed prefill batch (``mdn_chunk_fwd_varlen``): 8 heads, d = 128,
    C = 64, bf16, sequences with lengths ~ U{1..4096} packed to 32768 tokens
    (the token count of the 400M-layer step), zero initial states.  Tokens/s
    of the whole call (slot table, intra and inter kernels)."""
    H, d, C, total = 8, 128, 64, 32768
    lengths = inputs.serving_lengths(total, 1, 4096, seed=11)
    x = inputs.make_varlen_inputs(H, lengths, d, C=C, dtype="bf16", seed=11)
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    q, k, v = to(x.q).to(torch.bfloat16), to(x.k).to(torch.bfloat16), to(x.v).to(torch.bfloat16)
    call = mdn.VarlenCall(q, k, v, to(x.alpha), to(x.mu), to(x.beta), to(x.eta), to(x.cu), None, None, C)
    settle_device(args, torch, mdn)
    for _ in range(args.warmup):
        call.run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        call.run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    return {"metric": "packed prefill tokens/s", "value": total / (ms / 1e3), "unit": "tokens/s",
            "ms_per_call": ms, "workload": f"packed prefill H{H} d{d} C{C} bf16, {len(lengths)} sequences "
            f"with lengths ~U{{1..4096}} (seed 11) packed to {total} tokens, zero initial states",
            "nseq": int(len(lengths)), "max_len": int(lengths.max()),
            "fixed_layout_equivalent": "400M-layer step: the same token count in 8 sequences of 4096"}


def gates_bench(args, torch, mdn, inputs):
    """Gate pre-operation with the query correction on the 400M-layer shape
    (B8 H8 T4096, dk = 128, bf16): GB/s of algorithmic traffic."""
    B, H, T, d = 8, 8, 4096, 128
    g = inputs.make_gate_inputs(B, H, T, d, dtype="bf16", seed=1)
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    x, a, b, ml, dd = f(g.x), f(g.a), f(g.b), f(g.mu_log), f(g.d)
    q, k = f(g.q).to(torch.bfloat16), f(g.k).to(torch.bfloat16)
    outs = tuple(torch.empty((B, H, T), dtype=torch.float32, device="cuda") for _ in range(4))
    qo = torch.empty_like(q)
    run = lambda: mdn.gates(x, a, b, ml, q=q, k=k, d=dd, q_out=qo, out=outs)
    settle_device(args, torch, mdn)
    for _ in range(3):
        run()
    torch.cuda.synchronize()
    reps = 50
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    # per token-head: four fp32 inputs and four fp32 outputs, q and k read, q' written
    bytes_call = B * H * T * (8 * 4 + 3 * d * 2)
    gbs = bytes_call / (ms / 1e3) / 1e9
    sha = kernel_sources_sha(["mdn_gates.hip"])
    traffic = load_traffic("traffic_mdn_gates_kernel_gates_400M_layer.md", sha)
    return {"metric": "gate pre-op GB/s", "value": gbs, "unit": "GB/s",
            "workload": f"gates + query correction B{B} H{H} T{T} d{d} bf16", "ms_per_call": ms,
            "alg_bytes_per_call": bytes_call, "source_sha": sha,
            "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": gbs / PEAK_HBM_GBS, "traffic": traffic, "kernel": "mdn_gates_kernel"}}


def cpu_baseline(args, x):
    """The fp64 oracle, untuned, on the chunk workload, with all of the
    host's threads (or ``--cpu-threads``) and with one thread: each on the
    whole workload when that takes less than ``--cpu-seconds`` (repeated to
    fill that time, median reported), else on a prefix of the sequence on
    all heads."""
    import oracle
    full = oracle.threads()
    res = _cpu_baseline_at(args, x, oracle, args.cpu_threads if args.cpu_threads > 0 else full)
    res["one_core"] = _cpu_baseline_at(args, x, oracle, 1)
    oracle.set_threads(full)
    return res


def _cpu_baseline_at(args, x, oracle, threads):
    oracle.set_threads(threads)

    def run(Ts):
        sl = lambda a: np.ascontiguousarray(a[:, :, :Ts])
        t0 = time.perf_counter()
        oracle.fwd(sl(x.q), sl(x.k), sl(x.v), sl(x.alpha), sl(x.mu), sl(x.beta), sl(x.eta))
        return time.perf_counter() - t0

    t_probe = run(64)
    Ts = int(min(x.T, max(64, 64 * args.cpu_seconds / max(t_probe, 1e-3))))
    Ts = max(64, Ts // 64 * 64)
    walls = [run(Ts)]
    reps = int(min(20, max(1, args.cpu_seconds // max(walls[0], 1e-3))))
    walls += [run(Ts) for _ in range(reps - 1)]
    wall = float(np.median(walls))
    return {"value": x.B * Ts / wall, "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"fp64 oracle on all B{x.B} x H{x.H} heads, tokens 0..{Ts} of {x.T}; "
                      f"median of {len(walls)} runs of {wall:.2f} s",
            "cpu": _cpu_model(), "host_threads": os.cpu_count()}


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only: the MDN hot path here runs on a single MI355X "
              f"(requested --gpus {args.gpus}, WORLD_SIZE {world}); multi-GPU sharding is a design, "
              f"not a built path.", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(1)
    import linear_attention_sequence_mdn_amd as mdn
    from linear_attention_sequence_mdn_amd import inputs
    mdn.lib()                                            # fail loudly if the library is missing

    if args.calibration_copy:
        src = torch.ones(256 * 1024 * 1024, dtype=torch.float32, device="cuda")   # 1 GiB
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    out = {"metric": METRIC, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic"}
    ch = None
    if not args.no_chunk:
        ch = chunk_bench(args, torch, mdn, inputs)
        x = ch["x"]
        out.update({"value": ch["tokens_per_s"], "ms_per_step": ch["ms_step"],
                    "ms_per_call_median": ch["ms_call_median"],
                    "config": {"workload": WORKLOAD_NAMES[args.workload], "B": x.B, "H": x.H, "T": x.T,
                               "dk": x.dk, "dv": x.dv, "C": x.C, "tokens_per_step": x.B * x.T},
                    "mfma_frac_of_bf16_peak": ch["mfma_frac"], "flop_per_token_head": F_TOKEN_HEAD,
                    "mfma_frac_full_tiles": ch["mfma_frac"] * F_TOKEN_HEAD_FULL / F_TOKEN_HEAD,
                    "call_alg_bytes": ch["call_bytes"], "hbm_capped_tokens_per_s": ch["hbm_cap"],
                    "frac_of_hbm_cap": ch["tokens_per_s"] / ch["hbm_cap"],
                    "kernels": ch["kernels"], "roofline": ch["roofline"], "outputs_finite": ch["finite"]})
        out["forward_path"] = ch["path"]
        out["settle"] = ch["settle"]
        if ch["sustained"] is not None:
            out["sustained_load"] = ch["sustained"]
        if ch["fused"] is not None:
            out["fused_forward"] = ch["fused"]
    if not args.no_decode:
        out["decode"] = decode_bench(args, torch, mdn, inputs)
    if not args.no_gates:
        out["gates"] = gates_bench(args, torch, mdn, inputs)
    if not args.no_varlen:
        out["varlen"] = varlen_bench(args, torch, mdn, inputs)
    if ch is not None and not args.no_bwd and args.workload == 1:
        out["bwd"] = bwd_bench(args, torch, mdn, inputs, ch)
    if ch is not None and not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args, ch["x"])
    try:
        out["gpu"] = torch.cuda.get_device_name(0)
    except Exception:
        pass
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
