#!/usr/bin/env python3
"""Benchmark of the GDN hot path on one MI355X.

One step = one pass over every stage of the hot path on one batch of synthetic
input, all inputs resident in HBM before timing starts:

  1. gdn_prefill_chunked      4 packed bf16 sequences of 8192/5000/1031/63 tokens,
                              Hq=16, Hv=32, dk=dv=128, chunk 64, per-sequence
                              initial states, final states written
  2. gdn_state_snapshot       of those 4 final states
  3. gdn_recurrent_step       8 ragged rows of <= 7 bf16 tokens (Hq=16, Hv=32,
                              dk=dv=128) with compact capture (capacity 7)
  4. gdn_replay_state_updates every captured record onto the pre-step states

Prefill inputs rotate over 2 copies and decode/replay states over 48 distinct
16 MB state sets so the 256 MB Infinity Cache cannot hold a step's data.
Timing: torch.cuda events around K timed steps (our kernels run on torch's
current stream) give ms_per_step and value.  A second pass over K more steps,
with every launch bracketed by the library's own HIP-event pairs on the launch
stream, gives the per-kernel durations (roofline, breakdown); those event pairs
cost ~2-3 us per launch boundary, so they are kept off the first pass.

Those pairs add ~2 us to a short launch, so the breakdown's decode, replay and
snapshot times come from back-to-back loops through the C ABI (arguments
marshalled beforehand, so the host outruns the GPU) over every state set between
one event pair; medians over 120 calls of one event pair each are reported
beside them, with the inactive-capture call (zero fill) and the fp16 Qwen-like
2048-token prefill.
The breakdown also times, outside the step, the prefix-reuse batch: 16 rows x
256 bf16 tokens continuing from one broadcast snapshot of a 4096-token prefix
(event-timed loop over two distinct resident batches), without and with the
rows' final states.  Last, untimed, one copy of a cold 256 MiB buffer serves as
the calibration of the HBM traffic counters.  Prints ONE JSON line.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN prefill tokens/s (MFMA % of peak); decode/replay state GB/s (% of HBM peak)"
PEAK_MFMA_BF16_TFLOPS = 2500.0      # MI355X dense bf16/fp16 matrix peak
PEAK_HBM_GBS = 8000.0               # MI355X HBM3E
STATE_SETS = 48
CAL_STATES = 128                    # 128 x 32 x 128 x 128 fp32 = 256 MiB calibration copy


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle CPU baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


# ----------------------------------------------------------------------------- #
# algorithmic work
# ----------------------------------------------------------------------------- #
def chunk_sizes(lengths, C):
    out = []
    for L in lengths:
        out += [C] * (L // C) + ([L % C] if L % C else [])
    return out


def prefill_flops(lengths, C, Hq, Hv, dk, dv):
    """GEMM flops of the chunked method (dense counts, triangular solve excluded)."""
    return sum(Hq * 4 * c * c * dk + Hv * (2 * c * c * dk + 4 * c * c * dv + 6 * c * dk * dv)
               for c in chunk_sizes(lengths, C))


def state_kernel_flops(lengths, C, Hv, dk, dv):
    """Flops the sequential state pass performs: K S, Q S, K^T Delta (6 c dk dv) and
    A' X, MP Delta (4 c^2 dv), per chunk per value head (dense counts)."""
    return sum(Hv * (6 * c * dk * dv + 4 * c * c * dv) for c in chunk_sizes(lengths, C))


def prep_kernel_flops(lengths, C, Hq, dk):
    """Gram products K K^T and Q K^T per chunk per key head (the inverse is excluded)."""
    return sum(Hq * 4 * c * c * dk for c in chunk_sizes(lengths, C))


def prefill_bytes(T, N, Hq, Hv, dk, dv, es):
    return T * (2 * Hq * dk * es + 2 * Hv * dv * es + 8 * Hv) + 2 * N * Hv * dk * dv * 4


def decode_bytes(lengths, counts, cap, Hq, Hv, dk, dv, es):
    R = Hv + Hq * dk + Hv * dv
    toks = sum(lengths)
    n = [min(max(c, 0), cap, L) for c, L in zip(counts, lengths)]
    state = len(lengths) * Hv * dk * dv * 4 * 2
    io = toks * (2 * Hq * dk * es + 2 * Hv * dv * es + 8 * Hv)
    return state + io + sum(n) * R * 4, n


def replay_bytes(m, Hq, Hv, dk, dv):
    R = Hv + Hq * dk + Hv * dv
    rows = sum(1 for x in m if x > 0)
    return rows * Hv * dk * dv * 4 * 2 + sum(m) * R * 4


# ----------------------------------------------------------------------------- #
# traffic from committed rocprofv3 counter summaries
# ----------------------------------------------------------------------------- #
def kernel_source_sha():
    h = hashlib.sha256()
    for f in ("gdn_prefill.hip", "gdn_recurrent.hip", "gdn_mfma.h", "gdn_device.h", "gdn_internal.h"):
        with open(os.path.join(ROOT, "gated_deltanet_03_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def committed_traffic(kernel):
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha") != kernel_source_sha():
        return None          # counters were taken on another version of the kernels
    return rec.get("bytes_per_launch")


# ----------------------------------------------------------------------------- #
# CPU baseline: the fp64 oracle on a bounded sample of the same step
# ----------------------------------------------------------------------------- #
_WORKER_CASE = None


def _warm_worker(_):
    """Worker start-up (untimed): imports and the workload's inputs, drawn from
    the same seeded generator as the GPU's, so nothing large crosses processes."""
    global _WORKER_CASE
    os.environ.setdefault("OMP_NUM_THREADS", "1")
    import gdn_inputs
    import oracle  # noqa: F401
    if _WORKER_CASE is None:
        _WORKER_CASE = gdn_inputs.make("long_varlen")
    return 0


def _oracle_head(h):
    """One (all sequences, value head h) unit of the packed prefill on the fp64
    oracle, in a worker process; returns its wall time."""
    import oracle
    c = _WORKER_CASE
    t = time.perf_counter()
    oracle.recurrent(c["q"], c["k"], c["v"], c["g"], c["beta"], c["scale"], c["Hq"], c["Hv"],
                     cu_seqlens=c["cu_seqlens"], initial_state=c["s0"], heads=[h])
    return time.perf_counter() - t


def _box_cpus():
    """Cores this process may use, capped at 16 (the host cores that go with one GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def cpu_baseline(pre, dec, budget_s):
    """The fp64 oracle on the host, on a bounded sample of the same step: one
    core (decode stage + as many prefill value heads as the budget allows),
    then all cores (one worker process per core, one value head each)."""
    import multiprocessing as mp
    import oracle
    t0 = time.perf_counter()
    od = oracle.recurrent(dec["q"], dec["k"], dec["v"], dec["g"], dec["beta"], dec["scale"], dec["Hq"], dec["Hv"],
                          cu_seqlens=dec["cu_seqlens"], initial_state=dec["s0"])
    buf, _ = oracle.capture(dec["k"], od["alpha"], od["delta"], dec["Hq"], dec["Hv"], dec["capacity"],
                            dec["capture_count"].numpy(), 1, cu_seqlens=dec["cu_seqlens"])
    n = [min(max(int(c), 0), dec["capacity"], L) for c, L in zip(dec["capture_count"].tolist(), dec["lengths"])]
    oracle.replay(dec["s0"], buf, n, dec["Hq"], dec["Hv"], dec["dk"], dec["dv"], dec["capacity"])
    t_dec = time.perf_counter() - t0
    # prefill on one core: whole packed workload, a subset of value heads (each head is independent)
    heads, t_pre = [], 0.0
    order = [0, 31, 8, 23, 16, 5, 27, 12, 19, 2, 29, 10, 21, 14, 25, 6]
    for h in order:
        t1 = time.perf_counter()
        oracle.recurrent(pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], pre["scale"], pre["Hq"], pre["Hv"],
                         cu_seqlens=pre["cu_seqlens"], initial_state=pre["s0"], heads=[h])
        t_pre += time.perf_counter() - t1
        heads.append(h)
        if t_pre + t_dec > budget_s:
            break
    est_step = t_pre * pre["Hv"] / len(heads) + t_dec
    tokens = pre["T"] + dec["T"]
    one = {"value": tokens / est_step, "unit": "tokens/s", "cores": 1, "kind": "oracle",
           "sample": (f"fp64 numpy oracle, single thread: the full decode+capture+replay stage "
                      f"({t_dec:.2f} s) and the full {pre['T']}-token prefill for {len(heads)} of "
                      f"{pre['Hv']} value heads ({t_pre:.2f} s), scaled to all heads; "
                      f"est. {est_step:.1f} s per step")}
    # all cores: one worker process per core, each running one value head of the
    # whole packed prefill (fresh interpreters, BLAS/OpenMP pinned to one thread)
    W = _box_cpus()
    units = [h % pre["Hv"] for h in range(W)]
    env_keys = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")
    saved = {k: os.environ.get(k) for k in env_keys}
    for k in env_keys:
        os.environ[k] = "1"
    try:
        ctx = mp.get_context("spawn")
        with ctx.Pool(W) as pool:
            pool.map(_warm_worker, range(W), chunksize=1)   # start-up, imports, inputs: untimed
            t2 = time.perf_counter()
            per_unit = pool.map(_oracle_head, units, chunksize=1)
            wall = time.perf_counter() - t2
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    est_all = wall * pre["Hv"] / len(units) + t_dec / W
    all_cores = {"value": tokens / est_all, "unit": "tokens/s", "cores": W, "kind": "oracle",
                 "sample": (f"fp64 numpy oracle, {W} worker processes of one thread: {len(units)} value heads of "
                            f"the full {pre['T']}-token prefill at once ({wall:.2f} s wall, "
                            f"{sum(per_unit) / len(per_unit):.2f} s per head), scaled to all {pre['Hv']} heads, "
                            f"plus the decode stage split over the workers; est. {est_all:.2f} s per step")}
    out = dict(all_cores)
    out["one_core"] = one
    out["cpu"] = platform.processor() or platform.machine()
    out["host_cpus"] = os.cpu_count()
    return out


# ----------------------------------------------------------------------------- #
def _prefix_batch(gdn, gi, dev, C, iters):
    """Per-call time of the prefix-reuse batch prefill (event-timed loop over two
    distinct resident batches), its MFMA fraction, and per-kernel durations."""
    import torch
    pre = gi.make("prefix_reuse", part="prefix")
    Hq, Hv, dk, dv = pre["Hq"], pre["Hv"], pre["dk"], pre["dv"]
    p = {k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in pre.items()}
    _, pfin = gdn.gdn_prefill_chunked(*[p[x][None] for x in ("q", "k", "v", "g", "beta")], scale=pre["scale"],
                                      chunk_size=C)
    snap = gdn.gdn_state_snapshot(pfin)
    bts = []
    for bi in range(2):
        bt = gi.make("prefix_reuse", part="batch", batch_index=bi)
        B = bt["num_seqs"]
        bts.append([bt[x].to(dev).reshape(B, -1, *bt[x].shape[1:]) for x in ("q", "k", "v", "g", "beta")])
    B, L = bt["num_seqs"], bt["lengths"][0]
    o = torch.empty_like(bts[0][2])
    fin = torch.empty((B, Hv, dk, dv), device=dev)
    sh = gdn.gdn_shape(B, L, Hq, Hv, dk, dv, bt["scale"], gdn.GDN_BF16)
    ws = torch.empty(gdn.gdn_prefill_workspace_bytes(sh, C, False), dtype=torch.uint8, device=dev)
    F = prefill_flops([L] * B, C, Hq, Hv, dk, dv)
    res = {"workload": f"{B} rows x {L} tokens from one broadcast snapshot of a {pre['T']}-token prefix",
           "algorithmic_gflop": F / 1e9}
    for name, finals in (("no_finals", None), ("with_finals", fin)):
        def call(i):
            gdn.gdn_prefill_chunked(*bts[i % 2], scale=bt["scale"], initial_state=snap,
                                    initial_state_batch_stride=0, chunk_size=C, o=o, final_state=finals,
                                    output_final_state=finals is not None, workspace=ws)
        for i in range(3):
            call(i)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for i in range(iters):
            call(i)
        e1.record()
        torch.cuda.synchronize()
        us = 1000.0 * e0.elapsed_time(e1) / iters
        res[name] = {"us": us, "tokens_per_s": B * L / (us * 1e-6), "tflops": F / (us * 1e-6) / 1e12,
                     "mfma_frac": F / (us * 1e-6) / 1e12 / PEAK_MFMA_BF16_TFLOPS}
    gdn.gdn_profile_collect()
    gdn.gdn_profile_enable(True)
    for i in range(iters):
        gdn.gdn_prefill_chunked(*bts[i % 2], scale=bt["scale"], initial_state=snap, initial_state_batch_stride=0,
                                chunk_size=C, o=o, final_state=None, output_final_state=False, workspace=ws)
    torch.cuda.synchronize()
    gdn.gdn_profile_enable(False)
    res["kernels_no_finals"] = {k: {"avg_us": 1000.0 * ms / n} for k, (n, ms) in gdn.gdn_profile_collect().items()}
    return res


MEDIAN_CALLS = 120


def loop_us(fn, n):
    """Mean time per call of n calls back to back (one event pair)."""
    import torch
    for i in range(4):
        fn(i)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(n):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return 1000.0 * e0.elapsed_time(e1) / n


def median_call_us(fn, n, warm=10):
    """Median over n calls of one event pair per call (after warm-ups)."""
    import statistics
    import torch
    for i in range(warm):
        fn(i)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(ev):
        a.record()
        fn(warm + i)
        b.record()
    torch.cuda.synchronize()
    return statistics.median(1000.0 * a.elapsed_time(b) for a, b in ev)


def _qwen_prefill(gdn, gi, dev, torch):
    """The fp16 Qwen-like prefill (1 sequence of 2048 tokens, Hq=2, Hv=6,
    dk=dv=128, chunk 64, random initial state): median call time over
    MEDIAN_CALLS calls, tokens/s and the fraction of the fp16 MFMA peak."""
    c = gi.make("qwen_fp16")
    p = {k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in c.items()}
    args = [p[x][None] for x in ("q", "k", "v", "g", "beta")]
    o = torch.empty_like(args[2])
    fin = torch.empty((1, c["Hv"], c["dk"], c["dv"]), device=dev)
    sh = gdn.gdn_shape(1, c["T"], c["Hq"], c["Hv"], c["dk"], c["dv"], c["scale"], gdn.GDN_F16)
    ws = torch.empty(gdn.gdn_prefill_workspace_bytes(sh, c["chunk"], False), dtype=torch.uint8, device=dev)

    def call(i):
        gdn.gdn_prefill_chunked(*args, scale=c["scale"], initial_state=p["s0"], chunk_size=c["chunk"], o=o,
                                final_state=fin, workspace=ws)
    us = median_call_us(call, MEDIAN_CALLS)
    F = prefill_flops([c["T"]], c["chunk"], c["Hq"], c["Hv"], c["dk"], c["dv"])
    return {"workload": "fp16 prefill, 1 sequence x 2048 tokens, Hq=2, Hv=6, dk=dv=128, chunk 64, random initial "
                        "state, final state written", "us_median": us, "tokens_per_s": c["T"] / (us * 1e-6),
            "algorithmic_gflop": F / 1e9, "tflops": F / (us * 1e-6) / 1e12,
            "mfma_frac": F / (us * 1e-6) / 1e12 / PEAK_MFMA_BF16_TFLOPS,
            "note": "latency bound: 32 chunks in sequence over 6 value heads (24 workgroups)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on exactly one GPU (no multi-GPU path); --gpus must be 1",
                          "requested_gpus": args.gpus}))
        sys.exit(2)
    import torch
    import gated_deltanet_03_amd as gdn
    import gdn_inputs as gi

    gdn.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    pre = gi.make("long_varlen")
    dec = gi.make("spec_decode")
    Hq, Hv, dk, dv, C = pre["Hq"], pre["Hv"], pre["dk"], pre["dv"], pre["chunk"]
    es = 2
    N = pre["num_seqs"]

    # ---- resident device buffers (allocated before timing) --------------------
    def devcopy(c):
        return {k: (v.to(dev) if torch.is_tensor(v) else v) for k, v in c.items()}
    pre_sets = [devcopy(pre) for _ in range(2)]
    outs = [torch.empty_like(p["v"]) for p in pre_sets]
    fins = [torch.empty((N, Hv, dk, dv), device=dev) for _ in range(2)]
    snaps = [torch.empty_like(f) for f in fins]
    sh = gdn.gdn_shape(N, pre["T"], Hq, Hv, dk, dv, pre["scale"], gdn.GDN_BF16)
    ws = torch.empty(gdn.gdn_prefill_workspace_bytes(sh, C, True), dtype=torch.uint8, device=dev)

    # counter calibration source (256 MiB), allocated now so it is cold by the end
    cal_src = torch.zeros((CAL_STATES, Hv, dk, dv), device=dev)

    d = devcopy(dec)
    B, cap = dec["num_seqs"], dec["capacity"]
    states = [d["s0"].clone() for _ in range(STATE_SETS)]
    finals = [torch.empty_like(d["s0"]) for _ in range(STATE_SETS)]
    R = Hv + Hq * dk + Hv * dv
    su = torch.empty((B, cap, R), device=dev)
    dec_o = torch.empty_like(d["v"])
    counts = d["capture_count"]
    dbytes, n_cap = decode_bytes(dec["lengths"], dec["capture_count"].tolist(), cap, Hq, Hv, dk, dv, es)
    accept = torch.tensor(n_cap, dtype=torch.int32, device=dev)      # accept every captured token
    rbytes = replay_bytes(n_cap, Hq, Hv, dk, dv)

    def step(i):
        p = pre_sets[i % 2]
        gdn.gdn_prefill_chunked(p["q"], p["k"], p["v"], p["g"], p["beta"], scale=p["scale"],
                                initial_state=p["s0"], cu_seqlens=p["cu_seqlens"], chunk_size=C,
                                o=outs[i % 2], final_state=fins[i % 2], workspace=ws)
        gdn.gdn_state_snapshot(fins[i % 2], snaps[i % 2])
        j = i % STATE_SETS
        gdn.gdn_recurrent_step(d["q"], d["k"], d["v"], d["g"], d["beta"], scale=d["scale"],
                               initial_state=states[j], cu_seqlens=d["cu_seqlens"], o=dec_o,
                               final_state=finals[j], state_update_capacity=cap, capture_count=counts,
                               state_update_active=1, state_update=su)
        gdn.gdn_replay_state_updates(states[j], su, accept, Hq=Hq)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # Timed region 1: K plain steps -> ms_per_step and value.  The per-launch
    # event pairs of the library's profiler add ~2-3 us per launch boundary, so
    # they stay off this region.
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    for i in range(args.steps):
        step(args.warmup + i)
    ev1.record()
    torch.cuda.synchronize()
    total_ms = ev0.elapsed_time(ev1)
    ms_step = total_ms / args.steps

    # Timed region 2: the same K steps with every launch bracketed by HIP events
    # on its own stream -> per-kernel durations (roofline and breakdown).
    gdn.gdn_profile_collect()          # drop anything recorded before
    gdn.gdn_profile_enable(True)
    ep0, ep1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ep0.record()
    for i in range(args.steps):
        step(args.warmup + args.steps + i)
    ep1.record()
    torch.cuda.synchronize()
    gdn.gdn_profile_enable(False)
    prof = gdn.gdn_profile_collect()
    ms_step_profiled = ep0.elapsed_time(ep1) / args.steps

    # Timed region 3 (reported in the breakdown only): the prefix-reuse batch,
    # 16 rows x 256 tokens continuing from one broadcast snapshot of a
    # 4096-token prefix, without and with the rows' final states.
    batch = _prefix_batch(gdn, gi, dev, C, args.steps)

    # Timed region 4 (breakdown): the short launches through the C ABI with
    # their arguments marshalled beforehand, so the host issues them faster than
    # the GPU runs them: (a) back to back, one event pair around a loop over
    # every state set (each call's state cold); (b) one event pair per call over
    # MEDIAN_CALLS calls after 10 warm-ups, median reported.
    lib = gdn.load_library()
    vp = ctypes.c_void_p
    P = lambda t: vp(t.data_ptr())
    stream = vp(torch.cuda.current_stream(dev).cuda_stream)
    dsh = gdn.gdn_shape(B, dec["T"], Hq, Hv, dk, dv, dec["scale"], gdn.GDN_BF16)
    dargs = [(ctypes.byref(dsh), P(d["q"]), P(d["k"]), P(d["v"]), P(d["g"]), P(d["beta"]), P(states[j]),
              Hv * dk * dv, P(d["cu_seqlens"]), P(dec_o), P(finals[j])) for j in range(STATE_SETS)]
    cnt_p, su_p, acc_p = P(counts), P(su), P(accept)

    def dec_call(i, active=1):
        st = lib.gdn_recurrent_step(*dargs[i % STATE_SETS], cap, cnt_p, active, su_p, stream)
        assert st == 0, st

    def rep_call(i):
        st = lib.gdn_replay_state_updates(B, Hq, Hv, dk, dv, cap, su_p, acc_p, P(states[i % STATE_SETS]), stream)
        assert st == 0, st

    snap_args = [(P(fins[j]), P(snaps[j]), N, Hv, dk, dv, stream) for j in range(2)]

    def snap_call(i):
        assert lib.gdn_state_snapshot(*snap_args[i % 2]) == 0

    loop = {"decode": loop_us(dec_call, 2 * STATE_SETS),
            "decode_inactive": loop_us(lambda i: dec_call(i, 0), 2 * STATE_SETS),
            "replay": loop_us(rep_call, 2 * STATE_SETS),
            "snapshot": loop_us(snap_call, 2 * STATE_SETS)}
    med = {"decode": median_call_us(dec_call, MEDIAN_CALLS), "decode_inactive": median_call_us(lambda i: dec_call(i, 0), MEDIAN_CALLS),
           "replay": median_call_us(rep_call, MEDIAN_CALLS), "snapshot": median_call_us(snap_call, MEDIAN_CALLS)}
    # the replays above keep applying records to the rotating state sets; they
    # only serve timing (values grow but stay finite over these few calls)

    # Timed region 5 (breakdown): the two prefill workloads, median over
    # MEDIAN_CALLS calls of one event pair each: the step's packed prefill and
    # the fp16 Qwen-like single sequence (2048 tokens, Hq=2, Hv=6).
    def pre_call(i):
        p = pre_sets[i % 2]
        gdn.gdn_prefill_chunked(p["q"], p["k"], p["v"], p["g"], p["beta"], scale=p["scale"],
                                initial_state=p["s0"], cu_seqlens=p["cu_seqlens"], chunk_size=C,
                                o=outs[i % 2], final_state=fins[i % 2], workspace=ws)
    med["prefill"] = median_call_us(pre_call, MEDIAN_CALLS)
    qwen = _qwen_prefill(gdn, gi, dev, torch)

    # Untimed: one plain copy of a cold 256 MiB buffer (the largest copy_kernel
    # dispatch of the command), whose FETCH_SIZE / WRITE_SIZE readings calibrate
    # the HBM traffic counters of the other kernels.
    gdn.gdn_state_snapshot(cal_src)
    torch.cuda.synchronize()
    del cal_src

    kernels = {k: {"launches": n, "avg_us": 1000.0 * ms / n} for k, (n, ms) in prof.items()}
    per_step_us = {k: 1000.0 * ms / args.steps for k, (n, ms) in prof.items()}

    F = prefill_flops(pre["lengths"], C, Hq, Hv, dk, dv)
    Fstate = state_kernel_flops(pre["lengths"], C, Hv, dk, dv)
    Fprep = prep_kernel_flops(pre["lengths"], C, Hq, dk)
    pbytes = prefill_bytes(pre["T"], N, Hq, Hv, dk, dv, es)
    t_prefill_us = sum(per_step_us.get(k, 0.0) for k in ("chunk_plan_kernel", "chunk_prep_kernel",
                                                          "chunk_state_kernel"))
    # short launches: back-to-back loop times (region 4); the per-launch event
    # pairs of region 2 are reported beside them
    t_dec_us, t_rep_us, t_snap_us = loop["decode"], loop["replay"], loop["snapshot"]
    ev_us = {k: per_step_us.get(n, float("nan")) for k, n in (("decode", "recurrent_step_kernel"),
                                                              ("replay", "replay_kernel"),
                                                              ("snapshot", "copy_kernel"))}
    R = Hv + Hq * dk + Hv * dv
    dbytes_inactive = dbytes - sum(n_cap) * R * 4 + B * cap * R * 4   # no records, the whole buffer zeroed

    breakdown = {
        "prefill": {"us": t_prefill_us, "us_median": med["prefill"], "median_calls": MEDIAN_CALLS,
                    "tokens_per_s": pre["T"] / (t_prefill_us * 1e-6),
                    "algorithmic_gflop": F / 1e9, "tflops": F / (t_prefill_us * 1e-6) / 1e12,
                    "mfma_frac": F / (t_prefill_us * 1e-6) / 1e12 / PEAK_MFMA_BF16_TFLOPS,
                    "mfma_frac_median": F / (med["prefill"] * 1e-6) / 1e12 / PEAK_MFMA_BF16_TFLOPS,
                    "algorithmic_mb": pbytes / 1e6,
                    "hbm_frac": pbytes / (t_prefill_us * 1e-6) / 1e9 / PEAK_HBM_GBS},
        "decode": {"us": t_dec_us, "us_median": med["decode"], "us_event_pairs": ev_us["decode"], "tokens": dec["T"],
                   "algorithmic_mb": dbytes / 1e6,
                   "gbs": dbytes / (t_dec_us * 1e-6) / 1e9,
                   "hbm_frac": dbytes / (t_dec_us * 1e-6) / 1e9 / PEAK_HBM_GBS},
        "decode_inactive_capture": {"us": loop["decode_inactive"], "us_median": med["decode_inactive"],
                                    "note": "state_update_active=0: zero-fill of the whole capture buffer + the step",
                                    "algorithmic_mb": dbytes_inactive / 1e6,
                                    "gbs": dbytes_inactive / (loop["decode_inactive"] * 1e-6) / 1e9,
                                    "hbm_frac": dbytes_inactive / (loop["decode_inactive"] * 1e-6) / 1e9 / PEAK_HBM_GBS},
        "replay": {"us": t_rep_us, "us_median": med["replay"], "us_event_pairs": ev_us["replay"],
                   "records": sum(n_cap), "algorithmic_mb": rbytes / 1e6,
                   "gbs": rbytes / (t_rep_us * 1e-6) / 1e9,
                   "hbm_frac": rbytes / (t_rep_us * 1e-6) / 1e9 / PEAK_HBM_GBS},
        "snapshot": {"us": t_snap_us, "us_median": med["snapshot"], "us_event_pairs": ev_us["snapshot"],
                     "gbs": 2 * N * Hv * dk * dv * 4 / (t_snap_us * 1e-6) / 1e9},
        "qwen_fp16_prefill": qwen,
        "prefix_batch": batch,
        "timing": ("us: mean of back-to-back calls through the C ABI over rotating cold state sets (decode, "
                   "replay, snapshot) or the step's per-kernel event pairs (prefill); us_median: median over "
                   f"{MEDIAN_CALLS} calls of one event pair each, after 10 warm-ups"),
    }

    # dominant kernel: the one with the largest time per step
    dom = max(per_step_us, key=per_step_us.get)
    avg_s = kernels[dom]["avg_us"] * 1e-6
    if dom == "chunk_state_kernel":
        achieved, peak, unit, bound = Fstate / avg_s / 1e12, PEAK_MFMA_BF16_TFLOPS, "TFLOP/s", "mfma"
    elif dom == "chunk_prep_kernel":
        achieved, peak, unit, bound = Fprep / avg_s / 1e12, PEAK_MFMA_BF16_TFLOPS, "TFLOP/s", "mfma"
    elif dom == "recurrent_step_kernel":
        achieved, peak, unit, bound = dbytes / avg_s / 1e9, PEAK_HBM_GBS, "GB/s", "hbm"
    elif dom == "replay_kernel":
        achieved, peak, unit, bound = rbytes / avg_s / 1e9, PEAK_HBM_GBS, "GB/s", "hbm"
    else:
        achieved, peak, unit, bound = float("nan"), PEAK_HBM_GBS, "GB/s", "hbm"
    roofline = {"kernel": dom, "bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
                "frac": achieved / peak, "traffic": committed_traffic(dom),
                "avg_launch_us": kernels[dom]["avg_us"]}

    tokens = pre["T"] + dec["T"]
    out = {
        "metric": METRIC, "value": tokens / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": ("GDN hot path step: packed bf16 prefill 8192+5000+1031+63 tokens "
                                "(Hq=16, Hv=32, dk=dv=128, chunk 64, initial+final states) + snapshot of "
                                "the final states + ragged decode of 8 rows x <=7 tokens with capture "
                                "(capacity 7) + replay of the captured prefix"),
                   "prefill_tokens": pre["T"], "decode_tokens": dec["T"], "decode_lengths": dec["lengths"],
                   "capture_counts": n_cap, "state_sets_rotated": STATE_SETS},
        "roofline": roofline,
        "breakdown": breakdown,
        "kernels": kernels,
        "ms_per_step_with_kernel_events": ms_step_profiled,
        "kernel_source_sha": kernel_source_sha(),
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(pre, dec, args.cpu_seconds)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
