"""Benchmark of the DeltaLog decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1] [--rotate R] ...

One "step" is one DeltaLog decode step (dl_decode_step: one launch of the
step kernel, which also folds the log into the base on every M-th step) for
all B*H slot-heads of one state, with its inputs already resident in HBM.
The timed steps are replayed from a HIP graph of whole merge cycles, as a
decode loop runs on the GPU; the same steps as direct launches are reported
beside them.
The default workload is GDN B=64 H=32 d_k=d_v=128 M=8 with bf16 q/k/v and an
fp32 state.  With --rotate R (default 4) the steps go round R independent
states, as the layers of a model do, so the 512 MiB working set exceeds the
256 MB Infinity Cache and the state streams from HBM as in serving; the
single-state figure (cache-resident) is reported beside it.

Prints ONE JSON line with the throughput in (token*head)/s, the roofline of
the step kernel (algorithmic bytes per launch / mean launch time measured
with HIP events on the replay stream), the direct-launch, same-GPU eager,
two-stage and per-slot figures, the other operators' workloads, and the fp64
CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "state-update (token·head)/s + achieved HBM GB/s vs peak, GDN B=64 H=32 d=128"
PEAK_HBM_GBS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "recurrent_state_update_amd", "csrc", "dl_kernels.h")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "step_kernel_traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# --------------------------------------------------------------- byte model --
def _sizes(w):
    es = 2 if w.dtype == "bf16" else 4
    delta = w.op != "rwkv6"
    return dict(P=4 * w.dk * w.dv, es=es, delta=delta, bsz=4 if delta else es,
                lsz=4 if w.op == "gdn" else 4 * w.dk)


def step_launch_bytes(w, n: int, merge: bool) -> int:
    """Algorithmic HBM bytes of one launch of the one-launch step kernel over
    all B*H slot-heads, n = log entries before the step.  Per slot-head:
    base read P (+ base write P on a merge); the n logged entries' a_j, Lam_j
    and b_j; q, k, v, beta, log-decay (+ u for RWKV6); o; and on append steps
    the appended a_n, Lam_n, b_n."""
    z = _sizes(w)
    dk, dv = w.dk, w.dv
    per = z["P"] + n * (dk * z["es"] + z["lsz"] + dv * z["bsz"])
    per += 2 * dk * z["es"] + dv * z["es"] + (4 if z["delta"] else 4 * dk) + z["lsz"]
    per += dv * 4
    if merge:
        per += z["P"]
    else:
        per += dk * z["es"] + z["lsz"] + dv * z["bsz"]
    return per * w.BH


def eager_launch_bytes(w) -> int:
    """Eager step: read and write the base, inputs, o."""
    z = _sizes(w)
    per = 2 * z["P"] + 2 * w.dk * z["es"] + w.dv * z["es"] + z["lsz"] + w.dv * 4
    per += 4 if z["delta"] else 4 * w.dk
    return per * w.BH


def modelled_step_bytes(w) -> float:
    """Per-step bytes of the method averaged over an M-cycle (one launch per
    step): P(1 + 1/M) + E((M-1)/M + (M-1)/2) + I per slot-head, E the bytes of
    one log entry, I the step's inputs and outputs."""
    z = _sizes(w)
    M = w.M
    E = w.dk * z["es"] + w.dv * z["bsz"] + z["lsz"]
    I = 2 * w.dk * z["es"] + w.dv * z["es"] + w.dv * 4 + z["lsz"] + (4 if z["delta"] else 4 * w.dk)
    return (z["P"] * (1 + 1 / M) + E * ((M - 1) / M + (M - 1) / 2) + I) * w.BH


# ------------------------------------------------------------------- setup --
def stage_inputs(w, pool: int, dt):
    """Pre-stage `pool` distinct steps of inputs in device memory."""
    import torch
    import synth
    t0 = time.time()
    d = synth.steps(w, 0, pool)
    out = {}
    for key, a in d.items():
        out[key] = None if a is None else torch.from_numpy(a).to("cuda").to(
            dt if key in ("q", "k", "v") else torch.float32).contiguous()
    log(f"staged {pool} steps of inputs for {w.describe()} in {time.time() - t0:.1f}s")
    return out


def make_states(w, R: int, dt):
    import torch
    import synth
    import recurrent_state_update_amd as rsu
    X0, u = synth.initial(w)
    base0 = torch.from_numpy(X0).cuda()
    u_dev = None if u is None else torch.from_numpy(u).cuda()
    sts = [rsu.DeltaLogState(w.op, w.B, w.H, w.dk, w.dv, w.M, dtype=dt, base=base0.clone(),
                             u=u_dev) for _ in range(R)]
    return sts, base0, u_dev


def _ptrs(inp, s):
    g = lambda key: None if inp[key] is None else inp[key][s].data_ptr()
    return g("q"), g("k"), g("v"), g("beta"), g("ld")


# ------------------------------------------------------------------- timing --
def run_deltalog(w, inp, sts, K: int, W: int, instrument: bool, path: str = "fused"):
    """W warm-up + K timed steps on state i % R.  Returns wall ms and, when
    instrumented, per-launch kernel ms as (ms, n, merge) for the step kernel
    plus the ReplayPrep ms (two-stage path).  The timed loop passes raw device
    addresses straight to the C ABI."""
    import torch
    import recurrent_state_update_amd as rsu
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    pool = inp["q"].shape[0]
    R = len(sts)
    ptrs = [_ptrs(inp, s) for s in range(pool)]
    outs = [torch.empty(w.B, w.H, w.dv, device="cuda") for _ in range(2)]
    optr = [o.data_ptr() for o in outs]
    hs = [st._h for st in sts]
    L = rsu._lib

    def one(i, evs=None):
        h = hs[i % R]
        q, k, v, beta, ld = ptrs[i % pool]
        if path == "fused":
            if evs is not None:
                evs[0].record(stream)
            st = L.dl_decode_step(h, q, k, v, beta, ld, optr[i % 2], sp)
            if evs is not None:
                evs[1].record(stream)
        else:
            if evs is not None:
                evs[0].record(stream)
            st = L.dl_replay_prep(h, q, k, ld, sp)
            if evs is not None:
                evs[2].record(stream)
            st = st or L.dl_append_decode(h, q, k, v, beta, optr[i % 2], sp)
            if evs is not None:
                evs[1].record(stream)
        if st != 0:
            raise RuntimeError(f"DeltaLog step failed: {rsu.dl_status_string(st)}")

    for i in range(W):
        one(i)
    nev = 3 if path != "fused" else 2
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nev)] for _ in range(K)] if instrument else None
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    ns = []
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(K):
        if instrument:
            ns.append(sts[(W + i) % R].log_len)
        one(W + i, evs[i] if instrument else None)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = t0.elapsed_time(t1)
    launches, prep = [], []
    if instrument:
        for i in range(K):
            merge = ns[i] + 1 == w.M
            if path == "fused":
                launches.append((evs[i][0].elapsed_time(evs[i][1]), ns[i], merge))
            else:
                launches.append((evs[i][2].elapsed_time(evs[i][1]), ns[i], merge))
                prep.append(evs[i][0].elapsed_time(evs[i][2]))
    return wall, launches, prep


def graph_len(period: int, pool: int, K: int) -> int:
    """Launches per captured graph: whole schedule periods that also walk the
    whole input pool when that fits K whole times, else one period."""
    import math
    full = period * pool // math.gcd(period, pool)
    return full if K % full == 0 else period


def time_graph(launch, G: int, K: int, W: int) -> float:
    """Capture launch(0..G-1) as one HIP graph and replay it ceil(W/G) times
    untimed.  Then, between two HIP events on the replay stream, replay it
    K // G times and issue the remaining K % G launches directly (continuing
    the same sequence), so that exactly K launches are timed.  Returns ms per
    launch."""
    import torch
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sp = torch.cuda.current_stream().cuda_stream
        for i in range(G):
            launch(i, sp)
    for _ in range(max(1, -(-W // G))):
        g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(K // G):
        g.replay()
    for i in range(K % G):
        launch(i, sp)
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / K


def run_graph(w, inp, sts, K: int, W: int):
    """DeltaLog steps replayed from a HIP graph: G launches (state i % R,
    inputs i % pool; whole merge cycles of every state) captured once and
    replayed, any remainder of K launched directly.  Every state starts from
    an empty log.  Returns (ms per step, mean algorithmic bytes per launch of
    the K timed steps)."""
    import recurrent_state_update_amd as rsu
    import torch
    R = len(sts)
    pool = inp["q"].shape[0]
    ptrs = [_ptrs(inp, s) for s in range(pool)]
    o = torch.empty(w.B, w.H, w.dv, device="cuda")
    for st in sts:
        st.merge()
    hs = [st._h for st in sts]

    def launch(i, sp):
        q, k, v, beta, ld = ptrs[i % pool]
        if rsu._lib.dl_decode_step(hs[i % R], q, k, v, beta, ld, o.data_ptr(), sp) != 0:
            raise RuntimeError("dl_decode_step failed")

    G = graph_len(R * w.M, pool, K)
    ms = time_graph(launch, G, K, W)
    # bytes: whole cycles at the cycle mean; the remainder launch i steps
    # state i % R at log length (i // R) mod M
    rem = K % G
    tot = (K - rem) * cycle_launch_bytes(w)
    for i in range(rem):
        n = (i // R) % w.M
        tot += step_launch_bytes(w, n, n + 1 == w.M)
    return ms, tot / K


def run_eager_graph(w, inp, bases, u_dev, K: int, W: int):
    """The eager step on R dense states, replayed from a HIP graph the same
    way.  Returns ms per step."""
    import recurrent_state_update_amd as rsu
    import torch
    R = len(bases)
    pool = inp["q"].shape[0]
    ptrs = [_ptrs(inp, s) for s in range(pool)]
    o = torch.empty(w.B, w.H, w.dv, device="cuda")
    bptr = [b.data_ptr() for b in bases]
    uptr = None if u_dev is None else u_dev.data_ptr()
    opi, dti = rsu.OPS[w.op], rsu.DTYPES[inp["q"].dtype]

    def launch(i, sp):
        q, k, v, beta, ld = ptrs[i % pool]
        if rsu._lib.dl_eager_step(opi, w.B, w.H, w.dk, w.dv, dti, bptr[i % R], q, k, v, beta, ld,
                                  uptr, o.data_ptr(), sp) != 0:
            raise RuntimeError("dl_eager_step failed")

    return time_graph(launch, graph_len(R, pool, K), K, W)


def run_per_slot(w, inp, R: int, K: int, W: int):
    """Continuous batching: R fresh states with per-slot logs, slot b admitted
    at step b % M, so in steady state every launch merges the B/M slots whose
    logs are full and appends for the rest.  Then the odd slots are released
    (half-occupied batch) and the same K launches are timed again.  Returns
    (wall ms, algorithmic bytes) of K launches, full and half occupied."""
    import torch
    import synth
    import recurrent_state_update_amd as rsu
    dt = inp["q"].dtype
    X0, u = synth.initial(w)
    u_dev = None if u is None else torch.from_numpy(u).cuda()
    sts = [rsu.DeltaLogState(w.op, w.B, w.H, w.dk, w.dv, w.M, dtype=dt,
                             base=torch.from_numpy(X0).cuda(), u=u_dev) for _ in range(R)]
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    pool = inp["q"].shape[0]
    ptrs = [_ptrs(inp, s) for s in range(pool)]
    o = torch.empty(w.B, w.H, w.dv, device="cuda")
    L = rsu._lib
    for st in sts:
        st.enable_slots()

    def one(i):
        q, k, v, beta, ld = ptrs[i % pool]
        if L.dl_decode_step(sts[i % R]._h, q, k, v, beta, ld, o.data_ptr(), sp) != 0:
            raise RuntimeError("dl_decode_step failed on a per-slot state")

    for i in range(R * w.M):            # stagger: slot b starts at step b % M
        if i % R == 0:
            for b in range(i // R, w.B, w.M):
                for st in sts:
                    st.admit(b)
        one(i)
    for i in range(W):
        one(R * w.M + i)
    ones = w.with_(B=1, H=w.H)
    nbytes = 0
    for i in range(K):
        st = sts[(R * w.M + W + i) % R]
        if i < R * w.M:                 # the schedule repeats every R*M launches
            nbytes += sum(step_launch_bytes(ones, n, n + 1 == w.M)
                          for n in (st.slot_log_len(b) for b in range(w.B)))
        one(R * w.M + W + i)
    torch.cuda.synchronize()
    cyc = min(K, R * w.M)
    nbytes = nbytes * K / cyc
    def timed():
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for i in range(K):
            one(i)
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1)

    wall = timed()
    for st in sts:  # half of the requests finish: their slots are released
        for b in range(1, w.B, 2):
            st.release(b)
    half_bytes = nbytes * (w.B // 2 + w.B % 2) / w.B  # the slots b % M are spread evenly
    for i in range(W):
        one(i)
    wall_half = timed()
    for st in sts:
        st.close()
    return wall, nbytes, wall_half, half_bytes


def run_eager(w, inp, bases, u_dev, K: int, W: int, instrument: bool):
    import torch
    import recurrent_state_update_amd as rsu
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    pool = inp["q"].shape[0]
    R = len(bases)
    o = torch.empty(w.B, w.H, w.dv, device="cuda")
    ptrs = [_ptrs(inp, s) for s in range(pool)]
    bptr = [b.data_ptr() for b in bases]
    uptr = None if u_dev is None else u_dev.data_ptr()
    opi, dti = rsu.OPS[w.op], rsu.DTYPES[inp["q"].dtype]
    f = rsu._lib.dl_eager_step

    def one(i, evs=None):
        q, k, v, beta, ld = ptrs[i % pool]
        if evs is not None:
            evs[0].record(stream)
        if f(opi, w.B, w.H, w.dk, w.dv, dti, bptr[i % R], q, k, v, beta, ld, uptr,
             o.data_ptr(), sp) != 0:
            raise RuntimeError("dl_eager_step failed")
        if evs is not None:
            evs[1].record(stream)

    for i in range(W):
        one(i)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)] if instrument else None
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(K):
        one(W + i, evs[i] if instrument else None)
    t1.record(stream)
    torch.cuda.synchronize()
    per = [evs[i][0].elapsed_time(evs[i][1]) for i in range(K)] if instrument else []
    return t0.elapsed_time(t1), per


def cpu_baseline(w, budget_s=(8.0, 5.0), pool: int = 32):
    """The fp64 oracle's eager recurrence on the host cores, over all B*H
    slot-heads of the workload: the first `pool` steps' inputs are generated
    once (not timed) and stepped through repeatedly until the time budget is
    spent, first with all OpenMP threads, then with one."""
    import synth
    from oracle import Oracle
    orc = Oracle()
    X0, u = synth.initial(w)
    uu = None if u is None else u.astype(np.float64)
    steps = []
    for s_ in range(min(pool, w.steps)):
        s = synth.step(w, s_)
        steps.append([None if s[k] is None else s[k].astype(np.float64) for k in ("q", "k", "v", "beta", "ld")])
    threads = orc.max_threads()
    out = {}
    for nthr, budget in zip((threads, 1), budget_s):
        orc.set_threads(nthr)
        X = X0.astype(np.float64)
        done, spent = 0, 0.0
        while spent < budget:
            t0 = time.perf_counter()
            orc.eager_step(w.op, X, *steps[done % len(steps)], uu)
            spent += time.perf_counter() - t0
            done += 1
        out[nthr] = (w.BH * done / spent, done, spent)
    orc.set_threads(threads)
    v, done, spent = out[threads]
    v1, done1, spent1 = out[1]
    return dict(value=round(v, 1), unit="(token·head)/s", cores=threads, nproc=os.cpu_count(),
                kind="oracle",
                sample=f"fp64 eager oracle over all {w.BH} slot-heads of {w.describe()}, cycling its "
                       f"first {len(steps)} steps' inputs: {done} steps on {threads} threads in "
                       f"{spent:.1f} s; on 1 thread {round(v1, 1)} (token·head)/s ({done1} steps in "
                       f"{spent1:.1f} s); input generation not timed")


def measured_traffic():
    """HBM bytes per launch of the step kernel from the committed rocprofv3
    counter summary, if it was taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        with open(KERNEL_SRC, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != sha:
        return None
    return t.get("hbm_bytes_per_launch")


def cycle_launch_bytes(w) -> float:
    """Mean algorithmic bytes per launch over one merge cycle (log lengths
    0..M-1, the last launch merging)."""
    return sum(step_launch_bytes(w, n, n + 1 == w.M) for n in range(w.M)) / w.M


def bench_workload(w, K, W, R, pool, with_eager=True, with_staged=True, quick=False):
    """Time workload w.  Headline: K steps replayed from a HIP graph of whole
    merge cycles (the way a decode loop runs on the GPU), timed with HIP events
    on the replay stream; K / region length is the step rate and region length
    / K the mean launch duration of the step kernel (gaps included).  Beside it:
    the same steps as K direct launches, a per-launch event-bracketed pass that
    splits append and merge launches (each bracket adds event overhead), the
    two-stage path, per-slot logs, and the eager step (graph-replayed too)."""
    import torch
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    inp = stage_inputs(w, pool, dt)
    sts, base0, u_dev = make_states(w, R, dt)
    res = {}
    gms, per_launch = run_graph(w, inp, sts, K, W)
    res["wall_ms"] = gms * K
    res["value"] = w.BH / (gms * 1e-3)
    achieved = per_launch / (gms * 1e-3) / 1e9
    res["roofline"] = dict(
        bound="hbm", achieved=round(achieved, 1), peak=PEAK_HBM_GBS, unit="GB/s",
        frac=round(achieved / PEAK_HBM_GBS, 4), traffic=None,
        kernel="step_kernel, one-launch append/merge modes (dl_decode_step)",
        avg_launch_us=round(gms * 1e3, 2), bytes_per_launch=int(per_launch))
    res["modelled_step_GBs"] = round(modelled_step_bytes(w) / (gms * 1e-3) / 1e9, 1)
    if quick:  # counter runs: the headline and the eager baseline only
        with_staged = False
    # the same steps as direct launches
    for st in sts:
        st.merge()
    wall, _, _ = run_deltalog(w, inp, sts, K, W, instrument=False, path="fused")
    # the direct loop steps state i % R from an empty log, W of them untimed
    cnt = [0] * R
    direct_tot = 0
    for i in range(W + K):
        n = cnt[i % R] % w.M
        if i >= W:
            direct_tot += step_launch_bytes(w, n, n + 1 == w.M)
        cnt[i % R] += 1
    direct_bytes = direct_tot / K
    if quick:
        launches = []
    else:
        _, launches, _ = run_deltalog(w, inp, sts, K, W, instrument=True, path="fused")
    res["direct_launch"] = dict(value=round(w.BH * K / (wall * 1e-3), 1), ms_per_step=round(wall / K, 5),
                                achieved_GBs=round(direct_bytes / (wall / K * 1e-3) / 1e9, 1))
    if launches:  # not taken in quick runs
        app = [x[0] for x in launches if not x[2]]
        mer = [x[0] for x in launches if x[2]]
        res["roofline"]["event_bracketed_us"] = dict(append=round(1e3 * sum(app) / max(len(app), 1), 2),
                                                     merge=round(1e3 * sum(mer) / max(len(mer), 1), 2))
    if R > 1 and not quick:
        one, _, _ = run_deltalog(w, inp, sts[:1], K, W, instrument=False)
        res["single_state_value"] = round(w.BH * K / (one * 1e-3), 1)
    if not quick:
        pw, pbytes, hw, hbytes = run_per_slot(w, inp, R, K, W)
        res["per_slot"] = dict(value=round(w.BH * K / (pw * 1e-3), 1), ms_per_step=round(pw / K, 5),
                               achieved_GBs=round(pbytes / (pw * 1e-3) / 1e9, 1),
                               frac=round(pbytes / (pw * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                               launch="direct",
                               half_released=dict(ms_per_step=round(hw / K, 5),
                                                  achieved_GBs=round(hbytes / (hw * 1e-3) / 1e9, 1)))
    if with_staged:
        sw, _, _ = run_deltalog(w, inp, sts, K, W, instrument=False, path="staged")
        _, sl, sp = run_deltalog(w, inp, sts, K, W, instrument=True, path="staged")
        res["two_stage"] = dict(value=round(w.BH * K / (sw * 1e-3), 1), ms_per_step=round(sw / K, 5),
                                launch="direct",
                                event_bracketed_us=dict(
                                    append_decode=round(1e3 * sum(x[0] for x in sl) / len(sl), 2),
                                    replay_prep=round(1e3 * sum(sp) / len(sp), 2)))
    if with_eager:
        bases = [base0.clone() for _ in range(R)]
        ems = run_eager_graph(w, inp, bases, u_dev, K, W)
        ew, _ = run_eager(w, inp, bases, u_dev, K, W, instrument=False)
        res["eager_same_gpu"] = dict(
            value=round(w.BH / (ems * 1e-3), 1), ms_per_step=round(ems, 5),
            achieved_GBs=round(eager_launch_bytes(w) / (ems * 1e-3) / 1e9, 1),
            deltalog_speedup=round(ems / gms, 3),
            direct_launch_ms_per_step=round(ew / K, 5),
            deltalog_speedup_direct=round(ew / wall, 3))
    for st in sts:
        st.close()
    del inp, sts
    torch.cuda.empty_cache()
    return res


def deep_rotation(w, K: int, W: int, R: int, pool: int) -> dict:
    """The headline steps over R states instead of the default 4, as a deep
    model's many layers would step them: R x (state + log) far exceeds the
    Infinity Cache, so the log entries, like the state, come from HBM.
    DeltaLog and eager, both graph-replayed, over a whole number of merge
    cycles of every state (K rounded up to a multiple of R * M), so that the
    timed launches have the same append/merge mix as the headline's."""
    import torch
    K = -(-K // (R * w.M)) * (R * w.M)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    inp = stage_inputs(w, pool, dt)
    sts, base0, u_dev = make_states(w, R, dt)
    gms, per_launch = run_graph(w, inp, sts, K, W)
    for st in sts:
        st.close()
    del sts
    bases = [base0.clone() for _ in range(R)]
    ems = run_eager_graph(w, inp, bases, u_dev, K, W)
    del bases, inp
    torch.cuda.empty_cache()
    achieved = per_launch / (gms * 1e-3) / 1e9
    return dict(rotate_states=R, steps=K, value=round(w.BH / (gms * 1e-3), 1), ms_per_step=round(gms, 5),
                achieved_GBs=round(achieved, 1), frac=round(achieved / PEAK_HBM_GBS, 4),
                eager_ms_per_step=round(ems, 5), deltalog_speedup=round(ems / gms, 3))


def pages_context(res):
    """DeltaLog's published figures (the gist.science technical summary,
    "Results"; the authors' abstract) with their hardware, as context rather
    than a target, beside this run's comparable ones: the kernel speedup over
    the eager step on this GPU, and the state-write cut from the committed
    counter summary when it was taken on the current kernel source."""
    cut = None
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        with open(KERNEL_SRC, "rb") as f:
            if t.get("kernel_source_sha256") == hashlib.sha256(f.read()).hexdigest():
                cut = round(t["eager_write_bytes_per_step"] / t["write_bytes_per_launch"], 2)
    except (OSError, ValueError, KeyError, ZeroDivisionError):
        pass
    eager = res.get("eager_same_gpu") or {}
    return {
        "pages_hardware": "NVIDIA H200 and RTX 4090",
        "pages_kernel_speedup": "up to 1.86x over the FLA decode kernel",
        "pages_state_write_cut": "up to 7.83x",
        "pages_end_to_end": "1.05-1.20x (served models, outside this path)",
        "this_run_kernel_speedup_vs_eager_same_gpu": eager.get("deltalog_speedup"),
        "this_kernel_state_write_cut_rocprof": cut,
    }


# -------------------------------------------------------------------- main --
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--workload", type=int, default=1, choices=[1, 2, 3, 4])
    ap.add_argument("--op", default=None, help="operator of workload 4 (gdn|kda)")
    ap.add_argument("--M", type=int, default=None, help="merge interval (workload 4 sweep)")
    ap.add_argument("--B", type=int, default=None, help="override the workload's batch (slots)")
    ap.add_argument("--H", type=int, default=None, help="override the workload's head count")
    ap.add_argument("--rotate", type=int, default=4, help="independent states stepped in turn")
    ap.add_argument("--pool", type=int, default=None, help="distinct input steps staged")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-others", action="store_true", help="skip the KDA / RWKV6 workloads")
    ap.add_argument("--quick", action="store_true",
                    help="the headline and the eager baseline only (for counter runs)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB, 10 times (the "
                         "reference for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the DeltaLog decode step needs no exchange between "
              "GPUs (slot-heads shard with zero communication), so there is no multi-GPU "
              "figure to take; run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    if args.calibrate_copy:
        n = args.calibrate_copy * 2**20 // 4
        src = torch.ones(n, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(10):
            dst.copy_(src)
        t1.record()
        torch.cuda.synchronize()
        ms = t0.elapsed_time(t1) / 10
        print(json.dumps({"calibrate_copy_bytes_read": n * 4, "calibrate_copy_bytes_written": n * 4,
                          "dispatches": 10, "copy_GBs_read_plus_write": round(2 * n * 4 / ms / 1e6, 1)}),
              flush=True)
        return

    if args.workload == 4:
        w = synth.sweep_workload(args.op or "gdn", args.M or 8)
    else:
        w = synth.WORKLOADS[args.workload]
        if args.M:
            w = w.with_(M=args.M)
    if args.B:
        w = w.with_(B=args.B)
    if args.H:
        w = w.with_(H=args.H)
    K, W, R = args.steps, args.warmup, args.rotate
    pool = args.pool or min(w.steps, 256 if w.B <= 128 else 64)
    res = bench_workload(w, K, W, R, pool, quick=args.quick)
    default_shape = args.workload == 1 and not args.M and not args.B and not args.H
    traffic = measured_traffic() if default_shape else None
    res["roofline"]["traffic"] = traffic
    log(f"{w.describe()}: {res['wall_ms'] / K * 1e3:.2f} us/step")

    others = {}
    if not args.no_others and default_shape:
        for wid in (2, 3):
            o = synth.WORKLOADS[wid]
            r = bench_workload(o, K, W, R, min(o.steps, 256), with_staged=False)
            others[o.op] = dict(workload=o.describe(), value=round(r["value"], 1),
                                ms_per_step=round(r["wall_ms"] / K, 5),
                                achieved_GBs=r["roofline"]["achieved"], frac=r["roofline"]["frac"],
                                eager_value=r["eager_same_gpu"]["value"],
                                deltalog_speedup=r["eager_same_gpu"]["deltalog_speedup"])
            log(f"{o.describe()}: {r['wall_ms'] / K * 1e3:.2f} us/step")

    deep = None
    if default_shape and not args.quick:
        deep = deep_rotation(w, K, W, 24, pool)
        log(f"{w.describe()} over 24 states: {deep['ms_per_step'] * 1e3:.2f} us/step")

    cpu = None
    if not args.no_cpu:
        log("timing the CPU oracle ...")
        cpu = cpu_baseline(w)

    out = {
        "metric": METRIC,
        "value": round(res["value"], 1),
        "unit": "(token·head)/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(res["wall_ms"] / K, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded PCG64; bf16 q/k/v, fp32 state, beta and log-decay)",
        "config": {"workload": f"DeltaLog {w.op.upper()} decode step, B={w.B} H={w.H} "
                               f"d_k={w.dk} d_v={w.dv} M={w.M}, {R} states stepped in turn",
                   "B": w.B, "H": w.H, "d_k": w.dk, "d_v": w.dv, "M": w.M, "op": w.op,
                   "rotate_states": R, "input_pool_steps": pool},
        "roofline": res["roofline"],
        "cpu_baseline": cpu,
        "modelled_step_GBs": res["modelled_step_GBs"],
        "single_state_value": res.get("single_state_value"),
        "direct_launch": res.get("direct_launch"),
        "per_slot": res.get("per_slot"),
        "two_stage": res.get("two_stage"),
        "eager_same_gpu": res.get("eager_same_gpu"),
        "deep_rotation": deep,
        "other_workloads": others or None,
        "pages_context": pages_context(res),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
