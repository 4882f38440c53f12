"""Benchmark of the DeltaLog decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 1] [--rotate R] ...

One bench step is one whole pass of the method's schedule over one batch:
a merge cycle of M decode steps (M-1 append launches, then the merge launch,
each a dl_decode_step over all B*H slot-heads of one state), with its inputs
already resident in HBM.  K bench steps are therefore K*M launches holding
exactly K merges, whatever K is, and the throughput counts every decode step
of every slot-head: (token*head)/s = B*H*M*K / region time.

With --rotate R (default 4) the launches go round R independent states, one
launch each in turn, as the layers of a model are stepped; the 512 MiB working
set exceeds the 256 MB Infinity Cache, so the state streams from HBM as in
serving.  A round of R*M launches is a whole merge cycle of every state; K
mod R further cycles run M launches back to back on one state.  The timed
launches are issued directly on one stream, the host running ahead of the
GPU.  Beside them: the same rounds replayed from HIP graphs (one graph per
window of the staged input pool; each replay starts with a gap of about 9 us
on this ROCm, about 0.28 us per launch), and the same direct launches timed
before the process replayed any graph (about 3% slower: direct launches on
one stream run slower until a kernel has run on a second stream, which a
graph replay does; an effect below the library).
The default workload is GDN B=64 H=32 d_k=d_v=128 M=8 with bf16 q/k/v and an
fp32 state.

Prints ONE JSON line: the throughput, the roofline of the step kernel
(algorithmic bytes per launch, averaged over the merge cycle, / mean launch
time measured with HIP events on the launch stream), the launches and merges
timed, the graph-replayed, same-GPU eager, two-stage and per-slot figures, the
cache-resident and 24-state figures, the HBM rate of the step kernel's own
access pattern on the state (pattern_ceiling: context beside the 8 TB/s peak),
the other operators' workloads, and the fp64 CPU oracle timed on a bounded
sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
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
MAX_GRAPHS = 64  # input windows captured as separate graphs (beyond that, windows repeat)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# --------------------------------------------------------------- byte model --
def _sizes(w):
    es = 2 if w.dtype == "bf16" else 4
    delta = w.op != "rwkv6"
    return dict(P=4 * w.dk * w.dv, es=es, delta=delta, bsz=4 if delta else es,
                lsz=4 if w.op == "gdn" else 4 * w.dk,
                # RWKV6's bonus u [H, d_k] fp32: one copy per head, shared by
                # the B slots, so counted once per launch (not per slot-head)
                u=0 if delta else 4 * w.H * w.dk)


def slot_head_bytes(w, n: int, merge: bool) -> int:
    """Algorithmic HBM bytes of one slot-head in one launch of the one-launch
    step kernel, n = log entries before the step: base read P (+ base write P
    on a merge); the n logged entries' a_j, Lam_j and b_j; q, k, v, beta
    (delta rule), log-decay; o; and on append steps the appended a_n, Lam_n,
    b_n."""
    z = _sizes(w)
    dk, dv = w.dk, w.dv
    per = z["P"] + n * (dk * z["es"] + z["lsz"] + dv * z["bsz"])
    per += 2 * dk * z["es"] + dv * z["es"] + (4 if z["delta"] else 0) + z["lsz"]
    per += dv * 4
    if merge:
        per += z["P"]
    else:
        per += dk * z["es"] + z["lsz"] + dv * z["bsz"]
    return per


def step_launch_bytes(w, n: int, merge: bool) -> int:
    """Algorithmic HBM bytes of one launch over all B*H slot-heads at log
    length n: slot_head_bytes for each, plus RWKV6's bonus u [H, d_k] once."""
    return slot_head_bytes(w, n, merge) * w.BH + _sizes(w)["u"]


def cycle_launch_bytes(w) -> float:
    """Mean algorithmic bytes per launch over one merge cycle (log lengths
    0..M-1, the last launch merging).  Equals the per-step traffic model
    P(1 + 1/M) + E((M-1)/M + (M-1)/2) + I per slot-head, plus u once
    (modelled_step_bytes)."""
    return sum(step_launch_bytes(w, n, n + 1 == w.M) for n in range(w.M)) / w.M


def eager_launch_bytes(w) -> int:
    """Eager step: read and write the base, inputs, o (u once per launch)."""
    z = _sizes(w)
    per = 2 * z["P"] + 2 * w.dk * z["es"] + w.dv * z["es"] + z["lsz"] + w.dv * 4
    per += 4 if z["delta"] else 0
    return per * w.BH + z["u"]


def modelled_step_bytes(w) -> float:
    """Per-step bytes of the method averaged over an M-cycle (one launch per
    step): P(1 + 1/M) + E((M-1)/M + (M-1)/2) + I per slot-head, E the bytes of
    one log entry, I the step's inputs and outputs; plus RWKV6's u once."""
    z = _sizes(w)
    M = w.M
    E = w.dk * z["es"] + w.dv * z["bsz"] + z["lsz"]
    I = 2 * w.dk * z["es"] + w.dv * z["es"] + w.dv * 4 + z["lsz"] + (4 if z["delta"] else 0)
    return (z["P"] * (1 + 1 / M) + E * ((M - 1) / M + (M - 1) / 2) + I) * w.BH + z["u"]


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


# ----------------------------------------------------------- launch order --
def launch_order(K: int, R: int, M: int) -> list:
    """State index of each of the K*M launches of K merge cycles: K // R
    rounds in which the R states take one launch each in turn (each round a
    whole merge cycle of every state), then K % R cycles of one state each, M
    launches back to back.  Every state ends where it started: log empty."""
    order = [j % R for j in range((K // R) * R * M)]
    for c in range(K % R):
        order += [c] * M
    return order


def launch_kinds(order: list, M: int) -> list:
    """Log length before each launch of `order` (all states starting empty)
    and whether the launch merges."""
    cnt = {}
    out = []
    for s in order:
        n = cnt.get(s, 0) % M
        out.append((n, n + 1 == M))
        cnt[s] = cnt.get(s, 0) + 1
    return out


def time_cycles(launch, R: int, M: int, pool: int, K: int, W: int, graphs: bool = True,
                first_input: int = 0) -> float:
    """Run W warm-up cycles (rounded up to whole rounds, and replaying every
    graph at least once), then time K merge
    cycles (K*M launches, launch_order) between two HIP events on the launch
    stream.  launch(state, input_index, stream) issues one launch; launch j of
    the sequence uses input (first_input + j) % pool.  With graphs, each round
    of R*M launches is replayed from a HIP graph captured for its window of
    inputs; the K % R trailing cycles run directly.  Returns ms per launch."""
    import torch
    RM = R * M
    nwin = pool // math.gcd(RM, pool)
    nwin = min(nwin, MAX_GRAPHS)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def direct_round(win):
        base = first_input + win * RM
        for j in range(RM):
            launch(j % R, (base + j) % pool, sp)

    gs = []
    if graphs:
        torch.cuda.synchronize()
        for win in range(nwin):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                csp = torch.cuda.current_stream().cuda_stream
                base = first_input + win * RM
                for j in range(RM):
                    launch(j % R, (base + j) % pool, csp)
            gs.append(g)

    def round_(win):
        if graphs:
            gs[win % nwin].replay()
        else:
            direct_round(win % nwin)

    # warm-up: W cycles rounded up to whole rounds, and at least one replay
    # of every graph (a graph's first replay carries one-time setup)
    warm = max(1, -(-W // R), nwin if graphs else 0)
    for r in range(warm):
        round_(r)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for r in range(K // R):
        round_(warm + r)
    j0 = first_input + (warm + K // R) * RM
    for c in range(K % R):  # trailing cycles: M launches back to back on state c
        for m in range(M):
            launch(c, (j0 + c * M + m) % pool, sp)
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / (K * M)


PREWARM_ROUNDS = 64


def prewarm(launch, R: int, M: int, pool: int, rounds: int = PREWARM_ROUNDS) -> None:
    """Untimed whole rounds of the same launch sequence before anything is
    timed (64 rounds: 2048 launches, about 60 ms, at the default workload), so
    that clocks, caches and page mappings have settled."""
    import torch
    sp = torch.cuda.current_stream().cuda_stream
    RM = R * M
    for j in range(rounds):
        for i in range(RM):
            launch(i % R, (j * RM + i) % pool, sp)
    torch.cuda.synchronize()


def time_launches_bracketed(launch, R: int, M: int, pool: int, K: int, W: int) -> list:
    """The same sequence as direct launches, each bracketed by its own pair of
    HIP events (which adds event overhead to every launch).  Returns
    [(ms, log length before, merges)] for the K*M launches."""
    import torch
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    for j in range(max(1, -(-W // R)) * R * M):
        launch(j % R, j % pool, sp)
    order = launch_order(K, R, M)
    kinds = launch_kinds(order, M)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in order]
    torch.cuda.synchronize()
    for j, s in enumerate(order):
        evs[j][0].record(stream)
        launch(s, j % pool, sp)
        evs[j][1].record(stream)
    torch.cuda.synchronize()
    return [(a.elapsed_time(b), n, mg) for (a, b), (n, mg) in zip(evs, kinds)]


# ------------------------------------------------------------------- paths --
def deltalog_launcher(w, inp, sts, o):
    import recurrent_state_update_amd as rsu
    ptrs = [_ptrs(inp, s) for s in range(inp["q"].shape[0])]
    hs = [st._h for st in sts]
    f = rsu._lib.dl_decode_step
    optr = o.data_ptr()

    def launch(state, i, sp):
        q, k, v, beta, ld = ptrs[i]
        if f(hs[state], q, k, v, beta, ld, optr, sp) != 0:
            raise RuntimeError("dl_decode_step failed")
    return launch


def staged_launcher(w, inp, sts, o):
    """The two-stage path: dl_replay_prep then dl_append_decode."""
    import recurrent_state_update_amd as rsu
    ptrs = [_ptrs(inp, s) for s in range(inp["q"].shape[0])]
    hs = [st._h for st in sts]
    L = rsu._lib
    optr = o.data_ptr()

    def launch(state, i, sp):
        q, k, v, beta, ld = ptrs[i]
        if L.dl_replay_prep(hs[state], q, k, ld, sp) != 0 or \
                L.dl_append_decode(hs[state], q, k, v, beta, optr, sp) != 0:
            raise RuntimeError("two-stage DeltaLog step failed")
    return launch


def time_staged_bracketed(w, inp, sts, o, R: int, M: int, pool: int, K: int, W: int):
    """The two-stage path as direct launches in launch_order, with events
    before ReplayPrep, between the stages and after AppendDecode.  Returns the
    mean ms of each stage (each bracket adds event overhead)."""
    import torch
    import recurrent_state_update_amd as rsu
    ptrs = [_ptrs(inp, s) for s in range(pool)]
    hs = [st._h for st in sts]
    L = rsu._lib
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    launch = staged_launcher(w, inp, sts, o)
    for j in range(max(1, -(-W // R)) * R * M):
        launch(j % R, j % pool, sp)
    order = launch_order(K, R, M)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in order]
    torch.cuda.synchronize()
    for j, s in enumerate(order):
        q, k, v, beta, ld = ptrs[j % pool]
        evs[j][0].record(stream)
        st = L.dl_replay_prep(hs[s], q, k, ld, sp)
        evs[j][1].record(stream)
        if st != 0 or L.dl_append_decode(hs[s], q, k, v, beta, o.data_ptr(), sp) != 0:
            raise RuntimeError("two-stage DeltaLog step failed")
        evs[j][2].record(stream)
    torch.cuda.synchronize()
    n = len(order)
    return (sum(e[0].elapsed_time(e[1]) for e in evs) / n, sum(e[1].elapsed_time(e[2]) for e in evs) / n)


def eager_launcher(w, inp, bases, u_dev, o):
    import recurrent_state_update_amd as rsu
    ptrs = [_ptrs(inp, s) for s in range(inp["q"].shape[0])]
    bptr = [b.data_ptr() for b in bases]
    uptr = None if u_dev is None else u_dev.data_ptr()
    opi, dti = rsu.OPS[w.op], rsu.DTYPES[inp["q"].dtype]
    f = rsu._lib.dl_eager_step
    optr = o.data_ptr()

    def launch(state, i, sp):
        q, k, v, beta, ld = ptrs[i]
        if f(opi, w.B, w.H, w.dk, w.dv, dti, bptr[state], q, k, v, beta, ld, uptr, optr, sp) != 0:
            raise RuntimeError("dl_eager_step failed")
    return launch


def run_per_slot(w, inp, R: int, K: int, W: int):
    """Continuous batching: R fresh states with per-slot logs, slot b admitted
    at step b % M, so in steady state every launch merges the slots whose logs
    are full and appends for the rest.  K*M direct launches are timed (state
    j % R in turn), then the odd slots are released (half-occupied batch) and
    the same launches are timed again.  Returns (ms, algorithmic bytes) of the
    K*M launches, full and half occupied."""
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
    o = torch.zeros(w.B, w.H, w.dv, device="cuda")
    L = rsu._lib
    RM = R * w.M
    for st in sts:
        st.enable_slots()
    pos = [0]  # launches issued so far: launch i steps state i % R with input i % pool

    def run(count, count_bytes=None):
        """Issue `count` launches; with count_bytes(b) -> bool, also sum the
        algorithmic bytes of the slots it selects from the host mirror of
        every slot's log length."""
        tot = 0
        for _ in range(count):
            i = pos[0]
            st = sts[i % R]
            if count_bytes is not None:
                ns = [st.slot_log_len(b) for b in range(w.B) if count_bytes(b)]
                tot += sum(slot_head_bytes(w, n, n + 1 == w.M) * w.H for n in ns)
                tot += _sizes(w)["u"] if ns else 0
            q, k, v, beta, ld = ptrs[i % pool]
            if L.dl_decode_step(st._h, q, k, v, beta, ld, o.data_ptr(), sp) != 0:
                raise RuntimeError("dl_decode_step failed on a per-slot state")
            pos[0] += 1
        return tot

    for i in range(RM):                 # stagger: slot b starts at step b % M
        if i % R == 0:
            for b in range(i // R, w.B, w.M):
                for st in sts:
                    st.admit(b)
        run(1)
    nl = K * w.M
    # Bytes of the timed launches: the same launches run untimed first.  The
    # schedule returns to the same phase of every slot after any multiple of
    # R*M launches, so padding to such a multiple before the timed pass makes
    # it repeat the counted launches exactly.
    nbytes = run(nl, lambda b: True)
    run((-nl) % RM + -(-(W * w.M) // RM) * RM)

    def timed():
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        run(nl)
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1)

    wall = timed()
    run((-nl) % RM)
    for st in sts:  # half of the requests finish: their slots are released
        for b in range(1, w.B, 2):
            st.release(b)
    half_bytes = run(nl, lambda b: b % 2 == 0)
    run((-nl) % RM)
    wall_half = timed()
    for st in sts:
        st.close()
    return wall, nbytes, wall_half, half_bytes


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


def _traffic_record():
    """The committed rocprofv3 counter summary, if it was taken on the current
    kernel source (else None)."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
        with open(KERNEL_SRC, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError):
        return None
    return t if t.get("kernel_source_sha256") == sha else None


def measured_traffic(op: str):
    """HBM bytes per launch of the step kernel (mean over a merge cycle) of
    the default workload of `op`, from the committed counter summary taken on
    the current kernel source; None otherwise."""
    t = _traffic_record()
    return None if t is None or op not in t else t[op].get("hbm_bytes_per_launch")


def bench_workload(w, K, W, R, pool, with_eager=True, with_staged=True, quick=False):
    """Time workload w over K merge cycles (K*M launches; launch_order).
    Headline: direct launches timed with HIP events on the launch stream;
    region length / (K*M) is the step kernel's mean launch duration (gaps
    included).  Beside it: the same launches replayed from HIP graphs, a pass
    with every launch bracketed by events (append and merge means), the
    two-stage path, per-slot logs, and the eager step over the same number of
    launches (direct and graph-replayed)."""
    import torch
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    inp = stage_inputs(w, pool, dt)
    sts, base0, u_dev = make_states(w, R, dt)
    o = torch.empty(w.B, w.H, w.dv, device="cuda")
    M = w.M
    nl = K * M
    res = {}
    launch = deltalog_launcher(w, inp, sts, o)
    prewarm(launch, R, M, pool)
    # Order of the legs: direct launches in a process that has replayed no HIP
    # graph yet (if none ran before this call), then the graph-replayed leg,
    # then the direct headline.  Direct launches on one stream were measured
    # 3% slower until a kernel has run on a second stream (a graph replay
    # does that, as does one torch op on a new stream; from the second timed
    # region after it they settle), an effect below the library whose cause
    # is not identified here.
    fresh = time_cycles(launch, R, M, pool, K, W, graphs=False)
    gms = time_cycles(launch, R, M, pool, K, W, graphs=True)
    ms = time_cycles(launch, R, M, pool, K, W, graphs=False)
    cyc_bytes = cycle_launch_bytes(w)
    res["ms_per_launch"] = ms
    res["value"] = w.BH / (ms * 1e-3)
    achieved = cyc_bytes / (ms * 1e-3) / 1e9
    res["roofline"] = dict(
        bound="hbm", achieved=round(achieved, 1), peak=PEAK_HBM_GBS, unit="GB/s",
        frac=round(achieved / PEAK_HBM_GBS, 4), traffic=None,
        kernel="step_kernel, one-launch append/merge modes (dl_decode_step)",
        avg_launch_us=round(ms * 1e3, 2), bytes_per_launch=int(round(cyc_bytes)),
        launches_timed=nl, merge_launches_timed=sum(mg for _, mg in launch_kinds(launch_order(K, R, M), M)))
    res["modelled_step_GBs"] = round(modelled_step_bytes(w) / (ms * 1e-3) / 1e9, 1)
    if quick:  # counter runs: the headline and the eager baseline only
        with_staged = False
    res["graph_replay"] = dict(value=round(w.BH / (gms * 1e-3), 1), us_per_launch=round(gms * 1e3, 3),
                               achieved_GBs=round(cyc_bytes / (gms * 1e-3) / 1e9, 1))
    res["direct_first_leg_us_per_launch"] = round(fresh * 1e3, 3)
    if not quick:
        br = time_launches_bracketed(launch, R, M, pool, K, W)
        app = [x[0] for x in br if not x[2]]
        mer = [x[0] for x in br if x[2]]
        res["roofline"]["event_bracketed_us"] = dict(append=round(1e3 * sum(app) / max(len(app), 1), 2),
                                                     merge=round(1e3 * sum(mer) / max(len(mer), 1), 2))
    if R > 1 and not quick:
        one = deltalog_launcher(w, inp, sts[:1], o)
        sms = time_cycles(one, 1, M, pool, K, W, graphs=False)
        res["single_state_value"] = round(w.BH / (sms * 1e-3), 1)
    if not quick:
        pw, pbytes, hw, hbytes = run_per_slot(w, inp, R, K, W)
        res["per_slot"] = dict(value=round(w.BH * nl / (pw * 1e-3), 1), us_per_launch=round(pw / nl * 1e3, 3),
                               achieved_GBs=round(pbytes / (pw * 1e-3) / 1e9, 1),
                               frac=round(pbytes / (pw * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                               launch="direct",
                               half_released=dict(us_per_launch=round(hw / nl * 1e3, 3),
                                                  achieved_GBs=round(hbytes / (hw * 1e-3) / 1e9, 1)))
    if with_staged:
        staged = staged_launcher(w, inp, sts, o)
        sms = time_cycles(staged, R, M, pool, K, W, graphs=False)
        prep, app = time_staged_bracketed(w, inp, sts, o, R, M, pool, K, W)
        res["two_stage"] = dict(value=round(w.BH / (sms * 1e-3), 1), us_per_step=round(sms * 1e3, 3),
                                launch="direct",
                                event_bracketed_us=dict(replay_prep=round(1e3 * prep, 2),
                                                        append_decode=round(1e3 * app, 2)))
    if with_eager:
        bases = [base0.clone() for _ in range(R)]
        el = eager_launcher(w, inp, bases, u_dev, o)
        ems = time_cycles(el, R, M, pool, K, W, graphs=False)
        egms = time_cycles(el, R, M, pool, K, W, graphs=True)
        res["eager_same_gpu"] = dict(
            value=round(w.BH / (ems * 1e-3), 1), us_per_launch=round(ems * 1e3, 3),
            achieved_GBs=round(eager_launch_bytes(w) / (ems * 1e-3) / 1e9, 1),
            deltalog_speedup=round(ems / ms, 3),
            graph_us_per_launch=round(egms * 1e3, 3),
            deltalog_speedup_graph=round(egms / gms, 3))
    for st in sts:
        st.close()
    del inp, sts
    torch.cuda.empty_cache()
    if not quick:
        res["pattern_ceiling"] = pattern_ceiling(w, R, ms)
    return res


def deep_rotation(w, K: int, W: int, R: int, pool: int) -> dict:
    """The headline launches over R states instead of the default 4, as a deep
    model's many layers would step them: R x (state + log) far exceeds the
    Infinity Cache, so the log entries, like the state, come from HBM.
    DeltaLog and eager, both launched directly, over ceil(K / R) whole rounds
    (R*M launches each, a whole merge cycle of every state)."""
    import torch
    K = -(-K // R) * R
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    inp = stage_inputs(w, pool, dt)
    sts, base0, u_dev = make_states(w, R, dt)
    o = torch.empty(w.B, w.H, w.dv, device="cuda")
    dl = deltalog_launcher(w, inp, sts, o)
    prewarm(dl, R, w.M, pool)
    ms = time_cycles(dl, R, w.M, pool, K, W, graphs=False)
    for st in sts:
        st.close()
    del sts
    bases = [base0.clone() for _ in range(R)]
    ems = time_cycles(eager_launcher(w, inp, bases, u_dev, o), R, w.M, pool, K, W, graphs=False)
    del bases, inp
    torch.cuda.empty_cache()
    achieved = cycle_launch_bytes(w) / (ms * 1e-3) / 1e9
    return dict(rotate_states=R, merge_cycles=K, launches=K * w.M, value=round(w.BH / (ms * 1e-3), 1),
                us_per_launch=round(ms * 1e3, 3), achieved_GBs=round(achieved, 1),
                frac=round(achieved / PEAK_HBM_GBS, 4), eager_us_per_launch=round(ems * 1e3, 3),
                deltalog_speedup=round(ems / ms, 3))


def pattern_cycle_writes(count: int, R: int, M: int) -> list:
    """Write flag of each pass of the pattern ceiling's merge cycles: pass i
    goes to state i % R, as launch i of launch_order does, and rewrites on the
    M-th pass of each state's cycle, where the step would merge."""
    return [int((i // R) % M == M - 1) for i in range(count)]


def pattern_ceiling(w, R: int, ms_step: float) -> dict | None:
    """The HBM rate that the step kernel's own access pattern on the state
    reaches on this GPU, as context for the roofline (whose peak stays the
    published 8 TB/s): R rotating states of the workload's shape, each launch
    a pass over every value tile in the step kernel's block order, lane layout
    and load hint (libdlceiling, csrc/dl_ceiling.hip), either a pure read (an
    append's state traffic) or an in-place read and rewrite (a merge's),
    each timed back to back on its own; then whole merge cycles of such
    passes in the benchmark's launch order (the R states in turn, every M-th
    pass of a state a rewrite), the time the state traffic alone takes in
    that pattern.  `step_vs_pattern` is the DeltaLog step's achieved rate of
    algorithmic bytes (state, log, inputs and outputs) over that cycle's rate
    of state bytes."""
    import ctypes
    import torch
    path = os.path.join(ROOT, "recurrent_state_update_amd", "libdlceiling.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built (run __graft_entry__.build())")
    lib = ctypes.CDLL(path)
    lib.dlc_sink_floats.argtypes = [ctypes.c_int] * 3
    lib.dlc_sink_floats.restype = ctypes.c_long
    lib.dlc_tile_pass.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p]
    lib.dlc_tile_pass.restype = ctypes.c_int
    nsink = lib.dlc_sink_floats(w.BH, w.dk, w.dv)
    if nsink == 0:
        return None
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    states = [torch.randn(w.BH * w.dk * w.dv, device="cuda", generator=g) for _ in range(R)]
    sink = torch.empty(nsink, device="cuda")
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    M = w.M

    def passes(kind, count):
        # kind 0: reads, 1: rewrites, 2: merge cycles (pattern_cycle_writes)
        writes = pattern_cycle_writes(count, R, M) if kind == 2 else [kind] * count
        for i in range(count):
            write = writes[i]
            if lib.dlc_tile_pass(states[i % R].data_ptr(), w.BH, w.dk, w.dv, write, sink.data_ptr(),
                                 float("nan"), sp) != 0:
                raise RuntimeError("dlc_tile_pass failed")

    def timed(kind, count):
        passes(kind, count // 4)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        passes(kind, count)
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) * 1e3 / count

    state_bytes = 4 * w.BH * w.dk * w.dv
    out = dict(rotate_states=R)
    for kind, name in ((0, "read"), (1, "read_write")):
        us = timed(kind, 64 * R)
        out[name] = dict(us_per_launch=round(us, 2), GBs=round(state_bytes * (1 + kind) / us / 1e3, 1))
    cyc_us = timed(2, 16 * R * M)
    del states, sink
    torch.cuda.empty_cache()
    pattern_gbs = state_bytes * (1 + 1 / M) / cyc_us / 1e3
    step_gbs = cycle_launch_bytes(w) / (ms_step * 1e-3) / 1e9
    out["cycle_us_per_launch"] = round(cyc_us, 2)
    out["cycle_GBs"] = round(pattern_gbs, 1)
    out["cycle_frac_of_peak"] = round(pattern_gbs / PEAK_HBM_GBS, 4)
    out["step_vs_pattern"] = round(step_gbs / pattern_gbs, 4)
    return out


def pages_context(res):
    """DeltaLog's published figures (the gist.science technical summary,
    "Results"; the authors' abstract) with their hardware, as context rather
    than a target, beside this run's comparable ones: the kernel speedup over
    the eager step on this GPU (both over whole merge cycles), and the
    state-write cut from the committed counter summary when it was taken on
    the current kernel source."""
    cut = None
    t = _traffic_record()
    if t is not None and "gdn" in t:
        cut = round(t["gdn"]["eager_write_bytes_per_step"] / t["gdn"]["write_bytes_per_launch"], 2)
    eager = res.get("eager_same_gpu") or {}
    return {
        "pages_hardware": "NVIDIA H200 and RTX 4090",
        "pages_kernel_speedup": "up to 1.86x over the FLA decode kernel",
        "pages_state_write_cut": "up to 7.83x",
        "pages_end_to_end": "1.05-1.20x (served models, outside this path)",
        "this_run_kernel_speedup_vs_eager_same_gpu": eager.get("deltalog_speedup"),
        "this_kernel_state_write_cut_rocprof": cut,
    }


# ------------------------------------------- merge interval from measurement --
CHOOSE_SWEEP = tuple(range(1, 21)) + (24, 28, 32)


def _fixed_n_launch_us(st, launch, n, pool, G=16, reps=8):
    """Mean us of one launch on handle st with its log held at n entries
    (dl_set_log_len before each launch): G such launches captured in a HIP
    graph, replayed twice untimed, then `reps` times between HIP events."""
    import torch
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        sp = torch.cuda.current_stream().cuda_stream
        for i in range(G):
            st.set_log_len(n)
            launch(0, i % pool, sp)
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    for _ in range(reps):
        g.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) * 1e3 / (reps * G)


def choose_merge_interval(w, pool: int, repeats: int = 3, max_M: int = 32) -> dict:
    """The merge interval from measured launch times, next to a measured sweep
    of M on the same shape (one state, as the large-batch sweep runs it).

    Calibration: for every log length n < max_M, the time of an append launch
    with the log held at n entries (a handle with M = max_M after max_M - 1
    real steps, dl_set_log_len(n) before each launch) and of a merge launch at
    n (a handle with M = n + 1 after n real steps), each over graph replays.
    dl_choose_merge_interval takes these two tables.  Sweep: whole merge
    cycles at every M in CHOOSE_SWEEP and at each suggested M, the median of
    `repeats` passes in alternating order.  Reports the M each model (time,
    and the byte model of dl_suggest_merge_interval) suggests and how far its
    measured time per decode step lies above the measured best."""
    import torch
    import synth
    import recurrent_state_update_amd as rsu
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    inp = stage_inputs(w, pool, dt)
    X0, u = synth.initial(w)
    base = torch.from_numpy(X0).cuda()
    u_dev = None if u is None else torch.from_numpy(u).cuda()
    o = torch.empty(w.B, w.H, w.dv, device="cuda")

    def handle(M):
        return rsu.DeltaLogState(w.op, w.B, w.H, w.dk, w.dv, M, dtype=dt, base=base, u=u_dev)

    sp = lambda: torch.cuda.current_stream().cuda_stream
    st = handle(max_M)
    la = deltalog_launcher(w, inp, [st], o)
    prewarm(la, 1, max_M, pool)          # whole cycles: the log ends empty
    for i in range(max_M - 1):           # a full log of real entries
        la(0, i % pool, sp())
    app = [_fixed_n_launch_us(st, la, n, pool) for n in range(max_M - 1)]
    st.close()
    mer = []
    for n in range(max_M):
        st = handle(n + 1)
        lm = deltalog_launcher(w, inp, [st], o)
        for i in range(n):               # n real entries, then merges at n
            lm(0, i % pool, sp())
        mer.append(_fixed_n_launch_us(st, lm, n, pool))
        st.close()
    timed_M = rsu.dl_choose_merge_interval(app, mer, max_M)
    bytes_M = rsu.dl_suggest_merge_interval(w.B, w.H, w.dk, w.dv, rsu.OPS[w.op], rsu.DTYPES[dt])
    log(f"{w.describe()}: suggested M = {timed_M} (from calibrated launch times), {bytes_M} (from bytes)")

    Ms = sorted(set(CHOOSE_SWEEP) | {timed_M, bytes_M})
    runs = {M: [] for M in Ms}
    for rep in range(repeats):
        for M in (Ms if rep % 2 == 0 else reversed(Ms)):
            base.copy_(torch.from_numpy(X0))
            st = handle(M)
            K = max(4, -(-256 // M))
            ms = time_cycles(deltalog_launcher(w, inp, [st], o), 1, M, pool, K, 2, graphs=True)
            runs[M].append(ms * 1e3)
            st.close()
    sweep = {M: float(np.median(v)) for M, v in runs.items()}
    best = min(sweep, key=sweep.get)
    del inp
    torch.cuda.empty_cache()
    return dict(workload=w.describe(), rotate_states=1,
                calibration_us=dict(append=[round(x, 3) for x in app], merge=[round(x, 3) for x in mer]),
                suggested_M_from_time=timed_M, suggested_M_from_bytes=bytes_M,
                sweep_us_per_decode_step={str(M): round(v, 3) for M, v in sweep.items()},
                sweep_value={str(M): round(w.BH / (v * 1e-6), 1) for M, v in sweep.items()},
                measured_best_M=best,
                gap_time_model=round(sweep[timed_M] / sweep[best] - 1.0, 5),
                gap_byte_model=round(sweep[bytes_M] / sweep[best] - 1.0, 5))


# -------------------------------------------------------------------- main --
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64, help="merge cycles timed (M launches each)")
    ap.add_argument("--warmup", type=int, default=8, help="untimed merge cycles")
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
    ap.add_argument("--choose-M", action="store_true",
                    help="workload 4 only: calibrate launch costs, suggest M from them and from "
                         "bytes, and sweep M to find the measured best (one JSON line)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB, 10 times (the "
                         "reference for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the DeltaLog decode step needs no exchange between "
              "GPUs (slot-heads shard with zero communication), so there is no multi-GPU "
              "figure to take; run it with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("--steps must be >= 1 and --warmup >= 0", file=sys.stderr)
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
    if args.choose_M:
        print(json.dumps({"choose_M": choose_merge_interval(w, pool)}), flush=True)
        return
    res = bench_workload(w, K, W, R, pool, quick=args.quick)
    stock = args.workload in (1, 2, 3) and not args.M and not args.B and not args.H
    default_shape = stock and args.workload == 1
    res["roofline"]["traffic"] = measured_traffic(w.op) if stock else None
    log(f"{w.describe()}: {res['ms_per_launch'] * 1e3:.2f} us per decode step "
        f"({K} merge cycles, {K * w.M} launches)")

    others = {}
    if not args.no_others and default_shape:
        for wid in (2, 3):
            ow = synth.WORKLOADS[wid]
            r = bench_workload(ow, K, W, R, min(ow.steps, 256), with_staged=False)
            others[ow.op] = dict(workload=ow.describe(), value=round(r["value"], 1),
                                 us_per_launch=round(r["ms_per_launch"] * 1e3, 3),
                                 achieved_GBs=r["roofline"]["achieved"], frac=r["roofline"]["frac"],
                                 traffic=measured_traffic(ow.op),
                                 eager_value=r["eager_same_gpu"]["value"],
                                 deltalog_speedup=r["eager_same_gpu"]["deltalog_speedup"],
                                 pattern_cycle_GBs=(r.get("pattern_ceiling") or {}).get("cycle_GBs"),
                                 step_vs_pattern=(r.get("pattern_ceiling") or {}).get("step_vs_pattern"))
            log(f"{ow.describe()}: {r['ms_per_launch'] * 1e3:.2f} us per decode step")

    deep = None
    if default_shape and not args.quick:
        deep = deep_rotation(w, K, W, 24, pool)
        log(f"{w.describe()} over 24 states: {deep['us_per_launch']:.2f} us per decode step")

    cpu = None
    if not args.no_cpu:
        log("timing the CPU oracle ...")
        cpu = cpu_baseline(w)

    ms_launch = res["ms_per_launch"]
    out = {
        "metric": METRIC,
        "value": round(res["value"], 1),
        "unit": "(token·head)/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_launch * w.M, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded PCG64; bf16 q/k/v, fp32 state, beta and log-decay)",
        "config": {"workload": f"DeltaLog {w.op.upper()} decode, B={w.B} H={w.H} d_k={w.dk} "
                               f"d_v={w.dv} M={w.M}; one step = one merge cycle ({w.M} decode steps: "
                               f"{w.M - 1} appends + 1 merge) of one state; {R} states stepped in turn",
                   "B": w.B, "H": w.H, "d_k": w.dk, "d_v": w.dv, "M": w.M, "op": w.op,
                   "decode_steps_per_step": w.M, "rotate_states": R, "input_pool_steps": pool},
        "us_per_decode_step": round(ms_launch * 1e3, 3),
        "roofline": res["roofline"],
        "cpu_baseline": cpu,
        "modelled_step_GBs": res["modelled_step_GBs"],
        "single_state_value": res.get("single_state_value"),
        "graph_replay": res.get("graph_replay"),
        "direct_before_any_graph": dict(
            us_per_launch=res["direct_first_leg_us_per_launch"],
            value=round(w.BH / (res["direct_first_leg_us_per_launch"] * 1e-6), 1),
            note="the same direct launches timed before the process replayed any HIP graph"),
        "per_slot": res.get("per_slot"),
        "two_stage": res.get("two_stage"),
        "eager_same_gpu": res.get("eager_same_gpu"),
        "pattern_ceiling": res.get("pattern_ceiling"),
        "deep_rotation": deep,
        "other_workloads": others or None,
        "pages_context": pages_context(res),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
