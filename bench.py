"""Benchmark of the DeltaLog decode step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload 1] [--rotate R] ...

One "step" is one DeltaLog decode step (ReplayPrep + AppendDecode, with the
fused merge on every M-th step) for all B*H slot-heads of one state, inputs
already resident in HBM.  With --rotate R the steps go round R independent
states (like R layers), so the working set exceeds the 256 MB Infinity Cache
and the state really streams from HBM; the default R=4 is used for the
headline value.  Prints ONE JSON line (rank 0) with the throughput in
(token*head)/s, the roofline of the dominant kernel (the state kernel:
AppendDecode + fused merge) measured with HIP events on the launch stream,
the same-GPU eager baseline, and the fp64 CPU oracle timed on a bounded
sample.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "state-update (token·head)/s + achieved HBM GB/s vs peak, GDN B=64 H=32 d=128"
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# --------------------------------------------------------------- byte model --
def state_kernel_bytes(w, n: int, mode: str) -> int:
    """Algorithmic HBM bytes of one launch of the state kernel over all B*H
    slot-heads: the unique bytes the step must move by its definition.
    mode: 'append' | 'merge' (n = log entries before the step) | 'eager'."""
    dk, dv = w.dk, w.dv
    es = 2 if w.dtype == "bf16" else 4
    delta = w.op != "rwkv6"
    bsz = 4 if delta else es
    lsz = 4 if w.op == "gdn" else 4 * dk
    P = 4 * dk * dv
    io = dv * es + dv * 4 + (4 if delta else 0)           # v, o, beta
    if mode == "eager":
        per = 2 * P + io + (2 * dk * es) + lsz + (0 if delta else 4 * dk)  # + q,k, decay, u
        return per * w.BH
    per = P + io
    per += (2 * dk * es) if delta else dk * es             # q,k (RWKV6: r only)
    per += n * dv * bsz                                    # value-side log shard
    per += (2 * n + 1) * 4 if delta else (n + 1) * 4       # replay coefficients
    per += dv * bsz                                        # append b_t
    if w.op == "kda":
        per += lsz                                         # Lambda'
    elif w.op == "rwkv6":
        per += (lsz if n > 0 else 0)                       # Lambda_{n-1}
    else:
        per += 4
    if mode == "merge":
        per += P                                           # the one dense write
        per += n * dk * es + n * lsz                       # a_j, Lambda_j of logged entries
        if w.op == "rwkv6":
            per += lsz                                     # Lambda' for the fold
    return per * w.BH


def modelled_step_bytes(w) -> float:
    """Whole-step bytes (both kernels) averaged over an M-cycle, SURVEY-style
    model: P(1+1/M) + E((M-1)/M + (M-1)/2) + I, per slot-head."""
    dk, dv, M = w.dk, w.dv, w.M
    es = 2 if w.dtype == "bf16" else 4
    delta = w.op != "rwkv6"
    P = 4 * dk * dv
    E = dk * es + (dv * 4 if delta else dv * es) + (4 if w.op == "gdn" else 4 * dk)
    I = 2 * dk * es + dv * es + dv * 4 + (8 if w.op == "gdn" else 4 + 4 * dk)
    return (P * (1 + 1 / M) + E * ((M - 1) / M + (M - 1) / 2) + I) * w.BH


# ------------------------------------------------------------------- setup --
def stage_inputs(w, pool: int, dt):
    """Pre-stage `pool` distinct steps of inputs in device memory."""
    import torch
    import synth
    t0 = time.time()
    d = synth.steps(w, 0, pool)
    out = {}
    for key, a in d.items():
        if a is None:
            out[key] = None
            continue
        tdt = dt if key in ("q", "k", "v") else torch.float32
        out[key] = torch.from_numpy(a).to("cuda").to(tdt).contiguous()
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


# ------------------------------------------------------------------- timing --
def _ptrs(inp, s):
    """Raw device addresses of step s's inputs (so the timed loop does no
    tensor indexing)."""
    g = lambda key: None if inp[key] is None else inp[key][s].data_ptr()
    return g("q"), g("k"), g("v"), g("beta"), g("ld")


def run_deltalog(w, inp, sts, K: int, W: int, instrument: bool):
    """W warm-up + K timed steps, state i % R at step i.  Returns wall ms,
    per-launch state-kernel ms (list of (ms, n, mode)) and ReplayPrep ms."""
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
    prep_f, app_f = rsu._lib.dl_replay_prep, rsu._lib.dl_append_decode

    def one(i, evs=None):
        h = hs[i % R]
        q, k, v, beta, ld = ptrs[i % pool]
        if evs is not None:
            evs[0].record(stream)
        if prep_f(h, q, k, ld, sp) != 0:
            raise RuntimeError("dl_replay_prep failed")
        if evs is not None:
            evs[1].record(stream)
        if app_f(h, q, k, v, beta, optr[i % 2], sp) != 0:
            raise RuntimeError("dl_append_decode failed")
        if evs is not None:
            evs[2].record(stream)

    for i in range(W):
        one(i)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)] if instrument else None
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    ns = []
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(K):
        ns.append(sts[(W + i) % R].log_len)
        one(W + i, evs[i] if instrument else None)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = t0.elapsed_time(t1)
    launches, prep = [], []
    if instrument:
        for i in range(K):
            n = ns[i]
            mode = "merge" if n + 1 == w.M else "append"
            launches.append((evs[i][1].elapsed_time(evs[i][2]), n, mode))
            prep.append(evs[i][0].elapsed_time(evs[i][1]))
    return wall, launches, prep


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
    wall = t0.elapsed_time(t1)
    per = [evs[i][0].elapsed_time(evs[i][1]) for i in range(K)] if instrument else []
    return wall, per


def cpu_baseline(w, budget_s: float = 12.0, max_steps: int = 64):
    """The fp64 oracle's eager recurrence on the host cores, over all B*H
    slot-heads of the workload, for as many of its steps as fit the budget."""
    import synth
    from oracle import Oracle
    orc = Oracle()
    X0, u = synth.initial(w)
    X = X0.astype(np.float64)
    done, spent = 0, 0.0
    while done < max_steps and spent < budget_s:
        s = synth.step(w, done)
        args = [None if s[k] is None else s[k].astype(np.float64) for k in ("q", "k", "v", "beta", "ld")]
        t0 = time.perf_counter()
        orc.eager_step(w.op, X, *args, None if u is None else u.astype(np.float64))
        spent += time.perf_counter() - t0
        done += 1
    return dict(value=w.BH * done / spent, unit="(token·head)/s", cores=orc.max_threads(),
                kind="oracle",
                sample=f"fp64 eager oracle, all {w.BH} slot-heads of {w.describe()}, first {done} "
                       f"steps ({spent:.1f} s of compute, input generation excluded)")


# -------------------------------------------------------------------- main --
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=512)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--workload", type=int, default=1, choices=[1, 2, 3, 4])
    ap.add_argument("--op", default=None, help="op for workload 4 (gdn|kda)")
    ap.add_argument("--M", type=int, default=None, help="merge interval override (workload 4)")
    ap.add_argument("--rotate", type=int, default=4, help="independent states stepped in turn")
    ap.add_argument("--pool", type=int, default=None, help="distinct input steps staged")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-eager", action="store_true")
    ap.add_argument("--separate-instrument", action="store_true",
                    help="time the per-kernel events in a second pass instead of the timed one")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the DeltaLog decode step needs no exchange "
              "between GPUs (slot-heads shard with zero communication); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    if args.workload == 4:
        w = synth.sweep_workload(args.op or "gdn", args.M or 8)
    else:
        w = synth.WORKLOADS[args.workload]
        if args.M:
            w = w.with_(M=args.M)
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    K, W, R = args.steps, args.warmup, args.rotate
    pool = args.pool or min(w.steps, 256 if w.B <= 64 else 64)
    inp = stage_inputs(w, pool, dt)
    sts, base0, u_dev = make_states(w, R, dt)

    inst_in_timed = not args.separate_instrument
    wall, launches, prep = run_deltalog(w, inp, sts, K, W, instrument=inst_in_timed)
    if not inst_in_timed:
        _, launches, prep = run_deltalog(w, inp, sts, K, W, instrument=True)
    wall_pure, _, _ = run_deltalog(w, inp, sts, K, W, instrument=False)
    log(f"deltalog: {K} steps in {wall:.3f} ms (instrumented), {wall_pure:.3f} ms (no per-kernel events)")

    tot_ms = sum(x[0] for x in launches)
    tot_bytes = sum(state_kernel_bytes(w, n, mode) for (_, n, mode) in launches)
    achieved = tot_bytes / (tot_ms * 1e-3) / 1e9
    avg_ms = tot_ms / len(launches)
    app = [x[0] for x in launches if x[2] == "append"]
    mer = [x[0] for x in launches if x[2] == "merge"]
    roofline = dict(bound="hbm", achieved=round(achieved, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=round(achieved / PEAK_HBM_GBS, 4), traffic=None,
                    kernel="state_kernel (AppendDecode + fused merge)",
                    avg_launch_us=round(avg_ms * 1e3, 2),
                    append_us=round(1e3 * sum(app) / max(len(app), 1), 2),
                    merge_us=round(1e3 * sum(mer) / max(len(mer), 1), 2),
                    bytes_per_launch=int(tot_bytes / len(launches)))

    value = w.BH * K / (wall_pure * 1e-3)
    extra = dict(
        rotate_states=R,
        prep_avg_us=round(1e3 * sum(prep) / max(len(prep), 1), 2),
        modelled_step_GBs=round(modelled_step_bytes(w) / (wall_pure / K * 1e-3) / 1e9, 1),
    )

    if not args.no_eager:
        bases = [base0.clone() for _ in range(R)]
        e_wall, e_per = run_eager(w, inp, bases, u_dev, K, W, instrument=True)
        e_pure, _ = run_eager(w, inp, bases, u_dev, K, W, instrument=False)
        e_bytes = state_kernel_bytes(w, 0, "eager")
        e_avg = sum(e_per) / len(e_per)
        extra["eager_same_gpu"] = dict(
            value=round(w.BH * K / (e_pure * 1e-3), 1), ms_per_step=round(e_pure / K, 5),
            avg_launch_us=round(e_avg * 1e3, 2),
            achieved_GBs=round(e_bytes / (e_avg * 1e-3) / 1e9, 1),
            speedup_deltalog=round(e_pure / wall_pure, 3))
        log(f"eager: {K} steps in {e_pure:.3f} ms")

    # single state (fits the Infinity Cache) for context
    if R > 1:
        one, _, _ = run_deltalog(w, inp, sts[:1], K, W, instrument=False)
        extra["single_state_value"] = round(w.BH * K / (one * 1e-3), 1)

    cpu = None
    if not args.no_cpu:
        log("timing the CPU oracle ...")
        cpu = cpu_baseline(w)

    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "(token·head)/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(wall_pure / K, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded PCG64; bf16 q/k/v, fp32 state/beta/decay)",
        "config": {"workload": f"DeltaLog {w.op.upper()} decode B={w.B} H={w.H} d_k={w.dk} "
                               f"d_v={w.dv} M={w.M}, {R} states stepped in turn",
                   "B": w.B, "H": w.H, "d_k": w.dk, "d_v": w.dv, "M": w.M, "op": w.op,
                   "rotate_states": R, "input_pool_steps": pool},
        "roofline": roofline,
        "cpu_baseline": cpu,
        **extra,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
