"""GPU parity: the HIP path (through the C ABI) against the fp64 eager oracle,
element by element, on seeded synthetic workloads.

Checked every step: o_t.  Checked after every merge (and after forced merges):
the dense base S-bar, which must equal the eager state.  Bar: max-abs relative
error below the pages' 5e-3, and below the tighter fp32 bound FP32_TOL."""
import numpy as np
import pytest
import torch

import synth
from gpu_harness import FP32_TOL, PAGES_TOL, ParityRun, dev, in_dtype, rel, sample_slot_heads

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU")


def _report(run, name):
    print(f"[{name}] steps={run.t} worst o={run.worst_o:.2e} worst S={run.worst_S:.2e} "
          f"(states checked {run.checked_S})", flush=True)
    assert run.worst_o < PAGES_TOL and run.worst_S < PAGES_TOL
    assert run.worst_o < FP32_TOL and run.worst_S < FP32_TOL


@needs_gpu
def test_tiny_gdn_workload_full(orc):
    """GDN B=1 H=2 d=16 M=4, 32 steps, fp32: every output and every merge."""
    w = synth.WORKLOADS[0]
    run = ParityRun(w, orc=orc)
    for _ in range(w.steps):
        run.step()
    assert run.checked_S == w.steps // w.M
    _report(run, "w0")
    run.close()


@needs_gpu
@pytest.mark.parametrize("wid", [1, 2, 3])
def test_serving_ops_reduced_batch(orc, wid):
    """Workloads 1-3 at their d and M, with B*H cut to 15 slot-heads (ragged
    over the 8 XCDs and over 4-wave ReplayPrep groups), 3 merge cycles."""
    w = synth.WORKLOADS[wid].with_(B=3, H=5)
    run = ParityRun(w, orc=orc)
    for _ in range(3 * w.M):
        run.step()
    _report(run, f"w{wid} B=3 H=5")
    run.close()


@needs_gpu
@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
@pytest.mark.parametrize("dk", [16, 32, 64, 128])
@pytest.mark.parametrize("dv", [16, 32, 64, 128])
@pytest.mark.parametrize("path", ["fused", "staged"])
def test_all_shapes(orc, op, dk, dv, path):
    """Every supported (d_k, d_v) for every op and both paths, bf16 inputs,
    M=3, 7 steps (two merges and a pending log), then a forced merge."""
    w = synth.Workload(9, op, 2, 3, dk, dv, 3, 7, "bf16")
    run = ParityRun(w, orc=orc)
    for _ in range(7):
        run.step(staged=path == "staged")
    run.merge()
    _report(run, f"{op} dk={dk} dv={dv} {path}")
    run.close()


@needs_gpu
@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
@pytest.mark.parametrize("M", [1, 2, 4, 5, 8, 16, 32])
def test_merge_intervals(orc, op, M):
    """Outputs every step and the base after every merge, for M from 1
    (eager) to the maximum 32."""
    w = synth.Workload(10, op, 2, 4, 64, 64, M, max(2 * M, 8), "bf16")
    run = ParityRun(w, orc=orc)
    for _ in range(w.steps):
        run.step()
    run.merge()
    _report(run, f"{op} M={M}")
    run.close()


@needs_gpu
@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
def test_forced_merge_at_every_log_length(orc, op):
    """dl_merge after n = 1..M-1 appends gives the eager state; a second
    merge is a no-op; the schedule then continues correctly."""
    M = 8
    for stop in range(1, M):
        w = synth.Workload(11, op, 1, 5, 128, 128, M, stop, "bf16")
        run = ParityRun(w, orc=orc)
        for _ in range(stop):
            run.step()
        assert run.st.log_len == stop
        run.merge()
        before = run.state_gpu().copy()
        run.merge()
        assert np.array_equal(before, run.state_gpu())
        for _ in range(M + 1):
            run.step()
        _report(run, f"{op} forced merge at n={stop}")
        run.close()


@needs_gpu
@pytest.mark.parametrize("wid", [0, 1, 2, 3])
def test_eager_kernel(orc, wid):
    """The eager baseline kernel against the oracle (reduced batch)."""
    w = synth.WORKLOADS[wid]
    if wid:
        w = w.with_(B=2, H=7)
    run = ParityRun(w, eager=True, orc=orc)
    for _ in range(12):
        run.step()
    _report(run, f"eager w{wid}")


@needs_gpu
@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
def test_m1_matches_eager_kernel(op):
    """M = 1 DeltaLog and the eager kernel compute the same recurrence."""
    w = synth.Workload(12, op, 2, 3, 128, 64, 1, 6, "bf16")
    a = ParityRun(w)
    b = ParityRun(w, eager=True)
    for t in range(6):
        s = synth.step(w, t)
        a.step(s)
        b.step(s)
        assert rel(a.state_gpu(), b.state_gpu()) < 1e-5
    a.close()


@needs_gpu
@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
def test_staged_and_fused_paths(orc, op):
    """The two-stage path (dl_replay_prep + dl_append_decode) and the one-launch
    path (dl_decode_step) both match the oracle and each other; repeated runs
    of one path are bit-identical (no atomics, fixed reduction order)."""
    w = synth.Workload(13, op, 2, 3, 128, 128, 4, 10, "bf16")
    fused = [ParityRun(w, orc=orc) for _ in range(2)]
    staged = [ParityRun(w, orc=orc) for _ in range(2)]
    for t in range(10):
        s = synth.step(w, t)
        for r in fused:
            r.step(s)
        for r in staged:
            r.step(s, staged=True)
    g = [r.state_gpu() for r in fused + staged]
    assert np.array_equal(g[0], g[1]) and np.array_equal(g[2], g[3])
    assert rel(g[0], g[2]) < 1e-5
    for r in fused + staged:
        _report(r, f"{op} {'staged' if r in staged else 'fused'}")
        r.close()


@needs_gpu
@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
@pytest.mark.parametrize("M", [1, 3, 8, 32])
def test_staged_path_merge_intervals(orc, op, M):
    """The two-stage ReplayPrep/AppendDecode path over whole merge cycles."""
    w = synth.Workload(16, op, 3, 5, 64, 128, M, 2 * M + 1, "bf16")
    run = ParityRun(w, orc=orc)
    for _ in range(w.steps):
        run.step(staged=True)
    run.merge()
    _report(run, f"{op} staged M={M}")
    run.close()


@needs_gpu
def test_call_order_errors():
    import recurrent_state_update_amd as rsu
    w = synth.Workload(14, "gdn", 1, 2, 16, 16, 4, 2, "f32")
    run = ParityRun(w)
    s = synth.step(w, 0)
    q, k, ld = dev(s["q"]), dev(s["k"]), dev(s["ld"])
    run.st.replay_prep(q, k, ld)
    with pytest.raises(rsu.DeltaLogError):
        run.st.replay_prep(q, k, ld)          # prep twice
    with pytest.raises(rsu.DeltaLogError):
        run.st.merge()                        # merge between the stages
    run.st.append_decode(q, k, dev(s["v"]), dev(s["beta"]))
    assert run.st.log_len == 1
    run.close()


@needs_gpu
@pytest.mark.parametrize("op", ["gdn", "rwkv6"])
def test_checkpoint_restore_mid_cycle(op):
    """Saving base + workspace at log length n and restoring them into a new
    handle continues bit-identically to the uninterrupted run."""
    import recurrent_state_update_amd as rsu
    w = synth.Workload(15, op, 2, 2, 64, 64, 8, 14, "bf16")
    X0, u = synth.initial(w)
    dt = in_dtype(w)
    a = rsu.DeltaLogState(op, w.B, w.H, w.dk, w.dv, w.M, dtype=dt, base=dev(X0), u=dev(u))
    inputs = [synth.step(w, t) for t in range(w.steps)]

    def go(st, s):
        return st.step(dev(s["q"], dt), dev(s["k"], dt), dev(s["v"], dt), dev(s["beta"]), dev(s["ld"]))

    for t in range(3):
        go(a, inputs[t])
    snap_base, snap_ws, n = a.base.clone(), a.workspace.clone(), a.log_len
    assert n == 3
    outs_a = [go(a, inputs[t]).cpu() for t in range(3, w.steps)]
    b = rsu.DeltaLogState(op, w.B, w.H, w.dk, w.dv, w.M, dtype=dt, base=snap_base, u=dev(u))
    b.workspace.copy_(snap_ws)
    b.set_log_len(n)
    outs_b = [go(b, inputs[t]).cpu() for t in range(3, w.steps)]
    for x, y in zip(outs_a, outs_b):
        assert torch.equal(x, y)
    a.merge()
    b.merge()
    assert torch.equal(a.base, b.base)


@needs_gpu
@pytest.mark.parametrize("wid", [1, 2, 3])
def test_full_size_workloads(orc, wid):
    """Workloads 1-3 at full size and length (all B*H slot-heads, all 256
    steps, the one-launch path the benchmark times): every output at every
    step and the whole base after every merge, against the oracle."""
    w = synth.WORKLOADS[wid]
    run = ParityRun(w, orc=orc)
    for _ in range(w.steps):
        run.step()
    assert run.checked_S == w.steps // w.M
    _report(run, f"w{wid} full size, all {w.BH} slot-heads")
    run.close()


@needs_gpu
@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
def test_graph_capture_of_merge_cycles(orc, op):
    """M decode steps (one whole merge cycle) captured in a HIP graph through
    torch.cuda.graph, replayed three times with fresh inputs copied into the
    captured buffers and the program's own eager work and synchronisations in
    between.  Every replay must match the same steps launched directly, bit
    for bit, and the oracle."""
    import recurrent_state_update_amd as rsu
    M = 4
    w = synth.Workload(17, op, 2, 3, 64, 128, M, 3 * M, "bf16")
    X0, u = synth.initial(w)
    dt = in_dtype(w)
    a = rsu.DeltaLogState(op, w.B, w.H, w.dk, w.dv, M, dtype=dt, base=dev(X0), u=dev(u))
    b = rsu.DeltaLogState(op, w.B, w.H, w.dk, w.dv, M, dtype=dt, base=dev(X0), u=dev(u))
    first = [synth.step(w, t) for t in range(M)]
    static = [{k: dev(v, dt if k in ("q", "k", "v") else torch.float32) for k, v in s.items()} for s in first]
    outs = [torch.empty(w.B, w.H, w.dv, device="cuda") for _ in range(M)]

    def launch(st, s, o):
        return st.step(s["q"], s["k"], s["v"], s["beta"], s["ld"], o=o)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for t in range(M):
            launch(b, static[t], outs[t])
    assert b.log_len == 0  # a whole cycle: the host schedule is back where it started
    X = X0.reshape(w.BH, w.dk, w.dv).astype(np.float64)[None].copy()
    u_sub = None if u is None else u[np.arange(w.BH) % w.H].astype(np.float64)
    for cycle in range(3):
        inputs = [synth.step(w, cycle * M + t) for t in range(M)]
        for t in range(M):
            for k_, v_ in inputs[t].items():
                if v_ is not None:
                    static[t][k_].copy_(dev(v_, dt if k_ in ("q", "k", "v") else torch.float32))
        torch.cuda.synchronize()
        g.replay()
        ref_outs = [launch(a, static[t], None).clone() for t in range(M)]  # direct launches
        torch.cuda.synchronize()
        for t in range(M):
            assert torch.equal(outs[t], ref_outs[t]), (cycle, t)
            sub = synth.subset(inputs[t], np.arange(w.BH))
            o_ref = orc.eager_step(op, X, sub["q"], sub["k"], sub["v"], sub["beta"], sub["ld"], u_sub)
            assert rel(outs[t].reshape(w.BH, w.dv).cpu().numpy(), o_ref[0]) < FP32_TOL
        assert torch.equal(a.base, b.base)
        assert rel(b.base.reshape(w.BH, w.dk, w.dv).cpu().numpy(), X[0]) < FP32_TOL
    a.close()
    b.close()


@needs_gpu
@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
@pytest.mark.parametrize("M", [4, 8])
def test_per_slot_logs_continuous_batching(orc, op, M):
    """Per-slot logs: requests are admitted into slots at different steps
    (fresh initial states written into the slot's base rows), so slots merge
    at different steps within one launch; one slot is merged early to retire
    its request.  Every output is checked against the eager oracle, each
    slot's base right after its own merge, and all bases after dl_merge."""
    import recurrent_state_update_amd as rsu
    B, H = 5, 3
    w = synth.Workload(18, op, B, H, 64, 128, M, 3 * M + 5, "bf16")
    X0, u = synth.initial(w)
    dt = in_dtype(w)
    st = rsu.DeltaLogState(op, B, H, w.dk, w.dv, M, dtype=dt, base=dev(X0), u=dev(u))
    st.enable_slots()
    X = X0.reshape(B * H, w.dk, w.dv).astype(np.float64)[None].copy()
    u_sub = None if u is None else u[np.arange(B * H) % H].astype(np.float64)
    admissions = {1: [1], 3: [2], 5: [4, 1], M + 2: [3]}   # step -> slots admitted before it
    retire = {M + 1: 0}                                       # step -> slot merged before it
    worst_o = worst_S = 0.0
    checked = 0
    for t in range(w.steps):
        for b in admissions.get(t, []):
            new = synth.initial(w.with_(wid=1000 + 10 * t + b))[0][b]       # [H, dk, dv]
            st.base[b].copy_(dev(new))
            st.admit(b)
            X[0, b * H:(b + 1) * H] = new.astype(np.float64)
            assert st.slot_log_len(b) == 0
        if t in retire:
            b = retire[t]
            st.merge_slot(b)
            assert st.slot_log_len(b) == 0
            worst_S = max(worst_S, rel(st.base[b].cpu().numpy(), X[0, b * H:(b + 1) * H]))
        s = synth.step(w, t)
        d = {k_: dev(v_, dt if k_ in ("q", "k", "v") else torch.float32) for k_, v_ in s.items()}
        o = st.step(d["q"], d["k"], d["v"], d["beta"], d["ld"])
        sub = synth.subset(s, np.arange(B * H))
        o_ref = orc.eager_step(op, X, sub["q"], sub["k"], sub["v"], sub["beta"], sub["ld"], u_sub)
        worst_o = max(worst_o, rel(o.reshape(B * H, w.dv).cpu().numpy(), o_ref[0]))
        lens = [st.slot_log_len(b) for b in range(B)]
        assert len(set(lens)) > 1 or t < 1   # slots really are out of phase
        for b in range(B):
            if lens[b] == 0:                 # this slot merged at this step
                worst_S = max(worst_S, rel(st.base[b].cpu().numpy(), X[0, b * H:(b + 1) * H]))
                checked += 1
    st.merge()
    assert all(st.slot_log_len(b) == 0 for b in range(B))
    worst_S = max(worst_S, rel(st.base.reshape(B * H, w.dk, w.dv).cpu().numpy(), X[0]))
    print(f"[{op} per-slot M={M}] worst o={worst_o:.2e} S={worst_S:.2e} merges checked {checked}")
    assert checked >= B
    assert worst_o < FP32_TOL and worst_S < FP32_TOL
    st.close()


@needs_gpu
@pytest.mark.parametrize("wid", [1, 2, 3])
def test_full_size_graph_replay(orc, wid):
    """The launch configuration the benchmark times: dl_decode_step at the
    workload's full size, one merge cycle captured in a HIP graph and replayed
    for two cycles with fresh inputs copied into the captured buffers.  Every
    output and the base after each cycle are checked on all B*H slot-heads
    against the oracle."""
    import recurrent_state_update_amd as rsu
    w = synth.WORKLOADS[wid]
    M = w.M
    idx = np.arange(w.BH)
    X0, u = synth.initial(w)
    dt = in_dtype(w)
    base = dev(X0)
    st = rsu.DeltaLogState(w.op, w.B, w.H, w.dk, w.dv, M, dtype=dt, base=base, u=dev(u))
    static = [{k: dev(v, dt if k in ("q", "k", "v") else torch.float32) for k, v in synth.step(w, t).items()}
              for t in range(M)]
    outs = [torch.empty(w.B, w.H, w.dv, device="cuda") for _ in range(M)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for t in range(M):
            s = static[t]
            st.step(s["q"], s["k"], s["v"], s["beta"], s["ld"], o=outs[t])
    assert st.log_len == 0
    X = X0.reshape(w.BH, w.dk, w.dv)[idx].astype(np.float64)[None].copy()
    u_sub = None if u is None else u[idx % w.H].astype(np.float64)
    sel = torch.from_numpy(idx).cuda()
    worst_o = worst_S = 0.0
    for cycle in range(2):
        inputs = [synth.step(w, cycle * M + t) for t in range(M)]
        for t in range(M):
            for k_, v_ in inputs[t].items():
                if v_ is not None:
                    static[t][k_].copy_(dev(v_, dt if k_ in ("q", "k", "v") else torch.float32))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t in range(M):
            sub = synth.subset(inputs[t], idx)
            o_ref = orc.eager_step(w.op, X, sub["q"], sub["k"], sub["v"], sub["beta"], sub["ld"], u_sub)
            worst_o = max(worst_o, rel(outs[t].reshape(w.BH, w.dv)[sel].cpu().numpy(), o_ref[0]))
        worst_S = max(worst_S, rel(base.reshape(w.BH, w.dk, w.dv)[sel].cpu().numpy(), X[0]))
    print(f"[w{wid} full-size graph replay] worst o={worst_o:.2e} S={worst_S:.2e}", flush=True)
    st.close()
    assert worst_o < FP32_TOL and worst_S < FP32_TOL


@needs_gpu
def test_largest_state_the_abi_accepts(orc):
    """The largest state below the 2^33-element limit at d=128: B*H = 524287
    slot-heads (32 GiB of fp32 state, so the last slot-heads lie past 2^31
    elements and 2^32 bytes), GDN bf16, M=2, three steps (a merge and a
    pending log).  The base is zero except on 48 sampled slot-heads (first and
    last included), whose seeded initial states and every output are checked
    against the oracle, with the base after the final forced merge."""
    import recurrent_state_update_amd as rsu
    B, H, d, M = 524287, 1, 128, 2
    assert B * H * d * d < 2**33 and (B + 1) * H * d * d >= 2**33
    w = synth.Workload(19, "gdn", B, H, d, d, M, 3, "bf16")
    idx = sample_slot_heads(B * H, 48, seed=19)
    X0_rows = synth.initial(w.with_(B=len(idx)))[0].reshape(len(idx), d, d)  # seeded rows for the sample
    base = torch.zeros(B, H, d, d, device="cuda")
    sel = torch.from_numpy(idx).cuda()
    base.view(B * H, d, d)[sel] = torch.from_numpy(X0_rows).cuda()
    st = rsu.DeltaLogState("gdn", B, H, d, d, M, dtype=torch.bfloat16, base=base)
    X = X0_rows.astype(np.float64)[None].copy()
    worst_o = 0.0
    for t in range(3):
        s = synth.step(w, t)
        d_ = {k_: dev(v_, torch.bfloat16 if k_ in ("q", "k", "v") else torch.float32) for k_, v_ in s.items()}
        o = st.step(d_["q"], d_["k"], d_["v"], d_["beta"], d_["ld"])
        sub = synth.subset(s, idx)
        o_ref = orc.eager_step("gdn", X, sub["q"], sub["k"], sub["v"], sub["beta"], sub["ld"])
        worst_o = max(worst_o, rel(o.view(B * H, d)[sel].cpu().numpy(), o_ref[0]))
        del d_, o
    st.merge()
    worst_S = rel(base.view(B * H, d, d)[sel].cpu().numpy(), X[0])
    print(f"[largest state] worst o={worst_o:.2e} S={worst_S:.2e}", flush=True)
    st.close()
    del base
    torch.cuda.empty_cache()
    assert worst_o < FP32_TOL and worst_S < FP32_TOL


@needs_gpu
@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
@pytest.mark.parametrize("shape", [(16, 16), (32, 128), (128, 32), (64, 64), (128, 128)])
@pytest.mark.parametrize("path", ["fused", "staged", "eager"])
def test_fp32_inputs(orc, op, shape, path):
    """fp32 q/k/v (the kernels read whole 32-bit elements instead of picking
    bf16 halves, and the RWKV6 b-log is fp32): every operator, square and
    lopsided shapes, both DeltaLog paths and the eager kernel; M=3, 7 steps
    (two merges and a pending log), then a forced merge."""
    dk, dv = shape
    w = synth.Workload(20, op, 2, 3, dk, dv, 3, 7, "f32")
    run = ParityRun(w, eager=path == "eager", orc=orc)
    for _ in range(7):
        run.step(staged=path == "staged")
    if path != "eager":
        run.merge()
    _report(run, f"fp32 {op} dk={dk} dv={dv} {path}")
    run.close()


@needs_gpu
@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
def test_fp32_inputs_per_slot(orc, op):
    """fp32 inputs on a handle with per-slot logs: two requests admitted late
    with fresh seeded states, outputs every step and all bases after the
    final merge."""
    import recurrent_state_update_amd as rsu
    B, H, M = 4, 2, 4
    w = synth.Workload(21, op, B, H, 64, 64, M, 2 * M + 3, "f32")
    X0, u = synth.initial(w)
    st = rsu.DeltaLogState(op, B, H, 64, 64, M, dtype=torch.float32, base=dev(X0), u=dev(u))
    st.enable_slots()
    X = X0.reshape(B * H, 64, 64).astype(np.float64)[None].copy()
    u_sub = None if u is None else u[np.arange(B * H) % H].astype(np.float64)
    worst = 0.0
    for t in range(w.steps):
        if t in (1, 3):
            b = t  # a new request in slot 1, then slot 3, from a fresh seeded state
            new = synth.initial(w.with_(wid=2000 + t))[0][b]
            st.base[b].copy_(dev(new))
            st.admit(b)
            X[0, b * H:(b + 1) * H] = new.astype(np.float64)
        s = synth.step(w, t)
        d_ = {k_: dev(v_) for k_, v_ in s.items()}
        o = st.step(d_["q"], d_["k"], d_["v"], d_["beta"], d_["ld"])
        sub = synth.subset(s, np.arange(B * H))
        o_ref = orc.eager_step(op, X, sub["q"], sub["k"], sub["v"], sub["beta"], sub["ld"], u_sub)
        worst = max(worst, rel(o.reshape(B * H, 64).cpu().numpy(), o_ref[0]))
    st.merge()
    worst_S = rel(st.base.reshape(B * H, 64, 64).cpu().numpy(), X[0])
    st.close()
    print(f"[fp32 per-slot {op}] worst o={worst:.2e} S={worst_S:.2e}", flush=True)
    assert worst < FP32_TOL and worst_S < FP32_TOL


@needs_gpu
@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
def test_runs_are_bit_identical(op):
    """The kernels use no atomics and a fixed reduction order, so two runs of
    the same steps on fresh states give bit-identical outputs and bases, for
    lockstep and per-slot handles alike."""
    import recurrent_state_update_amd as rsu
    w = synth.Workload(22, op, 4, 8, 128, 128, 4, 11, "bf16")
    X0, u = synth.initial(w)
    dt = in_dtype(w)
    steps = [{k_: dev(v_, dt if k_ in ("q", "k", "v") else torch.float32) for k_, v_ in synth.step(w, t).items()}
             for t in range(w.steps)]
    for slots in (False, True):
        runs = []
        for _ in range(2):
            st = rsu.DeltaLogState(op, w.B, w.H, w.dk, w.dv, w.M, dtype=dt, base=dev(X0), u=dev(u))
            if slots:
                st.enable_slots()
            outs = []
            for t, s in enumerate(steps):
                if slots and t == 2:
                    st.admit(1)
                outs.append(st.step(s["q"], s["k"], s["v"], s["beta"], s["ld"]).clone())
            st.merge()
            runs.append((outs, st.base.clone()))
            st.close()
        (oa, ba), (ob, bb) = runs
        assert all(torch.equal(x, y) for x, y in zip(oa, ob)), (op, slots)
        assert torch.equal(ba, bb), (op, slots)


@needs_gpu
@pytest.mark.parametrize("op", ["gdn", "kda"])
@pytest.mark.parametrize("M", list(synth.SWEEP_MS))
def test_large_batch_long_run(orc, op, M):
    """The large-batch configuration at its full length, at every merge
    interval of the sweep: B=256 H=32 d=128 (512 MiB state), all 1024 decode
    steps (1024 / M merges), inputs cycling a staged pool of 64 steps as the
    benchmark does.  32 sampled slot-heads (first and last included; slot-heads
    are independent, so a subset is exact): every output, and the base after
    every merge, against the oracle (no drift over the run).  A forced merge at
    the end must leave the base as it is (the log is empty)."""
    import recurrent_state_update_amd as rsu
    w = synth.sweep_workload(op, M, steps=1024)
    pool = 64
    idx = sample_slot_heads(w.BH, 32, seed=41 + M)
    sel = torch.from_numpy(idx).cuda()
    X0, u = synth.initial(w)
    dt = in_dtype(w)
    base = dev(X0)
    st = rsu.DeltaLogState(op, w.B, w.H, w.dk, w.dv, w.M, dtype=dt, base=base, u=dev(u))
    staged, subs = [], []
    for s_ in range(pool):
        s = synth.step(w, s_)
        staged.append({k_: dev(v_, dt if k_ in ("q", "k", "v") else torch.float32) for k_, v_ in s.items()})
        subs.append(synth.subset(s, idx))
    X = X0.reshape(w.BH, w.dk, w.dv)[idx].astype(np.float64)[None].copy()
    worst_o = worst_S = 0.0
    merges = 0
    for t in range(w.steps):
        d_, sub = staged[t % pool], subs[t % pool]
        o = st.step(d_["q"], d_["k"], d_["v"], d_["beta"], d_["ld"])
        o_ref = orc.eager_step(op, X, sub["q"], sub["k"], sub["v"], sub["beta"], sub["ld"])
        worst_o = max(worst_o, rel(o.reshape(w.BH, w.dv)[sel].cpu().numpy(), o_ref[0]))
        if st.log_len == 0:
            merges += 1
            worst_S = max(worst_S, rel(base.reshape(w.BH, w.dk, w.dv)[sel].cpu().numpy(), X[0]))
    st.merge()
    worst_S = max(worst_S, rel(base.reshape(w.BH, w.dk, w.dv)[sel].cpu().numpy(), X[0]))
    print(f"[{op} B=256 M={M} 1024 steps] worst o={worst_o:.2e} S={worst_S:.2e} merges {merges}",
          flush=True)
    st.close()
    assert merges == w.steps // M
    assert worst_o < PAGES_TOL and worst_S < PAGES_TOL
    assert worst_o < FP32_TOL and worst_S < FP32_TOL


@needs_gpu
@pytest.mark.parametrize("op", ["gdn", "rwkv6"])
def test_released_slots_are_skipped(orc, op):
    """A finished request is merged and its slot released: later steps and
    merges leave that slot's base rows and outputs untouched (no traffic),
    while the other slots keep matching the oracle; the slot is then admitted
    again with a fresh state and matches the oracle from there."""
    import recurrent_state_update_amd as rsu
    B, H, M = 5, 2, 4
    w = synth.Workload(23, op, B, H, 64, 64, M, 14, "bf16")
    X0, u = synth.initial(w)
    dt = in_dtype(w)
    st = rsu.DeltaLogState(op, B, H, 64, 64, M, dtype=dt, base=dev(X0), u=dev(u))
    st.enable_slots()
    X = X0.reshape(B * H, 64, 64).astype(np.float64)[None].copy()
    u_sub = None if u is None else u[np.arange(B * H) % H].astype(np.float64)
    rows = lambda b: slice(b * H, (b + 1) * H)
    o = torch.full((B, H, 64), float("nan"), device="cuda")
    live = [True] * B
    worst = 0.0
    frozen = None
    for t in range(w.steps):
        if t == 5:   # slot 2 finishes: merge, keep its state, release
            st.merge_slot(2)
            st.release(2)
            frozen = st.base[2].clone()
            assert rel(frozen.cpu().numpy(), X[0, rows(2)]) < FP32_TOL
            live[2] = False
            o[2].fill_(float("nan"))
            assert st.slot_log_len(2) == 0
        if t == 10:  # a new request in slot 2
            new = synth.initial(w.with_(wid=3000))[0][2]
            st.base[2].copy_(dev(new))
            st.admit(2)
            X[0, rows(2)] = new.astype(np.float64)
            live[2] = True
        s = synth.step(w, t)
        d_ = {k_: dev(v_, dt if k_ in ("q", "k", "v") else torch.float32) for k_, v_ in s.items()}
        st.step(d_["q"], d_["k"], d_["v"], d_["beta"], d_["ld"], o=o)
        sub = synth.subset(s, np.arange(B * H))
        Xprev = X[0, rows(2)].copy()
        o_ref = orc.eager_step(op, X, sub["q"], sub["k"], sub["v"], sub["beta"], sub["ld"], u_sub)
        if not live[2]:
            X[0, rows(2)] = Xprev  # the oracle leaves the released slot alone too
            assert torch.isnan(o[2]).all()
            assert torch.equal(st.base[2], frozen)
        for b in range(B):
            if live[b]:
                worst = max(worst, rel(o[b].reshape(H, 64).cpu().numpy(), o_ref[0, rows(b)]))
    st.merge()
    worst_S = max(rel(st.base[b].cpu().numpy(), X[0, rows(b)]) for b in range(B))
    st.close()
    print(f"[{op} release] worst o={worst:.2e} S={worst_S:.2e}", flush=True)
    assert worst < FP32_TOL and worst_S < FP32_TOL


@needs_gpu
@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
def test_per_slot_long_logs(orc, op):
    """Per-slot logs at the largest merge interval (M=32, d=128, two value
    tiles): slots admitted at different steps hold logs of very different
    lengths in one launch, so long-log workgroups (the second staging pass of
    the log shard, one-entry-per-wave coefficients) run beside short-log and
    merging ones.  Every output and each slot's base after its own merge."""
    import recurrent_state_update_amd as rsu
    B, H, M = 3, 2, 32
    w = synth.Workload(25, op, B, H, 128, 128, M, 2 * M + 9, "bf16")
    X0, u = synth.initial(w)
    dt = in_dtype(w)
    st = rsu.DeltaLogState(op, B, H, 128, 128, M, dtype=dt, base=dev(X0), u=dev(u))
    st.enable_slots()
    X = X0.reshape(B * H, 128, 128).astype(np.float64)[None].copy()
    u_sub = None if u is None else u[np.arange(B * H) % H].astype(np.float64)
    rows = lambda b: slice(b * H, (b + 1) * H)
    admissions = {7: 1, 19: 2}
    worst_o = worst_S = 0.0
    merged = set()
    for t in range(w.steps):
        if t in admissions:
            b = admissions[t]
            new = synth.initial(w.with_(wid=4000 + t))[0][b]
            st.base[b].copy_(dev(new))
            st.admit(b)
            X[0, rows(b)] = new.astype(np.float64)
        s = synth.step(w, t)
        d_ = {k_: dev(v_, dt if k_ in ("q", "k", "v") else torch.float32) for k_, v_ in s.items()}
        o = st.step(d_["q"], d_["k"], d_["v"], d_["beta"], d_["ld"])
        sub = synth.subset(s, np.arange(B * H))
        o_ref = orc.eager_step(op, X, sub["q"], sub["k"], sub["v"], sub["beta"], sub["ld"], u_sub)
        worst_o = max(worst_o, rel(o.reshape(B * H, 128).cpu().numpy(), o_ref[0]))
        for b in range(B):
            if st.slot_log_len(b) == 0:
                merged.add(b)
                worst_S = max(worst_S, rel(st.base[b].cpu().numpy(), X[0, rows(b)]))
    st.merge()
    worst_S = max(worst_S, max(rel(st.base[b].cpu().numpy(), X[0, rows(b)]) for b in range(B)))
    st.close()
    print(f"[{op} per-slot M=32] worst o={worst_o:.2e} S={worst_S:.2e} slots merged {sorted(merged)}", flush=True)
    assert merged == {0, 1, 2}
    assert worst_o < FP32_TOL and worst_S < FP32_TOL


@needs_gpu
@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
def test_graph_capture_per_slot(orc, op):
    """Per-slot logs under HIP graph capture: one merge cycle captured, then
    replayed three times with fresh inputs; between replays a request is
    admitted (new state written into its slot) and another released, outside
    the graph.  Every replay matches a twin handle driven by direct launches
    bit for bit, and the oracle on the live slots."""
    import recurrent_state_update_amd as rsu
    B, H, M = 4, 2, 4
    w = synth.Workload(26, op, B, H, 64, 128, M, 3 * M, "bf16")
    X0, u = synth.initial(w)
    dt = in_dtype(w)
    a = rsu.DeltaLogState(op, B, H, 64, 128, M, dtype=dt, base=dev(X0), u=dev(u))
    b = rsu.DeltaLogState(op, B, H, 64, 128, M, dtype=dt, base=dev(X0), u=dev(u))
    for st in (a, b):
        st.enable_slots()
    # stagger slot 3 before capture (both handles alike)
    warm = [{k_: dev(v_, dt if k_ in ("q", "k", "v") else torch.float32) for k_, v_ in synth.step(w.with_(wid=27), t).items()}
            for t in range(2)]
    X = X0.reshape(B * H, 64, 128).astype(np.float64)[None].copy()
    u_sub = None if u is None else u[np.arange(B * H) % H].astype(np.float64)
    for t, s in enumerate(warm):
        for st in (a, b):
            st.step(s["q"], s["k"], s["v"], s["beta"], s["ld"])
        sub = synth.subset(synth.step(w.with_(wid=27), t), np.arange(B * H))
        orc.eager_step(op, X, sub["q"], sub["k"], sub["v"], sub["beta"], sub["ld"], u_sub)
    new3 = synth.initial(w.with_(wid=5003))[0][3]
    for st in (a, b):
        st.base[3].copy_(dev(new3))
        st.admit(3)
    X[0, 6:8] = new3.astype(np.float64)
    static = [{k_: dev(v_, dt if k_ in ("q", "k", "v") else torch.float32) for k_, v_ in synth.step(w, t).items()}
              for t in range(M)]
    outs = [torch.empty(B, H, 128, device="cuda") for _ in range(M)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for t in range(M):
            s = static[t]
            b.step(s["q"], s["k"], s["v"], s["beta"], s["ld"], o=outs[t])
    live = [True] * B
    rows = lambda s_: slice(s_ * H, (s_ + 1) * H)
    worst = 0.0
    for cycle in range(3):
        if cycle == 1:  # a new request in slot 0, slot 2 finishes
            new0 = synth.initial(w.with_(wid=5100))[0][0]
            for st in (a, b):
                st.base[0].copy_(dev(new0))
                st.admit(0)
                st.merge_slot(2)
                st.release(2)
            X[0, rows(0)] = new0.astype(np.float64)
            live[2] = False
        inputs = [synth.step(w, cycle * M + t) for t in range(M)]
        for t in range(M):
            for k_, v_ in inputs[t].items():
                if v_ is not None:
                    static[t][k_].copy_(dev(v_, dt if k_ in ("q", "k", "v") else torch.float32))
        torch.cuda.synchronize()
        g.replay()
        ref = [a.step(static[t]["q"], static[t]["k"], static[t]["v"], static[t]["beta"], static[t]["ld"]).clone()
               for t in range(M)]
        torch.cuda.synchronize()
        for t in range(M):
            for s_ in range(B):
                if live[s_]:
                    assert torch.equal(outs[t][s_], ref[t][s_]), (cycle, t, s_)
            sub = synth.subset(inputs[t], np.arange(B * H))
            Xkeep = X[0, rows(2)].copy()
            o_ref = orc.eager_step(op, X, sub["q"], sub["k"], sub["v"], sub["beta"], sub["ld"], u_sub)
            if not live[2]:
                X[0, rows(2)] = Xkeep
            for s_ in range(B):
                if live[s_]:
                    worst = max(worst, rel(outs[t][s_].cpu().numpy(), o_ref[0, rows(s_)]))
        assert torch.equal(a.base, b.base)
    print(f"[{op} per-slot graph] worst o={worst:.2e}", flush=True)
    a.close()
    b.close()
    assert worst < FP32_TOL


def _with_full_decay(s: dict, t: int, rng) -> dict:
    """Step inputs with full forgetting mixed in: log-decay -inf on ~15% of
    the (slot-head[, key]) entries and -1e4 (e^ell = 0 as well) on ~10%; at
    step 3 every entry is -inf, which wipes every state."""
    s = dict(s)
    ld = s["ld"].copy()
    pick = rng.uniform(size=ld.shape)
    ld[pick < 0.15] = -np.inf
    ld[(pick >= 0.15) & (pick < 0.25)] = -1e4
    if t == 3:
        ld[...] = -np.inf
    s["ld"] = ld
    return s


@needs_gpu
@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
@pytest.mark.parametrize("path", ["fused", "staged", "eager", "per-slot"])
def test_full_decay(orc, op, path):
    """Full forgetting (log-decay -inf) and extreme finite decays inside the
    log: the steps after a wipe replay entries whose decays are differences
    of cumulative log-decays.  M=4, 14 steps, then a forced merge; every
    output and every merged base against the eager oracle, all finite."""
    w = synth.Workload(22, op, 2, 3, 64, 64, 4, 14, "bf16")
    rng = np.random.default_rng(22)
    if path != "per-slot":
        run = ParityRun(w, eager=path == "eager", orc=orc)
        for t in range(w.steps):
            run.step(_with_full_decay(synth.step(w, t), t, rng), staged=path == "staged")
        if path != "eager":
            run.merge()
        _report(run, f"full decay {op} {path}")
        run.close()
        return
    import recurrent_state_update_amd as rsu
    X0, u = synth.initial(w)
    BH = w.B * w.H
    st = rsu.DeltaLogState(op, w.B, w.H, 64, 64, w.M, dtype=torch.bfloat16, base=dev(X0), u=dev(u))
    st.enable_slots()
    X = X0.reshape(BH, 64, 64).astype(np.float64)[None].copy()
    u_sub = None if u is None else u[np.arange(BH) % w.H].astype(np.float64)
    worst = 0.0
    for t in range(w.steps):
        if t == 2:  # slot 1 restarts from a fresh seeded state: the slots' logs fall out of step
            new = synth.initial(w.with_(wid=2200))[0][1]
            st.base[1].copy_(dev(new))
            st.admit(1)
            X[0, w.H:2 * w.H] = new.astype(np.float64)
        s = _with_full_decay(synth.step(w, t), t, rng)
        d_ = {k_: dev(v_, torch.bfloat16 if k_ in ("q", "k", "v") else torch.float32)
              for k_, v_ in s.items()}
        o = st.step(d_["q"], d_["k"], d_["v"], d_["beta"], d_["ld"])
        sub = synth.subset(s, np.arange(BH))
        o_ref = orc.eager_step(op, X, sub["q"], sub["k"], sub["v"], sub["beta"], sub["ld"], u_sub)
        worst = max(worst, rel(o.reshape(BH, 64).cpu().numpy(), o_ref[0]))
    st.merge()
    worst_S = rel(st.base.reshape(BH, 64, 64).cpu().numpy(), X[0])
    st.close()
    print(f"[full decay {op} per-slot] worst o={worst:.2e} S={worst_S:.2e}", flush=True)
    assert worst < FP32_TOL and worst_S < FP32_TOL


@needs_gpu
@pytest.mark.parametrize("op", ["gdn", "rwkv6"])
def test_inputs_may_alias(orc, op):
    """Read-only inputs may share memory: q and k passed as the same buffer
    (o_t then reads the state with the key it was just written with). M=4,
    9 steps, the eager oracle fed the same aliased inputs."""
    w = synth.Workload(23, op, 2, 3, 64, 64, 4, 9, "bf16")
    run = ParityRun(w, orc=orc)
    for t in range(w.steps):
        run.step(alias_qk=True)
    run.merge()
    _report(run, f"q aliases k, {op}")
    run.close()


@needs_gpu
def test_concurrent_handles_on_separate_streams(orc):
    """Two handles (GDN and KDA) stepped at the same time from two host
    threads, each on its own stream (default priority): the library keeps no
    state outside its handles, so both runs match the oracle.  M=4, 10 steps
    each, then a merge; every output and both merged bases."""
    import threading
    import recurrent_state_update_amd as rsu
    jobs = [("gdn", 24), ("kda", 25)]
    results, errors = {}, []

    def worker(i, op, wid):
        try:
            w = synth.Workload(wid, op, 2, 3, 64, 64, 4, 10, "bf16")
            stream = torch.cuda.Stream()
            with torch.cuda.stream(stream):
                X0, u = synth.initial(w)
                base = dev(X0)
                st = rsu.DeltaLogState(op, w.B, w.H, 64, 64, w.M, dtype=torch.bfloat16, base=base,
                                       u=dev(u))
                outs = []
                for t in range(w.steps):
                    s = synth.step(w, t)
                    d_ = {k_: dev(v_, torch.bfloat16 if k_ in ("q", "k", "v") else torch.float32)
                          for k_, v_ in s.items()}
                    outs.append(st.step(d_["q"], d_["k"], d_["v"], d_["beta"], d_["ld"]).clone())
                st.merge()
            stream.synchronize()
            results[i] = (w, X0, [o.cpu().numpy() for o in outs], base.cpu().numpy())
            st.close()
        except Exception as exc:  # re-raised in the main thread
            errors.append(exc)

    threads = [threading.Thread(target=worker, args=(i, op, wid)) for i, (op, wid) in enumerate(jobs)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    if errors:
        raise errors[0]
    for i, (op, _) in enumerate(jobs):
        w, X0, outs, base = results[i]
        BH = w.B * w.H
        X = X0.reshape(BH, 64, 64).astype(np.float64)[None].copy()
        worst = 0.0
        for t in range(w.steps):
            sub = synth.subset(synth.step(w, t), np.arange(BH))
            o_ref = orc.eager_step(op, X, sub["q"], sub["k"], sub["v"], sub["beta"], sub["ld"], None)
            worst = max(worst, rel(outs[t].reshape(BH, 64), o_ref[0]))
        worst_S = rel(base.reshape(BH, 64, 64), X[0])
        print(f"[concurrent {op}] worst o={worst:.2e} S={worst_S:.2e}", flush=True)
        assert worst < FP32_TOL and worst_S < FP32_TOL


@needs_gpu
@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
@pytest.mark.parametrize("path", ["fused", "staged"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_longest_log_at_d128(orc, op, path, dtype):
    """The largest LDS footprint a lockstep launch has: M=32 at d_k=d_v=128
    (a 32-entry fold table and value shard per tile; the log shard takes a
    second staging pass and the coefficients a per-wave loop past the first
    8 entries).  Two merge cycles plus 5 steps, then a forced merge."""
    w = synth.Workload(26, op, 2, 3, 128, 128, 32, 69, dtype)
    run = ParityRun(w, orc=orc)
    for _ in range(w.steps):
        run.step(staged=path == "staged")
    run.merge()
    _report(run, f"{op} M=32 d=128 {path} {dtype}")
    run.close()


@needs_gpu
@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
def test_checkpoint_restore_per_slot(orc, op):
    """Checkpoint of a handle with per-slot logs: dl_merge folds every active
    slot's log (all logs empty, released slots untouched); a new handle over
    a copy of the base, with per-slot logs enabled and the same slots
    released, then continues bit-identically to the original, through
    admissions and each slot's own merges.  Both match the oracle."""
    import recurrent_state_update_amd as rsu
    B, H, M = 4, 2, 4
    w = synth.Workload(27, op, B, H, 64, 64, M, 15, "bf16")
    X0, u = synth.initial(w)
    dt = in_dtype(w)
    a = rsu.DeltaLogState(op, B, H, 64, 64, M, dtype=dt, base=dev(X0), u=dev(u))
    a.enable_slots()
    X = X0.reshape(B * H, 64, 64).astype(np.float64)[None].copy()
    u_sub = None if u is None else u[np.arange(B * H) % H].astype(np.float64)

    def inputs(t):
        s = synth.step(w, t)
        return s, (dev(s["q"], dt), dev(s["k"], dt), dev(s["v"], dt), dev(s["beta"]), dev(s["ld"]))

    def fresh(b, t):  # a new request's seeded initial state for slot b
        return synth.initial(w.with_(wid=2700 + 10 * t + b))[0][b]

    def oracle_step(s):
        sub = synth.subset(s, np.arange(B * H))
        return orc.eager_step(op, X, sub["q"], sub["k"], sub["v"], sub["beta"], sub["ld"], u_sub)[0]

    worst = 0.0
    for t in range(6):           # slot 1 admitted late, slot 3 released: logs out of step
        if t == 2:
            new = fresh(1, t)
            a.base[1].copy_(dev(new))
            a.admit(1)
            X[0, H:2 * H] = new.astype(np.float64)
        if t == 3:
            a.release(3)
        s, d_ = inputs(t)
        o = a.step(*d_).reshape(B * H, 64).cpu().numpy()
        o_ref = oracle_step(s)
        live = np.arange(B * H) < 3 * H if t >= 3 else np.ones(B * H, bool)
        worst = max(worst, rel(o[live], o_ref[live]))
    a.merge()                    # the checkpoint: every active slot's log is empty
    b = rsu.DeltaLogState(op, B, H, 64, 64, M, dtype=dt, base=a.base.clone(), u=dev(u))
    b.enable_slots()
    b.release(3)
    for t in range(6, w.steps):
        if t == 9:               # a new request in the released slot, on both handles
            new = fresh(3, t)
            a.base[3].copy_(dev(new))
            b.base[3].copy_(dev(new))
            a.admit(3)
            b.admit(3)
            X[0, 3 * H:] = new.astype(np.float64)
        s, d_ = inputs(t)
        # zeroed outputs: a released slot's rows are left as they are
        oa = a.step(*d_, o=torch.zeros(B, H, 64, device="cuda"))
        ob = b.step(*d_, o=torch.zeros(B, H, 64, device="cuda"))
        assert torch.equal(oa, ob), (op, t)
        o_ref = oracle_step(s)
        live = np.arange(B * H) < 3 * H if t < 9 else np.ones(B * H, bool)
        worst = max(worst, rel(ob.reshape(B * H, 64).cpu().numpy()[live], o_ref[live]))
    a.merge()
    b.merge()
    assert torch.equal(a.base, b.base)
    worst_S = rel(b.base.reshape(B * H, 64, 64).cpu().numpy(), X[0])
    a.close()
    b.close()
    print(f"[checkpoint per-slot {op}] worst o={worst:.2e} S={worst_S:.2e}", flush=True)
    assert worst < FP32_TOL and worst_S < FP32_TOL


@needs_gpu
@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
@pytest.mark.parametrize("path", ["fused", "staged"])
def test_full_decay_long_log(orc, op, path):
    """Repeated full forgetting within one long log (M=32): 30% of the
    (slot-head[, key]) entries take log-decay -inf at every step, so the
    cumulative decays reach many times the floor before a merge and the
    entries appended after a wipe take their decays as differences of large
    numbers.  70 steps (two merges), then a forced merge."""
    w = synth.Workload(28, op, 2, 3, 64, 64, 32, 70, "bf16")
    rng = np.random.default_rng(28)
    run = ParityRun(w, orc=orc)
    for t in range(w.steps):
        s = dict(synth.step(w, t))
        ld = s["ld"].copy()
        ld[rng.uniform(size=ld.shape) < 0.3] = -np.inf
        s["ld"] = ld
        run.step(s, staged=path == "staged")
    run.merge()
    _report(run, f"full decay, long log, {op} {path}")
    run.close()


def _wipe_schedule(w):
    """Deterministic repeated full forgetting in an M=32 log, one pattern per
    slot-head (steps t of each 32-step cycle wiped with a log-decay of -inf:
    key 0 for KDA/RWKV6, the whole head for GDN):
      slot-head 0: t = 0..30 (every append step of the cycle; the merge step
                   decays normally),
      slot-heads 1, 2, 3: t < 24, 16, 8, then ordinary decays (cumulative
                   snapshots would lose the later decays' low bits here),
      slot-head 4: every other step,
      slot-head 5: no wipe.
    q and k put most of their weight on key 0, so the output follows that
    key's decay factors."""
    pats = [lambda t: t < 31, lambda t: t < 24, lambda t: t < 16, lambda t: t < 8,
            lambda t: t % 2 == 0, lambda t: False]
    steps = []
    for t in range(w.steps):
        s = {k_: (None if v_ is None else v_.copy()) for k_, v_ in synth.step(w, t).items()}
        BH = w.BH
        for name in ("q", "k"):
            x = s[name].reshape(BH, w.dk)
            x[:, 0] = 4.0 * np.sign(x[:, 0] + 1e-3)
            if w.op != "rwkv6":
                x /= np.linalg.norm(x, axis=1, keepdims=True)
            s[name] = synth.round_bf16(x.reshape(w.B, w.H, w.dk))
        ld = s["ld"].reshape(BH, -1)
        for sh in range(BH):
            if pats[sh % len(pats)](t % w.M):
                ld[sh, 0 if w.op != "gdn" else slice(None)] = -np.inf
        s["ld"] = ld.reshape(s["ld"].shape)
        steps.append(s)
    return steps


@needs_gpu
@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
@pytest.mark.parametrize("path", ["fused", "staged", "per-slot"])
def test_repeated_full_forgetting_worst_case(orc, op, path):
    """Up to 31 full-forgetting steps of one key (one head for GDN) inside one
    M=32 log, followed by ordinary decays, two cycles: every output and both
    merged states match the oracle at the fp32 bar, per slot-head (the
    factors are sums of the logged decays, so the wipes cost no precision)."""
    import recurrent_state_update_amd as rsu
    w = synth.Workload(77, op, 2, 3, 64, 64, 32, 64, "bf16")
    steps = _wipe_schedule(w)
    X0, u = synth.initial(w)
    dt = torch.bfloat16
    base = dev(X0)
    st = rsu.DeltaLogState(op, w.B, w.H, w.dk, w.dv, w.M, dtype=dt, base=base, u=dev(u))
    if path == "per-slot":
        st.enable_slots()
    X = X0.reshape(1, w.BH, w.dk, w.dv).astype(np.float64).copy()
    u_sub = None if u is None else u[np.arange(w.BH) % w.H].astype(np.float64)
    worst_o = worst_S = 0.0
    merges = 0
    for t, s in enumerate(steps):
        d_ = {k_: dev(v_, dt if k_ in ("q", "k", "v") else torch.float32) for k_, v_ in s.items()}
        if path == "staged":
            st.replay_prep(d_["q"], d_["k"], d_["ld"])
            o = st.append_decode(d_["q"], d_["k"], d_["v"], d_["beta"])
        else:
            o = st.step(d_["q"], d_["k"], d_["v"], d_["beta"], d_["ld"])
        sub = synth.subset(s, np.arange(w.BH))
        o_ref = orc.eager_step(op, X, sub["q"], sub["k"], sub["v"], sub["beta"], sub["ld"], u_sub)[0]
        worst_o = max(worst_o, rel(o.reshape(w.BH, w.dv).cpu().numpy(), o_ref))
        if (t + 1) % w.M == 0:
            merges += 1
            worst_S = max(worst_S, rel(base.reshape(w.BH, w.dk, w.dv).cpu().numpy(), X[0]))
    print(f"[{op} {path} wipes M=32] worst o={worst_o:.2e} S={worst_S:.2e}", flush=True)
    st.close()
    assert merges == 2
    assert worst_o < FP32_TOL and worst_S < FP32_TOL
