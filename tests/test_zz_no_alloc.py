"""dl_decode_step_staged_noalloc, the two-stage step that allocates nothing
(its per-step replay coefficients live in the library's static device
scratch), against the same step through dl_replay_prep + dl_append_decode on
a twin handle: identical results, call after call, on a large shape followed
by a smaller one, under graph capture, and after out-of-order calls."""
import numpy as np
import pytest
import torch

import synth
from gpu_harness import FP32_TOL, dev, rel

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU")


def _inputs(w, t, dt):
    s = synth.step(w, t)
    return s, {k_: dev(v_, dt if k_ in ("q", "k", "v") else torch.float32) for k_, v_ in s.items()}


def _twins(w, dt):
    import recurrent_state_update_amd as rsu
    X0, u = synth.initial(w)
    a = rsu.DeltaLogState(w.op, w.B, w.H, w.dk, w.dv, w.M, dtype=dt, base=dev(X0), u=dev(u))
    b = rsu.DeltaLogState(w.op, w.B, w.H, w.dk, w.dv, w.M, dtype=dt, base=dev(X0), u=dev(u))
    return a, b, X0, u


def _noalloc(st, d, o):
    import recurrent_state_update_amd as rsu
    return rsu.dl_decode_step_staged_noalloc(st._h, d["q"], d["k"], d["v"], d["beta"], d["ld"], o)


@needs_gpu
@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
def test_noalloc_matches_two_stage_large_then_small(orc, op):
    """A large shape (B*H = 15872 at M = 32: 1,047,552 of the scratch's
    1,048,576 floats; 40 calls, one merge and 8 pending entries), then a
    smaller one (a few slot-heads, M = 3, 7 calls), each call checked against
    the two-stage path bit for bit (o, and the base after every merge) and
    the small run also against the oracle."""
    import recurrent_state_update_amd as rsu
    dt = torch.bfloat16
    for w in (synth.Workload(91, op, 124, 128, 16, 32, 32, 40, "bf16"),
              synth.Workload(92, op, 2, 3, 64, 64, 3, 7, "bf16")):
        a, b, X0, u = _twins(w, dt)
        X = X0.reshape(1, w.BH, w.dk, w.dv).astype(np.float64).copy()
        u_sub = None if u is None else u[np.arange(w.BH) % w.H].astype(np.float64)
        worst = 0.0
        for t in range(w.steps):
            s, d = _inputs(w, t, dt)
            o = torch.full((w.B, w.H, w.dv), float("nan"), device="cuda")
            assert _noalloc(a, d, o) == 0
            b.replay_prep(d["q"], d["k"], d["ld"])
            ob = b.append_decode(d["q"], d["k"], d["v"], d["beta"])
            torch.cuda.synchronize()
            assert a.log_len == b.log_len == (t + 1) % w.M
            assert torch.equal(o, ob), (op, w.describe(), t)
            if a.log_len == 0:
                assert torch.equal(a.base, b.base), (op, w.describe(), t)
            if w.BH <= 64:
                sub = synth.subset(s, np.arange(w.BH))
                o_ref = orc.eager_step(op, X, sub["q"], sub["k"], sub["v"], sub["beta"], sub["ld"], u_sub)[0]
                worst = max(worst, rel(o.reshape(w.BH, w.dv).cpu().numpy(), o_ref))
        a.merge()
        b.merge()
        torch.cuda.synchronize()
        assert torch.equal(a.base, b.base)
        a.close()
        b.close()
        print(f"[noalloc {op} {w.describe()}] identical to the two-stage path; worst vs oracle {worst:.2e}",
              flush=True)
        assert worst < FP32_TOL


@needs_gpu
@pytest.mark.parametrize("op", ["gdn", "kda"])
def test_noalloc_under_graph_capture(op):
    """One merge cycle of the no-alloc call captured in a HIP graph and
    replayed twice with fresh inputs copied into the captured buffers (eager
    work and synchronisations between the replays): every replay equals the
    two-stage path run directly, bit for bit."""
    dt = torch.bfloat16
    w = synth.Workload(93, op, 8, 4, 128, 128, 4, 8, "bf16")
    a, b, _, _ = _twins(w, dt)
    static = [_inputs(w, t, dt)[1] for t in range(w.M)]
    outs = [torch.empty(w.B, w.H, w.dv, device="cuda") for _ in range(w.M)]
    # the first call on a device looks up the scratch address: do it outside
    # the capture, as a serving loop would before capturing
    s0, d0 = _inputs(w, 100, dt)
    assert _noalloc(a, d0, outs[0]) == 0
    b.replay_prep(d0["q"], d0["k"], d0["ld"])
    b.append_decode(d0["q"], d0["k"], d0["v"], d0["beta"])
    a.merge()
    b.merge()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for t in range(w.M):
            assert _noalloc(a, static[t], outs[t]) == 0
    assert a.log_len == 0
    for rep in range(2):
        fresh = [_inputs(w, 10 * (rep + 1) + t, dt)[1] for t in range(w.M)]
        for t in range(w.M):
            for k_, v_ in fresh[t].items():
                if v_ is not None:
                    static[t][k_].copy_(v_)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t in range(w.M):
            f = fresh[t]
            b.replay_prep(f["q"], f["k"], f["ld"])
            ob = b.append_decode(f["q"], f["k"], f["v"], f["beta"])
            torch.cuda.synchronize()
            assert torch.equal(outs[t], ob), (op, rep, t)
        assert torch.equal(a.base, b.base), (op, rep)
    a.close()
    b.close()


@needs_gpu
def test_noalloc_call_order():
    """The no-alloc call refuses to run between dl_replay_prep and
    dl_append_decode, and on a handle with per-slot logs (DL_E_STATE), and
    leaves the handle usable."""
    import recurrent_state_update_amd as rsu
    dt = torch.bfloat16
    w = synth.Workload(94, "gdn", 2, 2, 32, 32, 4, 2, "bf16")
    a, b, _, _ = _twins(w, dt)
    _, d = _inputs(w, 0, dt)
    o = torch.empty(w.B, w.H, w.dv, device="cuda")
    a.replay_prep(d["q"], d["k"], d["ld"])
    assert _noalloc(a, d, o) == 5
    a.append_decode(d["q"], d["k"], d["v"], d["beta"])
    assert _noalloc(a, d, o) == 0 and a.log_len == 2
    b.enable_slots()
    assert _noalloc(b, d, o) == 5
    torch.cuda.synchronize()
    a.close()
    b.close()
