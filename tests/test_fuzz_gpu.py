"""Seeded randomized parity on the GPU.  Each case draws the operator, d_k,
d_v, M in [1, 32], B and H (small, ragged), the input dtype and the path
(one-launch, two-stage, eager, or per-slot logs), a run length, and a
sequence of schedule events:
- lockstep paths: forced merges at random steps;
- per-slot logs: random admissions (fresh seeded states), early merges of
  one slot, and releases.

Every output of a live slot is checked against the fp64 eager oracle on the
same inputs; so is every base that a merge makes observable (forced merges,
slot merges, the final merge).  Bar: the fp32 bound FP32_TOL."""
import os

import numpy as np
import pytest
import torch

import synth
from gpu_harness import FP32_TOL, ParityRun, dev, in_dtype, rel

pytestmark = pytest.mark.gpu
needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU")

# cases [FIRST, FIRST + N_CASES); a wider sweep: DL_FUZZ_FIRST=1000 DL_FUZZ_CASES=1000
FIRST = int(os.environ.get("DL_FUZZ_FIRST", "0"))
N_CASES = int(os.environ.get("DL_FUZZ_CASES", "48"))
PATHS = ("fused", "staged", "eager", "per-slot")


def draw(i: int):
    rng = np.random.default_rng([4242, i])
    op = ("gdn", "kda", "rwkv6")[int(rng.integers(3))]
    dk, dv = (int(x) for x in rng.choice([16, 32, 64, 128], size=2))
    M = int(rng.integers(1, 33))
    B, H = int(rng.integers(1, 10)), int(rng.integers(1, 8))
    dtype = ("bf16", "f32")[int(rng.integers(2))]
    path = PATHS[i % len(PATHS)]          # every path equally often
    steps = int(rng.integers(1, min(3 * M + 3, 60) + 1))
    w = synth.Workload(5000 + i, op, B, H, dk, dv, M, steps, dtype)
    return w, path, rng


def _lockstep(w, path, rng, orc):
    run = ParityRun(w, eager=path == "eager", orc=orc)
    for _ in range(w.steps):
        if path != "eager" and rng.uniform() < 0.1:
            run.merge()                   # forced merge at whatever length the log has
        run.step(staged=path == "staged")
    if path != "eager":
        run.merge()
    run.close()
    return run.worst_o, run.worst_S


def _per_slot(w, rng, orc):
    import recurrent_state_update_amd as rsu
    B, H, dk, dv, BH = w.B, w.H, w.dk, w.dv, w.BH
    X0, u = synth.initial(w)
    dt = in_dtype(w)
    st = rsu.DeltaLogState(w.op, B, H, dk, dv, w.M, dtype=dt, base=dev(X0), u=dev(u))
    st.enable_slots()
    X = X0.reshape(BH, dk, dv).astype(np.float64)[None].copy()
    u_sub = None if u is None else u[np.arange(BH) % H].astype(np.float64)
    active = np.ones(B, bool)
    rows = lambda b: slice(b * H, (b + 1) * H)
    worst_o = worst_S = 0.0

    def check_slot(b):
        return rel(st.base[b].cpu().numpy(), X[0, rows(b)])

    for t in range(w.steps):
        ev, b = rng.uniform(), int(rng.integers(B))
        if ev < 0.15:                      # a new request in slot b
            new = synth.initial(w.with_(wid=w.wid * 100 + t))[0][b]
            st.base[b].copy_(dev(new))
            st.admit(b)
            X[0, rows(b)] = new.astype(np.float64)
            active[b] = True
        elif ev < 0.25 and active[b]:      # fold slot b's log now
            st.merge_slot(b)
            worst_S = max(worst_S, check_slot(b))
        elif ev < 0.32 and active[b] and active.sum() > 1:   # slot b's request ends
            st.merge_slot(b)
            worst_S = max(worst_S, check_slot(b))
            st.release(b)
            active[b] = False
        s = synth.step(w, t)
        d_ = {k_: dev(v_, dt if k_ in ("q", "k", "v") else torch.float32) for k_, v_ in s.items()}
        o = st.step(d_["q"], d_["k"], d_["v"], d_["beta"], d_["ld"],
                    o=torch.zeros(B, H, dv, device="cuda")).reshape(BH, dv).cpu().numpy()
        sub = synth.subset(s, np.arange(BH))
        o_ref = orc.eager_step(w.op, X, sub["q"], sub["k"], sub["v"], sub["beta"], sub["ld"], u_sub)[0]
        live = np.repeat(active, H)
        worst_o = max(worst_o, rel(o[live], o_ref[live]))
    st.merge()
    for b in np.flatnonzero(active):
        worst_S = max(worst_S, check_slot(b))
    st.close()
    return worst_o, worst_S


@needs_gpu
@pytest.mark.parametrize("i", range(FIRST, FIRST + N_CASES))
def test_random_case(orc, i):
    w, path, rng = draw(i)
    print(f"[fuzz {i}] {w.describe()} {path}", flush=True)
    if path == "per-slot":
        worst_o, worst_S = _per_slot(w, rng, orc)
    else:
        worst_o, worst_S = _lockstep(w, path, rng, orc)
    print(f"[fuzz {i}] worst o={worst_o:.2e} S={worst_S:.2e}", flush=True)
    assert worst_o < FP32_TOL and worst_S < FP32_TOL
