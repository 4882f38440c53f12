"""Shared driver for the GPU parity tests: runs the HIP path through the C ABI
on seeded synthetic workloads and the fp64 oracle on the same inputs, and
compares them.

Error metric: for each output tensor and step, and for each slot-head on its
own, max|x - ref| / max|ref| (the max-abs relative error of that slot-head's
output or state), then the worst slot-head.  The pages' accuracy bar is a
maximum output relative error below 5e-3 (the "Numerical correctness" item of
the gist.science summary's results).
"""
from __future__ import annotations

import numpy as np
import torch

import synth
from oracle import Oracle

PAGES_TOL = 5e-3
# fp32 arithmetic bound used as the tighter regression bar (derivation in the
# design notes): dot products of length <= 128 with fp32 accumulation and
# contractive decays keep the relative error near 1e-6; 2e-4 leaves margin.
FP32_TOL = 2e-4


def rel(x, ref) -> float:
    """Max-abs relative error, normalised per unit: x and ref are [units, ...]
    with the leading axis indexing the compared units (slot-heads, or slots),
    and the result is the max over units of max|x_u - ref_u| / max|ref_u|.  A
    unit whose reference is all zero is measured against the largest |ref| of
    the whole array.  So a unit with small values (a state just wiped by a
    full decay, say) is judged on its own scale, not hidden under a larger
    neighbour's.  inf where x holds a NaN or inf that the reference does not
    (so running maxima, which skip NaN, cannot hide one); non-finite
    reference entries that x matches are left out."""
    x, ref = np.broadcast_arrays(np.asarray(x, np.float64), np.asarray(ref, np.float64))
    fin = np.isfinite(ref)
    if (np.isfinite(x) != fin).any():
        return float("inf")
    if x.ndim < 2:
        x, ref, fin = x.reshape(1, -1), ref.reshape(1, -1), fin.reshape(1, -1)
    x = x.reshape(x.shape[0], -1)
    ref = ref.reshape(ref.shape[0], -1)
    fin = fin.reshape(fin.shape[0], -1)
    if ref.size == 0:
        return 0.0
    diff = np.where(fin, np.abs(x - ref), 0.0)
    mag = np.where(fin, np.abs(ref), 0.0)
    den = mag.max(axis=1)
    glob = den.max()
    den = np.where(den > 0, den, glob if glob > 0 else 1.0)
    return float(np.max(diff.max(axis=1) / den))


def dev(a, dtype=torch.float32):
    """numpy float32 -> contiguous device tensor (bf16 conversion is exact for
    values the generator already rounded to bf16)."""
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda").to(dtype).contiguous()


def in_dtype(w: synth.Workload):
    return torch.bfloat16 if w.dtype == "bf16" else torch.float32


def sample_slot_heads(BH: int, count: int, seed: int = 7) -> np.ndarray:
    """Deterministic spread of slot-heads: first, last, and a seeded sample."""
    if BH <= count:
        return np.arange(BH)
    rng = np.random.default_rng(seed)
    idx = set(rng.choice(BH, size=count - 2, replace=False).tolist()) | {0, BH - 1}
    return np.array(sorted(idx))


class ParityRun:
    """DeltaLog (or eager) on the GPU next to the eager fp64 oracle, on the
    slot-heads `idx` (all of them by default).  Records the worst errors."""

    def __init__(self, w: synth.Workload, idx=None, eager: bool = False, orc: Oracle | None = None):
        import recurrent_state_update_amd as rsu
        self.rsu = rsu
        self.w = w
        self.eager = eager
        self.orc = orc or Oracle()
        X0, u = synth.initial(w)
        self.idx = np.arange(w.BH) if idx is None else np.asarray(idx)
        self.dt = in_dtype(w)
        self.base = dev(X0)
        self.u_dev = dev(u)
        # oracle works on the sampled slot-heads as one batch row of len(idx) "heads"
        self.X = X0.reshape(w.BH, w.dk, w.dv)[self.idx].astype(np.float64)[None].copy()
        self.u_sub = None if u is None else u[self.idx % w.H].astype(np.float64)
        if not eager:
            self.st = rsu.DeltaLogState(w.op, w.B, w.H, w.dk, w.dv, w.M, dtype=self.dt,
                                        base=self.base, u=self.u_dev)
        self.t = 0
        self.worst_o = 0.0
        self.worst_S = 0.0
        self.checked_S = 0

    def step(self, s: dict | None = None, staged: bool = False, alias_qk: bool = False):
        """One step; with alias_qk, q is passed as k's device buffer (the
        oracle is fed s["k"] for both)."""
        w = self.w
        s = s if s is not None else synth.step(w, self.t)
        if alias_qk:
            s = dict(s, q=s["k"])
        q, k, v = dev(s["q"], self.dt), dev(s["k"], self.dt), dev(s["v"], self.dt)
        if alias_qk:
            q = k
        beta, ld = dev(s["beta"]), dev(s["ld"])
        if self.eager:
            o = self.rsu.eager_step(w.op, self.base, q, k, v, beta, ld, self.u_dev)
        elif staged:
            self.st.replay_prep(q, k, ld)
            o = self.st.append_decode(q, k, v, beta)
        else:
            o = self.st.step(q, k, v, beta, ld)
        sub = synth.subset(s, self.idx)
        o_ref = self.orc.eager_step(w.op, self.X, sub["q"], sub["k"], sub["v"], sub["beta"],
                                    sub["ld"], self.u_sub)
        o_gpu = o.reshape(w.BH, w.dv)[torch.from_numpy(self.idx).to(o.device)].cpu().numpy()
        e = rel(o_gpu, o_ref[0])
        self.worst_o = max(self.worst_o, e)
        self.t += 1
        if self.eager or self.st.log_len == 0:
            self.check_state()
        return e

    def state_gpu(self) -> np.ndarray:
        w = self.w
        b = self.base.reshape(w.BH, w.dk, w.dv)[torch.from_numpy(self.idx).to(self.base.device)]
        return b.cpu().numpy()

    def check_state(self):
        e = rel(self.state_gpu(), self.X[0])
        self.worst_S = max(self.worst_S, e)
        self.checked_S += 1
        return e

    def merge(self):
        self.st.merge()
        assert self.st.log_len == 0
        return self.check_state()

    def close(self):
        if not self.eager:
            self.st.close()
