"""Seeded synthetic workloads for the recurrent-state decode step.

Shared by the tests, the benchmark and the smoke check; used to feed both the
HIP library and the CPU oracle.  It draws random numbers and shapes them into
inputs; it holds none of the decode step's own arithmetic.

Generator: NumPy PCG64 seeded with ``SeedSequence([workload, op, stream])``.
Stream 0 draws the initial state (and RWKV6's bonus u); stream s+1 draws the
inputs of decode step s, so any step can be regenerated on its own.  Within a
step the draw order is q, k, v, beta, log-decay, each as a whole [B,H,...]
tensor.  Values are float32; bf16 inputs are float32 arrays rounded to the
nearest bf16 (ties to even), so the same numbers reach the GPU (as bf16) and
the oracle (as float64).

Workloads (the pages measure "various batch sizes and context lengths"
without naming sizes; these stand in for them):
  0  GDN   B=1   H=2  d=16  M=4  32 steps,   all fp32 (tiny)
  1  GDN   B=64  H=32 d=128 M=8  256 steps,  bf16 q/k/v (serving-shaped)
  2  KDA   B=64  H=32 d=128 M=8  256 steps,  bf16
  3  RWKV6 B=128 H=64 d=64  M=8  256 steps,  bf16
  4  GDN/KDA B=256 H=32 d=128, M in {1,2,4,8,16}, 1024 steps (large batch)
Distributions: state N(0, 0.1) (0.1 is the standard deviation); q,k ~ N(0,1)
L2-normalised per head in fp32 before any bf16 rounding (GDN, KDA); v ~ N(0,1);
beta = sigmoid(N(0,1)); GDN log-decay g = -softplus(N(-3, 0.5)) per head; KDA
log-decay -softplus(N(-3, 0.5)) per key; RWKV6 r,k,v ~ N(0,1) unnormalised,
log-decay -exp(N(-0.5, 0.5)) per key, u ~ N(0, 0.1) of shape [H, d_k].
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

OP_IDS = {"gdn": 0, "kda": 1, "rwkv6": 2}


@dataclass(frozen=True)
class Workload:
    """One synthetic decode workload."""
    wid: int          # workload id, first seed word
    op: str           # "gdn" | "kda" | "rwkv6"
    B: int
    H: int
    dk: int
    dv: int
    M: int
    steps: int
    dtype: str        # "f32" | "bf16" (q, k, v)

    @property
    def BH(self) -> int:
        return self.B * self.H

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    def describe(self) -> str:
        return (f"{self.op} B={self.B} H={self.H} dk={self.dk} dv={self.dv} "
                f"M={self.M} steps={self.steps} {self.dtype}")


WORKLOADS = {
    0: Workload(0, "gdn", 1, 2, 16, 16, 4, 32, "f32"),
    1: Workload(1, "gdn", 64, 32, 128, 128, 8, 256, "bf16"),
    2: Workload(2, "kda", 64, 32, 128, 128, 8, 256, "bf16"),
    3: Workload(3, "rwkv6", 128, 64, 64, 64, 8, 256, "bf16"),
}
SWEEP_MS = (1, 2, 4, 8, 16)


def sweep_workload(op: str, M: int, steps: int = 1024) -> Workload:
    """Large-batch sweep: B=256 H=32 d=128 at merge interval M."""
    assert op in ("gdn", "kda")
    return Workload(4, op, 256, 32, 128, 128, M, steps, "bf16")


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bf16 value (ties to even), kept in float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    r = (u + bias) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def _rng(w: Workload, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([w.wid, OP_IDS[w.op], stream])))


def _normal(rng, shape, loc=0.0, scale=1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    if loc != 0.0:
        x += np.float32(loc)
    return x


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(np.float32(0.0), x).astype(np.float32)


def _l2norm(x: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x.astype(np.float32) ** 2, axis=-1, keepdims=True, dtype=np.float32))
    return (x / np.maximum(n, np.float32(1e-12))).astype(np.float32)


def initial(w: Workload):
    """Initial state S-bar_0 [B,H,dk,dv] float32 and RWKV6's u [H,dk] (else None)."""
    rng = _rng(w, 0)
    X0 = _normal(rng, (w.B, w.H, w.dk, w.dv), 0.0, 0.1)
    u = _normal(rng, (w.H, w.dk), 0.0, 0.1) if w.op == "rwkv6" else None
    return X0, u


def step(w: Workload, s: int) -> dict:
    """Inputs of decode step s: q (r for RWKV6), k [B,H,dk], v [B,H,dv],
    beta [B,H] (None for RWKV6), ld (log-decay) [B,H] or [B,H,dk]; float32."""
    rng = _rng(w, s + 1)
    B, H, dk, dv = w.B, w.H, w.dk, w.dv
    q = _normal(rng, (B, H, dk))
    k = _normal(rng, (B, H, dk))
    v = _normal(rng, (B, H, dv))
    if w.op in ("gdn", "kda"):
        q, k = _l2norm(q), _l2norm(k)
        beta = (1.0 / (1.0 + np.exp(-_normal(rng, (B, H))))).astype(np.float32)
        shape = (B, H) if w.op == "gdn" else (B, H, dk)
        ld = -_softplus(_normal(rng, shape, -3.0, 0.5))
    else:
        beta = None
        ld = -np.exp(_normal(rng, (B, H, dk), -0.5, 0.5)).astype(np.float32)
    if w.dtype == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    return dict(q=q, k=k, v=v, beta=beta, ld=ld.astype(np.float32))


def steps(w: Workload, first: int, count: int) -> dict:
    """Steps [first, first+count) stacked on a leading axis."""
    per = [step(w, s) for s in range(first, first + count)]
    out = {}
    for key in per[0]:
        out[key] = None if per[0][key] is None else np.stack([p[key] for p in per])
    return out


def subset(d: dict, idx: np.ndarray, lead: int = 0) -> dict:
    """Restrict [.., B, H, ...] arrays to flat slot-head indices idx (sorted),
    keeping a [1, len(idx)] batch-head shape.  `lead` leading axes are kept."""
    out = {}
    for key, a in d.items():
        if a is None:
            out[key] = None
            continue
        B, H = a.shape[lead], a.shape[lead + 1]
        flat = a.reshape(a.shape[:lead] + (B * H,) + a.shape[lead + 2:])
        sel = np.take(flat, idx, axis=lead)
        out[key] = sel.reshape(a.shape[:lead] + (1, len(idx)) + a.shape[lead + 2:])
    return out


# ------------------------------------------------------- decoder harness --
@dataclass(frozen=True)
class DecoderShape:
    """A synthetic stack of L recurrent layers around the decode step."""
    op: str
    L: int
    B: int
    H: int
    dk: int
    dv: int
    M: int
    hidden: int
    ffn: int
    seed: int = 0

    def describe(self) -> str:
        return (f"{self.op} L={self.L} B={self.B} H={self.H} dk={self.dk} dv={self.dv} "
                f"M={self.M} hidden={self.hidden} ffn={self.ffn}")

    @property
    def proj_split(self) -> list:
        """Widths of the input projection's column blocks: q (r), k, v, beta
        logits (none for RWKV6), decay logits (per head for GDN, per key else)."""
        H = self.H
        nb = 0 if self.op == "rwkv6" else H
        nd = H if self.op == "gdn" else H * self.dk
        return [H * self.dk, H * self.dk, H * self.dv, nb, nd]


def _drng(ds: DecoderShape, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([1000 + ds.seed, OP_IDS[ds.op], stream])))


def decoder_layer(ds: DecoderShape, layer: int) -> dict:
    """Random weights of one layer, float32, each N(0, 1/fan_in): W_in
    [hidden, sum(proj_split)], W_o [H*dv, hidden], W_gu [hidden, 2*ffn] (gate
    then up), W_dn [ffn, hidden]; RWKV6's u [H, dk] ~ N(0, 0.1) (else None);
    and the layer's initial state [B, H, dk, dv] ~ N(0, 0.1).  Draw order as
    listed, from stream layer+1."""
    rng = _drng(ds, layer + 1)
    n_in = sum(ds.proj_split)
    out = {}
    for name, (fi, fo) in (("W_in", (ds.hidden, n_in)), ("W_o", (ds.H * ds.dv, ds.hidden)),
                           ("W_gu", (ds.hidden, 2 * ds.ffn)), ("W_dn", (ds.ffn, ds.hidden))):
        out[name] = _normal(rng, (fi, fo), 0.0, 1.0 / np.sqrt(fi))
    out["u"] = _normal(rng, (ds.H, ds.dk), 0.0, 0.1) if ds.op == "rwkv6" else None
    out["X0"] = _normal(rng, (ds.B, ds.H, ds.dk, ds.dv), 0.0, 0.1)
    return out


def decoder_input(ds: DecoderShape) -> np.ndarray:
    """The first step's hidden input [B, hidden] ~ N(0, 1), stream 0."""
    return _normal(_drng(ds, 0), (ds.B, ds.hidden))
