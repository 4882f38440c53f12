"""fp64 CPU oracle for the recurrent-state decode step (GDN, KDA, RWKV6).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
CPU-baseline leg of the benchmark, never by the product package.  The
arithmetic lives in ``oracle.c`` (plain C99, fp64, OpenMP over slot-heads);
this module compiles it with gcc when asked and wraps it with ctypes.  The
equations it follows, and the pages they come from, are in that file's header.

Operators are named as on the pages ("Kernel implementation" section of the
gist.science technical summary of DeltaLog): ``gdn`` (per-head scalar decay,
delta rule), ``kda`` (per-key decay, delta rule), ``rwkv6`` (per-key decay, raw
k v^T update with a per-head bonus u).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

OP_IDS = {"gdn": 0, "kda": 1, "rwkv6": 2}

_dp = ctypes.POINTER(ctypes.c_double)


def build(src: str = SRC, out: str = LIB) -> str:
    """Compile the oracle into a shared library with gcc (-O2, OpenMP)."""
    cmd = ["gcc", "-O2", "-std=c99", "-Wall", "-fopenmp", "-shared", "-fPIC",
           "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


def _ptr(a):
    if a is None:
        return None
    assert a.dtype == np.float64 and a.flags["C_CONTIGUOUS"], "oracle takes C-contiguous float64"
    return a.ctypes.data_as(_dp)


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


class Oracle:
    """ctypes wrapper around one build of ``oracle.c``."""

    def __init__(self, path: str | None = None):
        path = path or LIB
        if not os.path.exists(path):
            build(out=path)
        self.path = path
        lib = ctypes.CDLL(path)
        args_step = [ctypes.c_int] * 5 + [_dp] * 8
        lib.orc_eager_step.argtypes = args_step
        lib.orc_eager_step.restype = None
        lib.orc_dl_step.argtypes = [ctypes.c_int] * 7 + [_dp] * 11
        lib.orc_dl_step.restype = ctypes.c_int
        lib.orc_dl_merge.argtypes = [ctypes.c_int] * 6 + [_dp] * 4
        lib.orc_dl_merge.restype = ctypes.c_int
        lib.orc_max_threads.argtypes = []
        lib.orc_max_threads.restype = ctypes.c_int
        lib.orc_set_threads.argtypes = [ctypes.c_int]
        lib.orc_set_threads.restype = None
        self.lib = lib

    # -------------------------------------------------------------- threads --
    def max_threads(self) -> int:
        return int(self.lib.orc_max_threads())

    def set_threads(self, n: int) -> None:
        self.lib.orc_set_threads(int(n))

    # ---------------------------------------------------------------- eager --
    def eager_step(self, op, X, q, k, v, beta, ld, u=None):
        """One eager step on every slot-head; X [B,H,dk,dv] float64 is updated
        in place.  Returns o [B,H,dv]."""
        B, H, dk, dv = X.shape
        q, k, v, beta, ld, u = map(_f64, (q, k, v, beta, ld, u))
        o = np.empty((B, H, dv), np.float64)
        self.lib.orc_eager_step(OP_IDS[op], B, H, dk, dv, _ptr(X), _ptr(q), _ptr(k),
                                _ptr(v), _ptr(beta), _ptr(ld), _ptr(u), _ptr(o))
        return o


class DeltaLogModel:
    """fp64 DeltaLog model: base + bounded log, appends M-1 steps, merges on
    the M-th (the schedule of the "Core mechanism: Base + Log" section)."""

    def __init__(self, oracle: Oracle, op: str, X0, M: int):
        self.o_ = oracle
        self.op = op
        self.M = int(M)
        self.Xb = np.array(X0, dtype=np.float64, order="C", copy=True)
        B, H, dk, dv = self.Xb.shape
        self.a = np.zeros((B, H, M, dk))
        self.b = np.zeros((B, H, M, dv))
        self.L = np.zeros((B, H, M, dk))
        self.n = 0

    def step(self, q, k, v, beta, ld, u=None):
        B, H, dk, dv = self.Xb.shape
        q, k, v, beta, ld, u = map(_f64, (q, k, v, beta, ld, u))
        o = np.empty((B, H, dv), np.float64)
        n = self.o_.lib.orc_dl_step(OP_IDS[self.op], B, H, dk, dv, self.M, self.n,
                                    _ptr(self.Xb), _ptr(self.a), _ptr(self.b), _ptr(self.L),
                                    _ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(ld), _ptr(u),
                                    _ptr(o))
        assert n >= 0
        self.n = n
        return o

    def merge(self):
        B, H, dk, dv = self.Xb.shape
        n = self.o_.lib.orc_dl_merge(B, H, dk, dv, self.M, self.n, _ptr(self.Xb),
                                     _ptr(self.a), _ptr(self.b), _ptr(self.L))
        assert n == 0
        self.n = 0

    def logical_state(self):
        """X = e^{Lam_n} (.)row Xb + sum_j (e^{Lam_n - Lam_j} (.) a_j) b_j^T,
        computed on a copy without touching the model."""
        if self.n == 0:
            return self.Xb.copy()
        Ln = self.L[:, :, self.n - 1, :]
        X = np.exp(Ln)[..., None] * self.Xb
        for j in range(self.n):
            X = X + (np.exp(Ln - self.L[:, :, j, :]) * self.a[:, :, j, :])[..., None] \
                * self.b[:, :, j, None, :]
        return X

    def snapshot(self):
        """Everything that defines the logical state mid-cycle."""
        return dict(Xb=self.Xb.copy(), a=self.a.copy(), b=self.b.copy(), L=self.L.copy(), n=self.n)

    def restore(self, snap):
        self.Xb = snap["Xb"].copy()
        self.a = snap["a"].copy()
        self.b = snap["b"].copy()
        self.L = snap["L"].copy()
        self.n = int(snap["n"])
