"""The C ABI driven from a plain C program (tests/c_client.c, built by
__graft_entry__.build()): device memory from hipMalloc, raw pointers into
dl_state_create / dl_decode_step / dl_merge, no Python or torch on the GPU
side.  Its outputs and merged base are checked against the oracle."""
import os
import subprocess

import numpy as np
import pytest

import synth
from gpu_harness import FP32_TOL, rel

pytestmark = pytest.mark.gpu
HERE = os.path.dirname(os.path.abspath(__file__))
CLIENT = os.path.join(HERE, "c_client")


def _has_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.mark.skipif(not _has_gpu(), reason="no GPU")
@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
def test_c_client_matches_oracle(orc, tmp_path, op):
    if not os.path.exists(CLIENT):
        pytest.fail("tests/c_client is not built; run __graft_entry__.build()")
    w = synth.Workload(24, op, 2, 3, 32, 64, 3, 7, "f32")
    X0, u = synth.initial(w)
    steps = [synth.step(w, t) for t in range(w.steps)]
    inp = tmp_path / "in.bin"
    with open(inp, "wb") as f:
        np.array([synth.OP_IDS[op], w.B, w.H, w.dk, w.dv, w.M, w.steps], np.int32).tofile(f)
        X0.astype(np.float32).tofile(f)
        if u is not None:
            u.astype(np.float32).tofile(f)
        for s in steps:
            for key in ("q", "k", "v", "beta", "ld"):
                if s[key] is not None:
                    s[key].astype(np.float32).tofile(f)
    out = tmp_path / "out.bin"
    r = subprocess.run([CLIENT, str(inp), str(out)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    got = np.fromfile(out, np.float32)
    n_o = w.steps * w.BH * w.dv
    o_gpu = got[:n_o].reshape(w.steps, w.B, w.H, w.dv)
    base_gpu = got[n_o:].reshape(w.B, w.H, w.dk, w.dv)
    X = X0.astype(np.float64)
    worst = 0.0
    for t, s in enumerate(steps):
        o_ref = orc.eager_step(op, X, s["q"], s["k"], s["v"], s["beta"], s["ld"], u)
        worst = max(worst, rel(o_gpu[t], o_ref))
    worst_S = rel(base_gpu, X)
    print(f"[c client {op}] worst o={worst:.2e} S={worst_S:.2e}", flush=True)
    assert worst < FP32_TOL and worst_S < FP32_TOL
