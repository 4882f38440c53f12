"""GPU checks of the synthetic multi-layer decode harness (bench_decoder.py).

1. Parity: with fp32 weights and activations, every token's output of the
   harness on both state paths (DeltaLog, eager) matches a CPU model in fp64
   that uses the oracle's eager recurrence for the state step and numpy for
   the stand-in layers, written here from the harness's stated formulas.
2. Graph replay: a captured merge cycle, replayed three times with unrelated
   eager GPU work and synchronisations in between, gives the same outputs as
   running the same tokens directly.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_harness import FP32_TOL, rel

pytestmark = pytest.mark.gpu
needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU")

EPS = 1e-6
DECAY_SHIFT = 3.0


def _rms(x):
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + EPS)


def _heads(t):
    return t / np.sqrt(np.sum(t * t, axis=-1, keepdims=True) + t.shape[-1] * EPS)


class CpuDecoder:
    """fp64 model of the harness: RMS norm, projection, per-head prep, the
    oracle's eager step, output projection, gated MLP, residuals."""

    def __init__(self, ds, orc):
        self.ds, self.orc = ds, orc
        self.p = []
        for l in range(ds.L):
            p = synth.decoder_layer(ds, l)
            self.p.append({k: None if v is None else v.astype(np.float64) for k, v in p.items()})

    def token(self, x):
        ds = self.ds
        B, H = ds.B, ds.H
        cuts = np.cumsum(ds.proj_split)[:-1]
        for p in self.p:
            q, k, v, zb, zd = np.split(_rms(x) @ p["W_in"], cuts, axis=1)
            q, k, v = q.reshape(B, H, ds.dk), k.reshape(B, H, ds.dk), v.reshape(B, H, ds.dv)
            if ds.op != "rwkv6":
                q, k = _heads(q), _heads(k)
                beta = 1.0 / (1.0 + np.exp(-zb))
            else:
                beta = None
            ld = -np.logaddexp(0.0, zd - DECAY_SHIFT)
            ld = ld.reshape(B, H) if ds.op == "gdn" else ld.reshape(B, H, ds.dk)
            o = self.orc.eager_step(ds.op, p["X0"], q, k, v, beta, ld, p["u"])  # X0 evolves in place
            x = x + o.reshape(B, H * ds.dv) @ p["W_o"]
            gu = _rms(x) @ p["W_gu"]
            g, u = gu[:, :ds.ffn], gu[:, ds.ffn:]
            x = x + (g / (1.0 + np.exp(-g)) * u) @ p["W_dn"]
        return x, _rms(x)


def _shape(op, M=4):
    return synth.DecoderShape(op, L=2, B=2, H=2, dk=32, dv=64, M=M, hidden=64, ffn=96, seed=3)


@needs_gpu
@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
@pytest.mark.parametrize("path", ["deltalog", "eager"])
def test_decoder_matches_cpu_model(orc, op, path):
    from bench_decoder import SyntheticDecoder
    ds = _shape(op)
    dec = SyntheticDecoder(ds, path, torch.float32)
    ref = CpuDecoder(ds, orc)
    x_ref = synth.decoder_input(ds).astype(np.float64)
    x = torch.from_numpy(synth.decoder_input(ds)).cuda()
    worst = 0.0
    for _ in range(2 * ds.M + 1):          # two merges and a pending log
        out, x = dec.token(x)
        out_ref, x_ref = ref.token(x_ref)
        worst = max(worst, rel(out.cpu().numpy(), out_ref))
    worst_S = 0.0
    for lay, p in zip(dec.layers, ref.p):
        if path == "deltalog":
            lay["st"].merge()
        worst_S = max(worst_S, rel(lay["base"].cpu().numpy(), p["X0"]))
    print(f"[decoder {op} {path}] worst out={worst:.2e} state={worst_S:.2e}", flush=True)
    dec.close()
    assert worst < FP32_TOL and worst_S < FP32_TOL


@needs_gpu
@pytest.mark.parametrize("op", ["gdn", "rwkv6"])
def test_decoder_graph_replays_match_direct(op):
    from bench_decoder import SyntheticDecoder, warm_up
    ds = _shape(op, M=3)
    direct = SyntheticDecoder(ds, "deltalog", torch.float32)
    graphed = SyntheticDecoder(ds, "deltalog", torch.float32, weights_from=direct)
    x0 = torch.from_numpy(synth.decoder_input(ds)).cuda()
    want = []
    x = x0.clone()
    for _ in range(ds.M):
        _, x = direct.token(x)
    for _ in range(3 * ds.M):
        out, x = direct.token(x)
        want.append(out.clone())
    xs = warm_up(graphed, x0.clone(), ds.M)
    g, outs = graphed.capture_cycle(xs)
    junk = torch.randn(256, 256, device="cuda")
    worst = 0.0
    for r in range(3):
        g.replay()
        torch.cuda.synchronize()
        for t in range(ds.M):
            worst = max(worst, rel(outs[t].cpu().numpy(), want[r * ds.M + t].cpu().numpy()))
        junk = (junk @ junk).tanh_()          # unrelated eager work between replays
        torch.cuda.synchronize()
    print(f"[decoder graph {op}] worst replay vs direct = {worst:.2e}", flush=True)
    direct.close()
    graphed.close()
    assert worst < 1e-5
