"""Synthetic multi-layer decode harness around the recurrent-state step.

    python bench_decoder.py [--op gdn] [--layers 8] [--B 64] [--H 32] [--d 128]
                            [--M 8] [--hidden 2048] [--ffn 4096] [--cycles 8]

The pages find that the state-update kernel's speedup shrinks end to end,
since the rest of a decode step is unchanged ([sum] "Results" and
"Significance"; [abs]).  This harness shows that effect without trained
weights.  It stacks L layers with seeded random weights; per layer and token:

    h  = rms(x)                                 RMS normalisation, no gain
    [q | k | v | zb | zd] = h @ W_in            one input projection
    q, k <- q / sqrt(|q|^2 + d_k 1e-6)          per head (GDN, KDA only)
    beta = sigmoid(zb);  ld = -softplus(zd - 3) per head (GDN) or per key
    o  = state step                             DeltaLog or eager, libdeltalog
    x += o @ W_o
    [g | u] = rms(x) @ W_gu;   x += (silu(g) * u) @ W_dn

and the next token's input is rms of the last layer's output.  There is no
attention layer, expert routing, embedding or sampling: the stand-ins put a
realistic amount of weight streaming between the state steps (which also
keeps the states out of the Infinity Cache) and the small elementwise work of
a decode step.  The projections are plain library GEMMs (torch, hipBLASLt)
and the glue is torch elementwise work; neither belongs to the decode step,
which runs in libdeltalog.

Each path is captured as a HIP graph of one merge cycle (M tokens through all
layers) and replayed.  One JSON line reports tokens/s for both paths, the
end-to-end speedup, the state steps alone (same layers and shapes, also graph
replayed), and the end-to-end speedup Amdahl's law predicts from the eager
path's state-step share.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

EPS = 1e-6
DECAY_SHIFT = 3.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class SyntheticDecoder:
    """L layers of the stand-in model above on cuda:0.  `path` is "deltalog"
    (dl_decode_step on a DeltaLog state per layer) or "eager" (dl_eager_step
    on a dense state per layer).  `wdtype` is the weight and activation
    dtype of the GEMMs and of q, k, v (torch.bfloat16 or torch.float32).
    Layers can share weight tensors with another decoder (`weights_from`)."""

    def __init__(self, ds: synth.DecoderShape, path: str, wdtype, weights_from=None):
        import torch
        import recurrent_state_update_amd as rsu
        assert path in ("deltalog", "eager")
        self.ds, self.path, self.wd = ds, path, wdtype
        self.rsu = rsu
        self.layers = []
        for l in range(ds.L):
            if weights_from is None:
                p = synth.decoder_layer(ds, l)
                # kept as [out, in] (the nn.Linear layout, for which the
                # library GEMM picks a better kernel at decode batch sizes)
                lay = {k: torch.from_numpy(p[k]).cuda().to(wdtype).t().contiguous()
                       for k in ("W_in", "W_o", "W_gu", "W_dn")}
                lay["u"] = None if p["u"] is None else torch.from_numpy(p["u"]).cuda()
                lay["X0"] = p["X0"]
            else:
                src = weights_from.layers[l]
                lay = {k: src[k] for k in ("W_in", "W_o", "W_gu", "W_dn", "u", "X0")}
            lay["base"] = torch.from_numpy(lay["X0"]).cuda()
            if path == "deltalog":
                lay["st"] = rsu.DeltaLogState(ds.op, ds.B, ds.H, ds.dk, ds.dv, ds.M, dtype=wdtype,
                                              base=lay["base"], u=lay["u"])
            self.layers.append(lay)

    def _norm_heads(self, t, d):
        import torch.nn.functional as F
        # t / sqrt(|t|^2 + d*EPS) == rms_norm(t, eps=EPS) / sqrt(d)
        return F.rms_norm(t, (d,), eps=EPS) * (1.0 / d ** 0.5)

    def layer_inputs(self, x, lay):
        """Projection and per-head prep of one layer: q, k, v in the input
        dtype, beta and ld in fp32, shaped as the decode step takes them."""
        import torch
        import torch.nn.functional as F
        ds = self.ds
        B, H = ds.B, ds.H
        h = F.rms_norm(x, (ds.hidden,), eps=EPS).to(self.wd)
        p = F.linear(h, lay["W_in"]).float()
        q, k, v, zb, zd = torch.split(p, ds.proj_split, dim=1)
        q = q.reshape(B, H, ds.dk)
        k = k.reshape(B, H, ds.dk)
        if ds.op != "rwkv6":
            q, k = self._norm_heads(q, ds.dk), self._norm_heads(k, ds.dk)
            beta = torch.sigmoid(zb).contiguous()
        else:
            beta = None
        ld = -F.softplus(zd - DECAY_SHIFT)
        ld = ld.reshape(B, H) if ds.op == "gdn" else ld.reshape(B, H, ds.dk)
        return (q.to(self.wd).contiguous(), k.to(self.wd).contiguous(),
                v.reshape(B, H, ds.dv).to(self.wd).contiguous(), beta, ld.contiguous())

    def state_step(self, lay, q, k, v, beta, ld):
        if self.path == "deltalog":
            return lay["st"].step(q, k, v, beta, ld)
        return self.rsu.eager_step(self.ds.op, lay["base"], q, k, v, beta, ld, lay["u"])

    def token(self, x):
        """One token through all layers.  x [B, hidden] fp32.  Returns the
        last layer's output (fp32) and the next token's input rms(output)."""
        import torch.nn.functional as F
        ds = self.ds
        for lay in self.layers:
            o = self.state_step(lay, *self.layer_inputs(x, lay))
            x = x + F.linear(o.reshape(ds.B, ds.H * ds.dv).to(self.wd), lay["W_o"]).float()
            gu = F.linear(F.rms_norm(x, (ds.hidden,), eps=EPS).to(self.wd), lay["W_gu"]).float()
            g, u = gu.split(ds.ffn, dim=1)
            x = x + F.linear((F.silu(g) * u).to(self.wd), lay["W_dn"]).float()
        return x, F.rms_norm(x, (ds.hidden,), eps=EPS)

    def capture_cycle(self, x_static):
        """A HIP graph of M tokens (one merge cycle, so the host-side log
        schedule ends where it began) that reads its input from x_static,
        writes every token's output into the returned [M, B, hidden] buffer
        and leaves the next input in x_static."""
        import torch
        ds = self.ds
        outs = torch.empty(ds.M, ds.B, ds.hidden, device="cuda")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            x = x_static
            for t in range(ds.M):
                out, x = self.token(x)
                outs[t].copy_(out)
            x_static.copy_(x)
        return g, outs

    def close(self):
        for lay in self.layers:
            if "st" in lay:
                lay["st"].close()


def warm_up(dec, x, tokens: int):
    """Run `tokens` tokens directly on a side stream (library handles and
    workspaces are created outside any capture), then rejoin."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(tokens):
            _, x = dec.token(x)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    return x


def time_graph(g, replays: int) -> float:
    import torch
    g.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(replays):
        g.replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / replays


def state_only_graph(dec, inputs):
    """A graph of the same state steps as one merge cycle of the model (M
    tokens x L layers) on fixed, pre-staged inputs."""
    import torch
    ds = dec.ds
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for t in range(ds.M):
            for lay in dec.layers:
                dec.state_step(lay, *inputs)
    return g


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--op", default="gdn", choices=["gdn", "kda", "rwkv6"])
    ap.add_argument("--layers", type=int, default=8)
    ap.add_argument("--B", type=int, default=64)
    ap.add_argument("--H", type=int, default=32)
    ap.add_argument("--d", type=int, default=128)
    ap.add_argument("--M", type=int, default=8)
    ap.add_argument("--hidden", type=int, default=2048)
    ap.add_argument("--ffn", type=int, default=4096)
    ap.add_argument("--cycles", type=int, default=8, help="timed graph replays (M tokens each)")
    args = ap.parse_args()

    import torch
    assert torch.cuda.is_available(), "bench_decoder.py needs a GPU"
    torch.cuda.set_device(0)
    ds = synth.DecoderShape(args.op, args.layers, args.B, args.H, args.d, args.d, args.M,
                            args.hidden, args.ffn)
    wd = torch.bfloat16
    t0 = time.time()
    dl = SyntheticDecoder(ds, "deltalog", wd)
    eg = SyntheticDecoder(ds, "eager", wd, weights_from=dl)
    log(f"built {ds.describe()} in {time.time() - t0:.1f}s")
    x0 = torch.from_numpy(synth.decoder_input(ds)).cuda()

    res = {}
    for name, dec in (("deltalog", dl), ("eager", eg)):
        x = warm_up(dec, x0.clone(), ds.M)
        g, _ = dec.capture_cycle(x)
        ms = time_graph(g, args.cycles) / ds.M
        res[name] = dict(tokens_per_s=round(ds.B / (ms * 1e-3), 1), ms_per_token=round(ms, 5))
        log(f"{name}: {ms * 1e3:.1f} us per token step ({ds.L} layers)")
        del g

    w = synth.Workload(11, ds.op, ds.B, ds.H, ds.dk, ds.dv, ds.M, 1, "bf16")
    s = synth.step(w, 0)
    inputs = tuple(None if s[k] is None else
                   torch.from_numpy(s[k]).cuda().to(wd if k in ("q", "k", "v") else torch.float32)
                   for k in ("q", "k", "v", "beta", "ld"))
    st_ms = {}
    for name, dec in (("deltalog", dl), ("eager", eg)):
        g = state_only_graph(dec, inputs)
        st_ms[name] = time_graph(g, args.cycles) / ds.M
        del g
    kernel_speedup = st_ms["eager"] / st_ms["deltalog"]
    share = st_ms["eager"] / res["eager"]["ms_per_token"]
    e2e = res["eager"]["ms_per_token"] / res["deltalog"]["ms_per_token"]
    out = {
        "metric": "synthetic decoder tokens/s, DeltaLog vs eager state step",
        "unit": "tokens/s",
        "config": {"workload": f"synthetic {ds.op.upper()} decoder: {ds.L} recurrent layers, B={ds.B} "
                               f"H={ds.H} d_k=d_v={ds.dk} M={ds.M}, hidden {ds.hidden}, gated MLP "
                               f"{ds.ffn}, bf16 weights, random init",
                   "op": ds.op, "layers": ds.L, "B": ds.B, "H": ds.H, "d": ds.dk, "M": ds.M,
                   "hidden": ds.hidden, "ffn": ds.ffn},
        "deltalog": res["deltalog"],
        "eager": res["eager"],
        "e2e_speedup": round(e2e, 3),
        "state_step_only": {"deltalog_ms_per_token": round(st_ms["deltalog"], 5),
                            "eager_ms_per_token": round(st_ms["eager"], 5),
                            "kernel_speedup": round(kernel_speedup, 3)},
        "eager_state_share": round(share, 3),
        "amdahl_predicted_e2e": round(1.0 / ((1.0 - share) + share / kernel_speedup), 3),
        "data": "synthetic (seeded PCG64 weights, states and first input)",
    }
    dl.close()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
