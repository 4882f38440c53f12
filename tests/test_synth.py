"""The seeded workload generator: determinism, shapes, bf16 rounding and the
distributions it claims."""
import numpy as np
import pytest
import torch

import synth


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(size=100000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e-39, -7.5e37], np.float32)])
    ours = synth.round_bf16(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))
    # bf16 values survive a second rounding unchanged
    assert np.array_equal(synth.round_bf16(ours), ours)


@pytest.mark.parametrize("wid", [0, 1, 2, 3])
def test_deterministic_and_regenerable(wid):
    w = synth.WORKLOADS[wid].with_(B=2, H=3)
    a = synth.step(w, 5)
    b = synth.steps(w, 4, 3)
    for key in a:
        if a[key] is None:
            assert b[key] is None
        else:
            assert np.array_equal(a[key], b[key][1])
    X0a, ua = synth.initial(w)
    X0b, ub = synth.initial(w)
    assert np.array_equal(X0a, X0b)
    assert (ua is None) == (w.op != "rwkv6")


@pytest.mark.parametrize("wid", [0, 1, 2, 3])
def test_shapes_and_ranges(wid):
    w = synth.WORKLOADS[wid].with_(B=4)
    s = synth.step(w, 0)
    B, H, dk, dv = w.B, w.H, w.dk, w.dv
    assert s["q"].shape == (B, H, dk) and s["k"].shape == (B, H, dk) and s["v"].shape == (B, H, dv)
    assert all(s[x].dtype == np.float32 for x in ("q", "k", "v", "ld"))
    assert np.all(s["ld"] < 0)
    if w.op == "gdn":
        assert s["ld"].shape == (B, H)
    else:
        assert s["ld"].shape == (B, H, dk)
    if w.op in ("gdn", "kda"):
        assert s["beta"].shape == (B, H) and np.all((s["beta"] > 0) & (s["beta"] < 1))
        n = np.linalg.norm(s["k"].astype(np.float64), axis=-1)
        assert np.allclose(n, 1.0, atol=1e-2 if w.dtype == "bf16" else 1e-5)
    else:
        assert s["beta"] is None
    if w.dtype == "bf16":
        for x in ("q", "k", "v"):
            assert np.array_equal(synth.round_bf16(s[x]), s[x])


def test_distributions():
    w = synth.WORKLOADS[1].with_(B=16)
    X0, _ = synth.initial(w)
    assert abs(X0.std() - 0.1) < 2e-3 and abs(X0.mean()) < 2e-3
    s = synth.step(w, 1)
    g = s["ld"].astype(np.float64)
    pre = np.log(np.expm1(-g))             # invert -softplus: N(-3, 0.5)
    assert abs(pre.mean() + 3.0) < 0.05 and abs(pre.std() - 0.5) < 0.05
    logit = np.log(s["beta"] / (1 - s["beta"]))
    assert abs(logit.mean()) < 0.1 and abs(logit.std() - 1.0) < 0.1
    r = synth.WORKLOADS[3].with_(B=8)
    s = synth.step(r, 0)
    pre = np.log(-s["ld"].astype(np.float64))   # invert -exp: N(-0.5, 0.5)
    assert abs(pre.mean() + 0.5) < 0.05 and abs(pre.std() - 0.5) < 0.05
    _, u = synth.initial(r)
    assert u.shape == (r.H, r.dk) and abs(u.std() - 0.1) < 0.02


def test_subset_keeps_slot_heads():
    w = synth.WORKLOADS[3].with_(B=3)
    d = synth.steps(w, 0, 2)
    idx = np.array([0, 5, 64, 191])
    sub = synth.subset(d, idx, lead=1)
    flat = d["k"].reshape(2, w.B * w.H, w.dk)
    assert sub["k"].shape == (2, 1, 4, w.dk)
    assert np.array_equal(sub["k"][:, 0], flat[:, idx])


def test_decoder_params_are_seeded_and_scaled():
    ds = synth.DecoderShape("kda", L=2, B=2, H=3, dk=16, dv=32, M=4, hidden=256, ffn=384)
    a, b = synth.decoder_layer(ds, 1), synth.decoder_layer(ds, 1)
    c = synth.decoder_layer(ds, 0)
    for k in ("W_in", "W_o", "W_gu", "W_dn", "X0"):
        assert np.array_equal(a[k], b[k]) and not np.array_equal(a[k], c[k])
    assert a["W_in"].shape == (256, sum(ds.proj_split)) == (256, 3 * 16 + 3 * 16 + 3 * 32 + 3 + 3 * 16)
    assert a["W_gu"].shape == (256, 768) and a["W_dn"].shape == (384, 256)
    assert abs(a["W_in"].std() * np.sqrt(256) - 1) < 0.02 and abs(a["W_dn"].std() * np.sqrt(384) - 1) < 0.02
    assert a["u"] is None and synth.decoder_layer(ds.__class__(**{**ds.__dict__, "op": "rwkv6"}), 0)["u"].shape == (3, 16)
    assert synth.DecoderShape("gdn", 1, 1, 4, 16, 16, 2, 8, 8).proj_split == [64, 64, 64, 4, 4]
    assert synth.DecoderShape("rwkv6", 1, 1, 4, 16, 16, 2, 8, 8).proj_split == [64, 64, 64, 0, 64]
    x = synth.decoder_input(ds)
    assert x.shape == (2, 256) and np.array_equal(x, synth.decoder_input(ds))
