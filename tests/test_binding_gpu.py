"""The Python binding's argument checks and defaults, on the GPU (the binding
takes device tensors, so a handle needs one)."""
import numpy as np
import pytest
import torch

import synth
from gpu_harness import FP32_TOL, dev, rel

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU")


@needs_gpu
@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
def test_replay_prep_rejects_bad_tensors(op):
    """dl_replay_prep through the binding validates q, k and the log-decay
    like step() does: a wrong shape (a GDN-shaped [B,H] decay on a per-key
    operator and the reverse), a short q, the wrong dtype or a host tensor
    raise ValueError before any launch, and the handle stays usable."""
    import recurrent_state_update_amd as rsu
    B, H, d = 2, 3, 32
    st = rsu.DeltaLogState(op, B, H, d, d, 4, dtype=torch.bfloat16,
                           u=torch.zeros(H, d, device="cuda") if op == "rwkv6" else None)
    q = torch.zeros(B, H, d, dtype=torch.bfloat16, device="cuda")
    good_ld = torch.zeros((B, H) if op == "gdn" else (B, H, d), device="cuda")
    bad_ld = torch.zeros((B, H, d) if op == "gdn" else (B, H), device="cuda")
    with pytest.raises(ValueError):
        st.replay_prep(q, q, bad_ld)
    with pytest.raises(ValueError):
        st.replay_prep(q[:, :, : d // 2].contiguous(), q, good_ld)
    with pytest.raises(ValueError):
        st.replay_prep(q.float(), q, good_ld)
    with pytest.raises(ValueError):
        st.replay_prep(q, q.cpu(), good_ld)
    with pytest.raises(ValueError):
        st.replay_prep(q, q, good_ld.double())
    assert st.log_len == 0
    st.replay_prep(q, q, good_ld)           # still usable: a full step
    o = st.append_decode(q, q, torch.zeros(B, H, d, dtype=torch.bfloat16, device="cuda"),
                         torch.zeros(B, H, device="cuda") if op != "rwkv6" else None)
    torch.cuda.synchronize()
    assert st.log_len == 1 and torch.isfinite(o).all()
    st.close()


@needs_gpu
@pytest.mark.parametrize("op", ["gdn", "rwkv6"])
def test_per_slot_default_output_zero_for_released_slots(orc, op):
    """On a per-slot handle, step() without an output buffer returns zeros in
    the rows of released slots (their workgroups store nothing) and the
    oracle's outputs in the others."""
    import recurrent_state_update_amd as rsu
    w = synth.Workload(31, op, 4, 3, 64, 64, 4, 6, "bf16")
    X0, u = synth.initial(w)
    st = rsu.DeltaLogState(op, w.B, w.H, w.dk, w.dv, w.M, dtype=torch.bfloat16, base=dev(X0), u=dev(u))
    st.enable_slots()
    st.release(1)
    st.release(3)
    X = X0.reshape(w.BH, w.dk, w.dv).astype(np.float64)[None].copy()
    u_sub = None if u is None else u[np.arange(w.BH) % w.H].astype(np.float64)
    live = np.repeat(np.array([True, False, True, False]), w.H)
    worst = 0.0
    for t in range(w.steps):
        # fill the allocator's free blocks with NaN so that an uninitialised
        # default output could not pass for zeros
        torch.full((w.B, w.H, w.dv), float("nan"), device="cuda")
        s = synth.step(w, t)
        d_ = {k_: dev(v_, torch.bfloat16 if k_ in ("q", "k", "v") else torch.float32) for k_, v_ in s.items()}
        o = st.step(d_["q"], d_["k"], d_["v"], d_["beta"], d_["ld"]).reshape(w.BH, w.dv).cpu().numpy()
        o_ref = orc.eager_step(op, X, s["q"].reshape(1, w.BH, w.dk), s["k"].reshape(1, w.BH, w.dk),
                               s["v"].reshape(1, w.BH, w.dv),
                               None if s["beta"] is None else s["beta"].reshape(1, w.BH),
                               s["ld"].reshape((1, w.BH) + s["ld"].shape[2:]), u_sub)[0]
        assert (o[~live] == 0).all(), "released slots' rows must stay zero"
        worst = max(worst, rel(o[live], o_ref[live]))
    st.close()
    assert worst < FP32_TOL
