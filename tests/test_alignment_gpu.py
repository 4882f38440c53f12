"""Inputs at the smallest alignment the C ABI accepts: q, k, v aligned only to
their element size (a view one element into a larger buffer), and beta, the
log-decay and u one fp32 element in.  The kernels read inputs with buffer
loads whose width is a multiple of the element (a 32-bit word holding two
bf16 keys, four v elements at once), so these loads are not aligned to their
own width.  Every path must give exactly the results of the same call on
aligned copies of the same inputs (the arithmetic is the same, so bit for
bit); the aligned runs are checked against the oracle by the parity tests."""
import numpy as np
import pytest
import torch

import synth
from gpu_harness import dev

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU")


def _shifted(t):
    """The same values as t, contiguous, one element past an aligned address."""
    flat = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
    view = flat[1:].view(t.shape)
    view.copy_(t)
    return view


def _inputs(w, t, dt):
    s = synth.step(w, t)
    return {k_: None if v_ is None else dev(v_, dt if k_ in ("q", "k", "v") else torch.float32)
            for k_, v_ in s.items()}


@needs_gpu
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
def test_element_aligned_inputs(op, dtype):
    import recurrent_state_update_amd as rsu
    w = synth.Workload(37, op, 2, 3, 128, 128, 4, 9, dtype)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    X0, u = synth.initial(w)
    u_al = dev(u)
    u_sh = None if u is None else _shifted(u_al)
    if u_sh is not None:
        assert u_sh.data_ptr() % 8 == 4
    handles = {}
    for path in ("one_launch", "two_stage"):
        for shifted in (False, True):
            handles[path, shifted] = rsu.DeltaLogState(op, w.B, w.H, w.dk, w.dv, w.M, dtype=dt, base=dev(X0),
                                                       u=u_sh if shifted else u_al)
    S_al, S_sh = dev(X0), dev(X0)
    esz = 2 if dtype == "bf16" else 4
    for t in range(w.steps):
        al = _inputs(w, t, dt)
        sh = {k_: None if v_ is None else _shifted(v_) for k_, v_ in al.items()}
        assert sh["q"].data_ptr() % (2 * esz) == esz  # not aligned beyond the element
        outs = {}
        for (path, shifted), st in handles.items():
            x = sh if shifted else al
            if path == "one_launch":
                outs[path, shifted] = st.step(x["q"], x["k"], x["v"], x["beta"], x["ld"])
            else:
                st.replay_prep(x["q"], x["k"], x["ld"])
                outs[path, shifted] = st.append_decode(x["q"], x["k"], x["v"], x["beta"])
        o_al = rsu.eager_step(op, S_al, al["q"], al["k"], al["v"], al["beta"], al["ld"], u=u_al)
        o_sh = rsu.eager_step(op, S_sh, sh["q"], sh["k"], sh["v"], sh["beta"], sh["ld"], u=u_sh)
        torch.cuda.synchronize()
        for path in ("one_launch", "two_stage"):
            assert torch.equal(outs[path, True], outs[path, False]), (op, dtype, path, t)
        assert torch.equal(o_sh, o_al), (op, dtype, "eager", t)
    for st in handles.values():
        st.merge()
    torch.cuda.synchronize()
    for path in ("one_launch", "two_stage"):
        assert torch.equal(handles[path, True].base, handles[path, False].base), (op, dtype, path)
    assert torch.equal(S_sh, S_al), (op, dtype, "eager")
    # the run did reach the state: the aligned one-launch base moved off X0
    assert not np.array_equal(handles["one_launch", False].base.cpu().numpy(), X0.astype(np.float32))
    for st in handles.values():
        st.close()
