"""The fp64 oracle against its pins (closed forms, brute force, invariants,
hand-worked examples); see pins.py for what each pin fixes."""
import pytest

from pins import ALL_PINS


@pytest.mark.parametrize("pin", ALL_PINS, ids=[p.__name__ for p in ALL_PINS])
def test_pin(orc, pin):
    pin(orc)


def test_eager_run_is_repeated_steps(orc):
    """orc_eager_run (used for multi-step CPU work) is T calls of the pinned
    orc_eager_step."""
    import numpy as np
    from pins import _inputs
    for op in ("gdn", "kda", "rwkv6"):
        X0, q, k, v, beta, ld, u = _inputs(op, 2, 3, 8, 16, 5, 31)
        Xa, Xb = X0.copy(), X0.copy()
        oa = orc.eager_run(op, Xa, q, k, v, beta, ld, u)
        ob = np.stack([orc.eager_step(op, Xb, q[t], k[t], v[t], None if beta is None else beta[t],
                                      ld[t], u) for t in range(5)])
        assert np.array_equal(oa, ob) and np.array_equal(Xa, Xb)
