"""Pins for the fp64 oracle: checks against what the mathematics fixes, each
independent of the oracle's own code path.

Every pin is a plain function ``pin_*(orc)`` that raises AssertionError when
the oracle ``orc`` (an ``oracle.Oracle``) is wrong.  The CPU test suite runs
them against the real oracle; the mutant test runs them against deliberately
broken copies of the oracle source and requires each copy to fail at least
one pin.

What pins what:
  hand examples (tests/golden/hand_examples.json) -- orientation, which axis
      the decay acts on, the output timing and the bonus term of each op;
  brute-force unrolling -- the eager recurrences over many steps, built from
      explicit d_k x d_k transition products (GDN, KDA) or decay products
      (RWKV6);
  delta-rule property -- beta = 1, |k| = 1 makes X_t^T k_t = v_t;
  frozen state -- beta = 0, no decay: o is a plain matrix-vector product;
  full decay -- log-decay -inf wipes the history: X_t = beta k v^T;
  RWKV6 without decay is a prefix sum of outer products; with u = 0 the
      output is X_{t-1}^T r;
  linearity -- scaling X_0 and every v scales o and X;
  DeltaLog model -- M = 1 is eager; after every merge the base equals the
      eager state, for every M; outputs equal eager outputs at every step; a
      forced merge at any log length gives the eager state; the model's
      logical state equals the eager state between merges; with full decay
      (log-decay -inf) and extreme finite decays scattered through the
      steps it still equals eager decoding, and stays finite.
"""
from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
OPS = ("gdn", "kda", "rwkv6")


def rel(x, ref):
    """Max-abs error relative to the max-abs of the reference."""
    x, ref = np.asarray(x, np.float64), np.asarray(ref, np.float64)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    num = np.max(np.abs(x - ref)) if ref.size else 0.0
    return float(num / den) if den > 0 else float(num)


def _inputs(op, B, H, dk, dv, T, seed, unit_k=True):
    """Random fp64 inputs for T steps (test-local; not the workload generator)."""
    rng = np.random.default_rng(seed)
    X0 = rng.normal(0, 0.3, (B, H, dk, dv))
    q = rng.normal(size=(T, B, H, dk))
    k = rng.normal(size=(T, B, H, dk))
    if unit_k and op != "rwkv6":
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.normal(size=(T, B, H, dv))
    beta = rng.uniform(0.05, 1.0, (T, B, H))
    if op == "gdn":
        ld = -rng.uniform(0.01, 0.7, (T, B, H))
    else:
        ld = -rng.uniform(0.01, 0.9, (T, B, H, dk))
    u = rng.normal(0, 0.5, (H, dk)) if op == "rwkv6" else None
    return X0, q, k, v, (None if op == "rwkv6" else beta), ld, u


def _decay_vec(op, ld_t, dk):
    """Per-key multipliers e^ell for one slot-head."""
    return np.full(dk, np.exp(ld_t)) if op == "gdn" else np.exp(ld_t)


def _eager_all(orc, op, X0, q, k, v, beta, ld, u):
    X = X0.copy()
    os_, Xs = [], []
    for t in range(q.shape[0]):
        os_.append(orc.eager_step(op, X, q[t], k[t], v[t],
                                  None if beta is None else beta[t], ld[t], u))
        Xs.append(X.copy())
    return np.stack(os_), np.stack(Xs)


# ------------------------------------------------------------ hand examples --
def pin_hand_examples(orc):
    with open(os.path.join(GOLDEN, "hand_examples.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        op = case["op"]
        S0 = np.array(case["S0"], np.float64)
        # oracle layout X is [d_k, d_v]; GDN/KDA write S = X^T, RWKV6 S = X
        X = (S0.T if op != "rwkv6" else S0).copy()[None, None]
        u = np.array(case["u"], np.float64)[None] if op == "rwkv6" else None
        for st in case["steps"]:
            q = np.array(st["q"], np.float64)[None, None]
            k = np.array(st["k"], np.float64)[None, None]
            v = np.array(st["v"], np.float64)[None, None]
            beta = np.array([[st.get("beta", 0.0)]], np.float64)
            ld = np.log(np.array(st["decay"], np.float64))
            ld = ld.reshape(1, 1) if op == "gdn" else ld.reshape(1, 1, -1)
            o = orc.eager_step(op, X, q, k, v, beta, ld, u)
            S = X[0, 0].T if op != "rwkv6" else X[0, 0]
            np.testing.assert_allclose(o[0, 0], st["o"], rtol=0, atol=1e-12,
                                       err_msg=f"{case['name']} o")
            np.testing.assert_allclose(S, st["S"], rtol=0, atol=1e-12,
                                       err_msg=f"{case['name']} S")


# ------------------------------------------------------ brute-force unrolling --
def _brute_delta(op, X0, q, k, v, beta, ld):
    """GDN/KDA: X_t = A_t X_{t-1} + beta_t k_t v_t^T with
    A_t = (I - beta_t k_t k_t^T) D_t, unrolled as explicit matrix products:
    X_t = A_t...A_1 X_0 + sum_j A_t...A_{j+1} beta_j k_j v_j^T."""
    T, dk = q.shape[0], q.shape[-1]
    A = []
    for t in range(T):
        D = np.diag(_decay_vec(op, ld[t], dk))
        A.append((np.eye(dk) - beta[t] * np.outer(k[t], k[t])) @ D)
    os_, Xs = [], []
    for t in range(T):
        P = np.eye(dk)
        for s in range(t, -1, -1):
            P = P @ A[s]
        X = P @ X0
        for j in range(t + 1):
            P = np.eye(dk)
            for s in range(t, j, -1):
                P = P @ A[s]
            X = X + P @ (beta[j] * np.outer(k[j], v[j]))
        Xs.append(X)
        os_.append(X.T @ q[t])
    return np.array(os_), np.array(Xs)


def _brute_rwkv(X0, q, k, v, ld, u):
    """RWKV6: X_t = diag(prod_{s<=t} w_s) X_0 + sum_j diag(prod_{j<s<=t} w_s) k_j v_j^T,
    o_t = X_{t-1}^T r_t + (r_t . (u * k_t)) v_t."""
    T = q.shape[0]
    w = np.exp(ld)

    def state(t):  # X after t steps (t = 0 is X0)
        X = np.diag(np.prod(w[:t], axis=0) if t > 0 else np.ones(X0.shape[0])) @ X0
        for j in range(t):
            X = X + np.diag(np.prod(w[j + 1:t], axis=0) if t > j + 1 else np.ones(X0.shape[0])) \
                @ np.outer(k[j], v[j])
        return X

    os_, Xs = [], []
    for t in range(T):
        Xp = state(t)
        os_.append(Xp.T @ q[t] + np.dot(q[t], u * k[t]) * v[t])
        Xs.append(state(t + 1))
    return np.array(os_), np.array(Xs)


def pin_brute_force(orc):
    for op in OPS:
        for (B, H, dk, dv, T, seed) in ((1, 2, 4, 3, 12, 1), (2, 1, 8, 8, 20, 2), (1, 1, 16, 16, 8, 3)):
            X0, q, k, v, beta, ld, u = _inputs(op, B, H, dk, dv, T, seed)
            o, Xs = _eager_all(orc, op, X0, q, k, v, beta, ld, u)
            for b in range(B):
                for h in range(H):
                    sl = (slice(None), b, h)
                    if op == "rwkv6":
                        ob, Xb = _brute_rwkv(X0[b, h], q[sl], k[sl], v[sl], ld[sl], u[h])
                    else:
                        ob, Xb = _brute_delta(op, X0[b, h], q[sl], k[sl], v[sl], beta[sl], ld[sl])
                    assert rel(o[sl], ob) < 1e-12, (op, "o", rel(o[sl], ob))
                    assert rel(Xs[sl], Xb) < 1e-12, (op, "X", rel(Xs[sl], Xb))


# ------------------------------------------------------------- closed forms --
def pin_delta_rule(orc):
    """beta = 1 and |k| = 1: the updated state maps k_t exactly to v_t."""
    for op in ("gdn", "kda"):
        X0, q, k, v, beta, ld, u = _inputs(op, 2, 3, 16, 8, 6, 11)
        X = X0.copy()
        for t in range(6):
            orc.eager_step(op, X, q[t], k[t], v[t], np.ones_like(beta[t]), ld[t], u)
            got = np.einsum("bhij,bhi->bhj", X, k[t])
            assert rel(got, v[t]) < 1e-12, (op, rel(got, v[t]))


def pin_frozen_gemv(orc):
    """beta = 0 and zero log-decay (delta ops), or zero decay and k = 0 for
    RWKV6: the state never changes and o is a plain X^T q."""
    for op in OPS:
        X0, q, k, v, beta, ld, u = _inputs(op, 2, 2, 8, 16, 4, 12)
        X = X0.copy()
        for t in range(4):
            zero_ld = np.zeros_like(ld[t])
            if op == "rwkv6":
                o = orc.eager_step(op, X, q[t], np.zeros_like(k[t]), v[t], None, zero_ld, u)
            else:
                o = orc.eager_step(op, X, q[t], k[t], v[t], np.zeros_like(beta[t]), zero_ld, u)
            ref = np.matmul(np.swapaxes(X0, -1, -2), q[t][..., None])[..., 0]
            assert rel(o, ref) < 1e-13, (op, rel(o, ref))
            assert np.array_equal(X, X0), op


def pin_full_decay(orc):
    """log-decay -inf on every key: the history vanishes; X_t = beta k v^T
    (delta ops, with b = beta v since the decayed state is zero) or k v^T
    (RWKV6, whose output still reads the old state)."""
    for op in OPS:
        X0, q, k, v, beta, ld, u = _inputs(op, 1, 2, 8, 4, 1, 13)
        X = X0.copy()
        full = np.full_like(ld[0], -np.inf)
        o = orc.eager_step(op, X, q[0], k[0], v[0], None if beta is None else beta[0], full, u)
        if op == "rwkv6":
            ref_X = np.einsum("bhi,bhj->bhij", k[0], v[0])
            ref_o = np.einsum("bhij,bhi->bhj", X0, q[0]) + \
                np.einsum("bhi,hi,bhi->bh", q[0], u, k[0])[..., None] * v[0]
        else:
            ref_X = beta[0][..., None, None] * np.einsum("bhi,bhj->bhij", k[0], v[0])
            ref_o = np.einsum("bhij,bhi->bhj", ref_X, q[0])
        assert rel(X, ref_X) < 1e-14, (op, "X")
        assert rel(o, ref_o) < 1e-13, (op, "o")


def pin_rwkv_prefix_sum(orc):
    """RWKV6 with zero log-decay: X_t = X_0 + sum_{j<=t} k_j v_j^T (cumulative
    sum); with u = 0 the output is X_{t-1}^T r_t."""
    X0, q, k, v, _, ld, u = _inputs("rwkv6", 2, 2, 8, 8, 10, 14)
    X = X0.copy()
    outer = np.einsum("tbhi,tbhj->tbhij", k, v)
    cums = X0[None] + np.cumsum(outer, axis=0)
    zero_u = np.zeros_like(u)
    for t in range(10):
        prev = X.copy()
        o = orc.eager_step("rwkv6", X, q[t], k[t], v[t], None, np.zeros_like(ld[t]), zero_u)
        assert rel(X, cums[t]) < 1e-13
        assert rel(o, np.einsum("bhij,bhi->bhj", prev, q[t])) < 1e-13


def pin_linearity(orc):
    """Scaling X_0 and every v by c scales every o and X by c."""
    c = 3.0
    for op in OPS:
        X0, q, k, v, beta, ld, u = _inputs(op, 1, 2, 8, 8, 6, 15)
        o1, X1 = _eager_all(orc, op, X0, q, k, v, beta, ld, u)
        o2, X2 = _eager_all(orc, op, c * X0, q, k, c * v, beta, ld, u)
        assert rel(o2, c * o1) < 1e-13 and rel(X2, c * X1) < 1e-13, op


# ------------------------------------------------------------ DeltaLog model --
def _dl_run(orc, op, M, X0, q, k, v, beta, ld, u):
    from oracle import DeltaLogModel
    m = DeltaLogModel(orc, op, X0, M)
    os_, Xbs, ns = [], [], []
    for t in range(q.shape[0]):
        os_.append(m.step(q[t], k[t], v[t], None if beta is None else beta[t], ld[t], u))
        Xbs.append(m.Xb.copy())
        ns.append(m.n)
    return np.stack(os_), np.stack(Xbs), ns, m


def pin_dl_m1_is_eager(orc):
    """M = 1: every step merges, so base and outputs are the eager ones."""
    for op in OPS:
        X0, q, k, v, beta, ld, u = _inputs(op, 2, 2, 8, 8, 7, 21)
        oe, Xe = _eager_all(orc, op, X0, q, k, v, beta, ld, u)
        od, Xd, ns, _ = _dl_run(orc, op, 1, X0, q, k, v, beta, ld, u)
        assert all(n == 0 for n in ns)
        assert rel(od, oe) < 1e-12 and rel(Xd, Xe) < 1e-12, op


def pin_dl_merge_invariant(orc):
    """For every M, outputs match eager at every step; right after each merge
    the base equals the eager state; between merges the base is unchanged and
    the logical state (base + replayed log) equals the eager state."""
    for op in OPS:
        T = 24
        X0, q, k, v, beta, ld, u = _inputs(op, 2, 2, 16, 8, T, 22)
        oe, Xe = _eager_all(orc, op, X0, q, k, v, beta, ld, u)
        for M in (2, 3, 4, 5, 8, 16):
            from oracle import DeltaLogModel
            m = DeltaLogModel(orc, op, X0, M)
            prev_base = m.Xb.copy()
            for t in range(T):
                o = m.step(q[t], k[t], v[t], None if beta is None else beta[t], ld[t], u)
                assert rel(o, oe[t]) < 1e-11, (op, M, t, "o")
                if (t + 1) % M == 0:
                    assert m.n == 0
                    assert rel(m.Xb, Xe[t]) < 1e-11, (op, M, t, "merged base")
                else:
                    assert m.n == (t + 1) % M
                    assert np.array_equal(m.Xb, prev_base), (op, M, t, "base written on append")
                    assert rel(m.logical_state(), Xe[t]) < 1e-11, (op, M, t, "logical state")
                prev_base = m.Xb.copy()


def pin_dl_forced_merge(orc):
    """A forced merge after any number of appends gives the eager state, and a
    second merge changes nothing."""
    for op in OPS:
        X0, q, k, v, beta, ld, u = _inputs(op, 1, 3, 8, 16, 7, 23)
        oe, Xe = _eager_all(orc, op, X0, q, k, v, beta, ld, u)
        M = 8
        for stop in range(1, 8):
            from oracle import DeltaLogModel
            m = DeltaLogModel(orc, op, X0, M)
            for t in range(stop):
                m.step(q[t], k[t], v[t], None if beta is None else beta[t], ld[t], u)
            assert m.n == stop
            m.merge()
            assert m.n == 0 and rel(m.Xb, Xe[stop - 1]) < 1e-11, (op, stop)
            before = m.Xb.copy()
            m.merge()
            assert np.array_equal(before, m.Xb)


def pin_dl_full_decay(orc):
    """Full forgetting inside a log.  Log-decays of -inf (and of -1e4, where
    e^ell is 0 as well) at scattered steps, heads and keys: outputs at every
    step, the base after each merge and the logical state between merges
    all equal eager decoding, which is pinned on full decay above, and all
    are finite.  This includes entries appended after a wipe, whose decays
    are differences of cumulative log-decays."""
    from oracle import DeltaLogModel
    rng = np.random.default_rng(27)
    for op in OPS:
        T = 14
        X0, q, k, v, beta, ld, u = _inputs(op, 2, 2, 8, 8, T, 26)
        ld = ld.copy()
        pick = rng.uniform(size=ld.shape)
        ld[pick < 0.15] = -np.inf
        ld[(pick >= 0.15) & (pick < 0.25)] = -1e4
        ld[3] = -np.inf  # one step that wipes every slot-head entirely
        oe, Xe = _eager_all(orc, op, X0, q, k, v, beta, ld, u)
        assert np.isfinite(oe).all() and np.isfinite(Xe).all()
        for M in (2, 3, 5, 8):
            m = DeltaLogModel(orc, op, X0, M)
            for t in range(T):
                o = m.step(q[t], k[t], v[t], None if beta is None else beta[t], ld[t], u)
                assert np.isfinite(o).all(), (op, M, t, "o not finite")
                assert rel(o, oe[t]) < 1e-11, (op, M, t, "o")
                X = m.Xb if m.n == 0 else m.logical_state()
                assert np.isfinite(X).all(), (op, M, t, "state not finite")
                assert rel(X, Xe[t]) < 1e-11, (op, M, t, "state")


ALL_PINS = [
    pin_hand_examples, pin_brute_force, pin_delta_rule, pin_frozen_gemv,
    pin_full_decay, pin_rwkv_prefix_sum, pin_linearity, pin_dl_m1_is_eager,
    pin_dl_merge_invariant, pin_dl_forced_merge, pin_dl_full_decay,
]
