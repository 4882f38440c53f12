"""Host logic of bench.py (no GPU): the launch order times whole merge
cycles at any --steps, and the byte model gives the traffic model's figures
for the three serving workloads (P(1 + 1/M) + E((M-1)/M + (M-1)/2) + I per
slot-head and step, the "Traffic model" section of the gist.science
technical summary, priced with the library's log layout: a_t in the input
dtype, b_t in fp32 (RWKV6: the input dtype), the log-decay in fp32)."""
import pytest

import bench
import synth


@pytest.mark.parametrize("K", [1, 3, 4, 5, 20, 64])
@pytest.mark.parametrize("R,M", [(4, 8), (1, 8), (24, 8), (4, 1), (3, 5)])
def test_launch_order_times_whole_merge_cycles(K, R, M):
    order = bench.launch_order(K, R, M)
    kinds = bench.launch_kinds(order, M)
    assert len(order) == K * M
    assert sum(mg for _, mg in kinds) == K                  # exactly K merges, whatever K is
    assert all(0 <= s < R for s in order)
    for s in range(R):                                      # every state ends with an empty log
        assert order.count(s) % M == 0
    # the log lengths before each launch walk 0..M-1 per state, merging at M-1
    for (n, mg) in kinds:
        assert mg == (n == M - 1)


def test_driver_command_times_merges():
    """The driver's --steps 20 at the default 4 states and M = 8: 160
    launches, 20 of them merges (none were timed before the order was fixed
    to whole cycles)."""
    kinds = bench.launch_kinds(bench.launch_order(20, 4, 8), 8)
    assert len(kinds) == 160 and sum(mg for _, mg in kinds) == 20


@pytest.mark.parametrize("R,M", [(4, 8), (1, 8), (3, 5), (4, 1)])
def test_pattern_cycles_follow_the_launch_order(R, M):
    count = 3 * R * M
    writes = bench.pattern_cycle_writes(count, R, M)
    kinds = bench.launch_kinds(bench.launch_order(3 * R, R, M), M)
    assert writes == [int(mg) for _, mg in kinds]


@pytest.mark.parametrize("wid,E,I,cycle_bytes", [
    (1, 772, 1288, 160_549_888),    # GDN B=64 H=32 d=128: 78,393.5 B per slot-head per step
    (2, 1280, 1796, 166_141_952),   # KDA, same shape, per-key log-decays
    (3, 512, 896, 176_701_440),     # RWKV6 B=128 H=64 d=64, b_t = v_t in bf16, u once
])
def test_byte_model_is_the_traffic_model(wid, E, I, cycle_bytes):
    w = synth.WORKLOADS[wid]
    P, M = 4 * w.dk * w.dv, w.M
    per = P * (1 + 1 / M) + E * ((M - 1) / M + (M - 1) / 2) + I
    u = 4 * w.H * w.dk if w.op == "rwkv6" else 0   # RWKV6's bonus [H, d_k], shared by the B slots
    assert bench.modelled_step_bytes(w) == pytest.approx(per * w.BH + u, rel=1e-12)
    # the per-launch sum over a cycle (log lengths 0..M-1, the last merging)
    # is the same number, and it is the figure the bench line's roofline uses
    assert bench.cycle_launch_bytes(w) == pytest.approx(per * w.BH + u, rel=1e-12)
    assert round(bench.cycle_launch_bytes(w)) == cycle_bytes
    # eager: read and write the state, plus the step's inputs and output
    assert bench.eager_launch_bytes(w) == (2 * P + I) * w.BH + u


def test_byte_model_counts_merges_and_appends():
    """One launch's bytes: the log grows by one entry per append, a merge
    writes the state once and appends nothing."""
    w = synth.WORKLOADS[1]
    P = 4 * w.dk * w.dv
    E = 772
    a0 = bench.step_launch_bytes(w, 0, False)
    a1 = bench.step_launch_bytes(w, 1, False)
    m7 = bench.step_launch_bytes(w, 7, True)
    assert a1 - a0 == E * w.BH                     # one more logged entry read
    assert m7 - bench.step_launch_bytes(w, 7, False) == (P - E) * w.BH   # the write, no append
