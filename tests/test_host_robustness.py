"""CPU-tier robustness checks (no GPU):

1. Checkpoint/restore of the fp64 DeltaLog model mid-cycle: base, log entries
   and log length snapshotted, restored into a fresh model, and continued,
   give bit-for-bit the uninterrupted run (and the eager state).
2. The oracle's C code built with AddressSanitizer and UndefinedBehavior-
   Sanitizer (gcc), driven through every operator's eager step and DeltaLog
   model on lopsided shapes, with the two compared: no sanitizer report and
   agreement to fp64 rounding.
3. Handle life cycle through the C ABI without a launch: a forced merge of an
   empty log twice, destroy then re-create on the same buffers.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest

import synth
from oracle import SRC, DeltaLogModel

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.parametrize("op", ["gdn", "kda", "rwkv6"])
def test_model_checkpoint_restore_mid_cycle(orc, op):
    w = synth.Workload(30, op, 2, 3, 16, 8, 5, 13, "f32")
    X0, u = synth.initial(w)
    steps = [synth.step(w, t) for t in range(w.steps)]

    def feed(m, s):
        return m.step(s["q"], s["k"], s["v"], s["beta"], s["ld"], u)

    ref = DeltaLogModel(orc, op, X0, w.M)
    for s in steps[:7]:
        feed(ref, s)
    assert ref.n == 2  # mid-cycle: 7 = 5 + 2
    snap = ref.snapshot()
    out_ref = [feed(ref, s) for s in steps[7:]]
    ref.merge()

    fresh = DeltaLogModel(orc, op, np.zeros_like(X0), w.M)
    fresh.restore(snap)
    out_new = [feed(fresh, s) for s in steps[7:]]
    fresh.merge()
    for a, b in zip(out_ref, out_new):
        assert np.array_equal(a, b)
    assert np.array_equal(ref.Xb, fresh.Xb)

    X = X0.astype(np.float64).copy()
    for s in steps:
        orc.eager_step(op, X, s["q"], s["k"], s["v"], s["beta"], s["ld"], u)
    assert np.max(np.abs(fresh.Xb - X)) / np.max(np.abs(X)) < 1e-12


DRIVER = r"""
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
void orc_eager_step(int, int, int, int, int, double *, const double *, const double *,
                    const double *, const double *, const double *, const double *, double *);
int orc_dl_step(int, int, int, int, int, int, int, double *, double *, double *, double *,
                const double *, const double *, const double *, const double *, const double *,
                const double *, double *);
int orc_dl_merge(int, int, int, int, int, int, double *, const double *, const double *,
                 const double *);

static unsigned long long st = 88172645463325252ULL;
static double uni(void) /* xorshift64, in [-1, 1) */
{
    st ^= st << 13; st ^= st >> 7; st ^= st << 17;
    return (double)(st >> 11) / 4503599627370496.0 - 1.0;
}
static double *arr(long n, double scale)
{
    double *p = malloc(sizeof(double) * (size_t)n);
    for (long i = 0; i < n; ++i) p[i] = scale * uni();
    return p;
}

int main(void)
{
    const int B = 2, H = 3, shapes[2][2] = {{16, 8}, {8, 32}}, M = 3, T = 7;
    for (int op = 0; op < 3; ++op)
        for (int si = 0; si < 2; ++si) {
            const int dk = shapes[si][0], dv = shapes[si][1];
            const long BH = (long)B * H, P = BH * dk * dv;
            double *X = arr(P, 0.1), *Xb = malloc(sizeof(double) * (size_t)P);
            for (long i = 0; i < P; ++i) Xb[i] = X[i];
            double *a = calloc((size_t)(BH * M * dk), sizeof(double));
            double *bl = calloc((size_t)(BH * M * dv), sizeof(double));
            double *L = calloc((size_t)(BH * M * dk), sizeof(double));
            double *u = arr((long)H * dk, 0.1);
            double *o1 = malloc(sizeof(double) * (size_t)(BH * dv));
            double *o2 = malloc(sizeof(double) * (size_t)(BH * dv));
            int n = 0;
            double worst = 0.0;
            for (int t = 0; t < T; ++t) {
                double *q = arr(BH * dk, 0.3), *k = arr(BH * dk, 0.3), *v = arr(BH * dv, 1.0);
                double *beta = arr(BH, 0.5), *ld = arr(op == 0 ? BH : BH * dk, 0.5);
                for (long i = 0; i < BH; ++i) beta[i] = 0.5 + beta[i];
                for (long i = 0; i < (op == 0 ? BH : BH * dk); ++i) ld[i] = -fabs(ld[i]);
                orc_eager_step(op, B, H, dk, dv, X, q, k, v, beta, ld, u, o1);
                n = orc_dl_step(op, B, H, dk, dv, M, n, Xb, a, bl, L, q, k, v, beta, ld, u, o2);
                if (n < 0) return 2;
                for (long i = 0; i < BH * dv; ++i)
                    if (fabs(o1[i] - o2[i]) > worst) worst = fabs(o1[i] - o2[i]);
                free(q); free(k); free(v); free(beta); free(ld);
            }
            if (orc_dl_merge(B, H, dk, dv, M, n, Xb, a, bl, L) != 0) return 3;
            for (long i = 0; i < P; ++i)
                if (fabs(X[i] - Xb[i]) > worst) worst = fabs(X[i] - Xb[i]);
            printf("op %d dk %d dv %d worst %.3g\n", op, dk, dv, worst);
            if (!(worst < 1e-9)) return 4;
            free(X); free(Xb); free(a); free(bl); free(L); free(u); free(o1); free(o2);
        }
    return 0;
}
"""


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_address_and_ub_sanitizers(tmp_path):
    drv = tmp_path / "driver.c"
    drv.write_text(DRIVER)
    exe = tmp_path / "oracle_asan"
    cmd = ["gcc", "-std=c99", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           str(drv), SRC, "-o", str(exe), "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "sanitize" in r.stderr:
        pytest.skip("sanitizer runtimes not available: " + r.stderr[-200:])
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ERROR" not in r.stderr and "runtime error" not in r.stderr, r.stderr
    assert r.stdout.count("worst") == 6


def test_abi_handle_life_cycle():
    import recurrent_state_update_amd as rsu
    BASE, WS = 0x7f0000000000, 0x7f0000100000  # fake device addresses, never dereferenced
    st, h = rsu.dl_state_create(2, 3, 16, 16, 4, 0, 0, BASE, WS, None)
    assert st == 0
    assert rsu.dl_merge(h, 0) == 0 and rsu.dl_merge(h, 0) == 0  # empty log: no launch, twice
    assert rsu.dl_log_len(h) == 0
    assert rsu.dl_state_destroy(h) == 0
    st, h2 = rsu.dl_state_create(2, 3, 16, 16, 4, 0, 0, BASE, WS, None)
    assert st == 0 and rsu.dl_log_len(h2) == 0
    assert rsu.dl_set_log_len(h2, 3) == 0 and rsu.dl_log_len(h2) == 3
    assert rsu.dl_state_destroy(h2) == 0
