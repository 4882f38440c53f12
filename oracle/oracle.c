/*
 * oracle.c -- plain fp64 CPU oracle for the linear-attention recurrent-state
 * decode step (GDN, KDA, RWKV6) and for the DeltaLog base+log schedule.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file; only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no code, header or table with the HIP
 * path.
 *
 * Sources (the five pages about "DeltaLog: Deferred Materialization of
 * Recurrent States for Linear Attention Decoding", arXiv 2608.15533):
 *   - arXiv abstract (fugumt.com paper page, "Abstract"): the state is a dense
 *     base plus a bounded log of compact updates; most steps only append,
 *     periodic merges fold the log into the base, and the model observes the
 *     same dense state as eager decoding.
 *   - gist.science technical summary, "Core mechanism: Base + Log": base S-bar
 *     holds history up to the last merge; the log holds factors (a_t, b_t) and
 *     log-decay metadata Lambda; append phase for M-1 steps, merge every M.
 *   - same summary, "Kernel implementation": GDN has a per-head scalar decay
 *     with the delta-rule correction, KDA a per-key decay with the delta rule,
 *     RWKV6 a per-key decay with a raw (uncorrected) value update.
 *   - same summary, "Problem": the state S_t is d_k x d_v per head, stored as
 *     a [B,H,d_k,d_v] tensor.
 *
 * Notation.  One slot-head holds X (d_k rows = keys, d_v columns = values),
 * row-major, X[i*dv + j].  ell_t is the log-decay (<= 0): one scalar per
 * slot-head for GDN, one value per key for KDA and RWKV6.  D_t = diag(e^ell_t)
 * acts on the key (row) index.
 *
 * Eager recurrences (the plain definitions of the three operators):
 *   GDN / KDA (gated delta rule; the usual S = X^T form is
 *     S_t = S_{t-1} D_t + beta_t (v_t - S_{t-1} D_t k_t) k_t^T, o_t = S_t q_t):
 *       X'  = D_t X_{t-1}
 *       b_t = beta_t (v_t - X'^T k_t)
 *       X_t = X' + k_t b_t^T
 *       o_t = X_t^T q_t
 *   RWKV6 (decay plus raw outer product, output read before the update with
 *     the per-head bonus u):
 *       o_t = X_{t-1}^T r_t + (r_t . (u (.) k_t)) v_t
 *       X_t = D_t X_{t-1} + k_t v_t^T
 *
 * DeltaLog model (the pages name a_t, b_t, Lambda but print no formulas; the
 * reading used here): between steps a slot-head holds the base Xb, n log
 * entries (a_j, b_j, Lam_j) and the logical state
 *       X = e^{Lam_n} (.)row Xb + sum_{j<=n} (e^{Lam_n - Lam_j} (.) a_j) b_j^T
 * with Lam_0 = 0.  a_j = k_j (key side), b_j = the value-side factor of the
 * eager update (b_t above for the delta rule, v_t for RWKV6), Lam_j the
 * cumulative log-decay since the last merge, snapshotted when entry j is
 * appended.  The step that brings the log to M entries folds it into Xb
 * (merge) and empties it.  GDN's scalar decay is stored here broadcast over
 * the keys, which is the same number in every row.
 *
 * Full forgetting (a log-decay of -inf, e^ell = 0) is part of the domain of
 * the eager recurrences.  In the DeltaLog model, a cumulative Lam of -inf
 * would make a later difference Lam_n - Lam_j undefined (-inf - -inf).  So
 * the model takes each log-decay at no less than ORC_MIN_LOG_DECAY, where
 * e^ell is already exactly 0 in fp64: the step still zeroes every older term
 * exactly, and Lam stays finite (the reading taken for the pages' Lambda
 * snapshots; the abstract's claim that the model observes the same dense
 * state as eager decoding fixes the result).  The eager functions use ell
 * as given.
 *
 * All arithmetic is IEEE fp64, slot-heads are independent (OpenMP over them).
 * parity pinned: see the CPU test suite (brute-force unrolling, closed forms,
 * special cases, invariants, hand-worked examples).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_GDN 0
#define ORC_KDA 1
#define ORC_RWKV6 2

/* e^x is exactly 0 in fp64 for x below about -745.2 */
#define ORC_MIN_LOG_DECAY (-800.0)

/* log-decay of key i of slot-head sh */
static double log_decay(int op, const double *ld, long sh, int dk, int i)
{
    return op == ORC_GDN ? ld[sh] : ld[sh * dk + i];
}

/* ---------------------------------------------------------------- eager -- */

static void eager_one(int op, int h, long sh, int dk, int dv, double *X,
                      const double *q, const double *k, const double *v,
                      const double *beta, const double *ld, const double *u,
                      double *o, double *b)
{
    if (op == ORC_RWKV6) {
        /* o = X_{t-1}^T r + (r . (u (.) k)) v, read before the update */
        double mu = 0.0;
        for (int i = 0; i < dk; ++i)
            mu += q[i] * u[(long)h * dk + i] * k[i];
        for (int j = 0; j < dv; ++j) {
            double acc = 0.0;
            for (int i = 0; i < dk; ++i)
                acc += X[(long)i * dv + j] * q[i];
            o[j] = acc + mu * v[j];
        }
        /* X_t = D_t X_{t-1} + k v^T */
        for (int i = 0; i < dk; ++i) {
            double w = exp(log_decay(op, ld, sh, dk, i));
            for (int j = 0; j < dv; ++j)
                X[(long)i * dv + j] = w * X[(long)i * dv + j] + k[i] * v[j];
        }
        return;
    }
    /* X' = D_t X */
    for (int i = 0; i < dk; ++i) {
        double w = exp(log_decay(op, ld, sh, dk, i));
        for (int j = 0; j < dv; ++j)
            X[(long)i * dv + j] *= w;
    }
    /* b = beta (v - X'^T k) */
    for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i)
            acc += X[(long)i * dv + j] * k[i];
        b[j] = beta[sh] * (v[j] - acc);
    }
    /* X_t = X' + k b^T */
    for (int i = 0; i < dk; ++i)
        for (int j = 0; j < dv; ++j)
            X[(long)i * dv + j] += k[i] * b[j];
    /* o = X_t^T q */
    for (int j = 0; j < dv; ++j) {
        double acc = 0.0;
        for (int i = 0; i < dk; ++i)
            acc += X[(long)i * dv + j] * q[i];
        o[j] = acc;
    }
}

/*
 * One eager decode step for all B*H slot-heads.
 *   X    [B,H,dk,dv] in/out        q (r for RWKV6), k  [B,H,dk]
 *   v    [B,H,dv]                  beta [B,H] (ignored for RWKV6)
 *   ld   GDN [B,H], KDA/RWKV6 [B,H,dk] log-decay (<= 0)
 *   u    RWKV6 bonus [H,dk], else ignored
 *   o    [B,H,dv] out
 */
void orc_eager_step(int op, int B, int H, int dk, int dv, double *X,
                    const double *q, const double *k, const double *v,
                    const double *beta, const double *ld, const double *u,
                    double *o)
{
    long BH = (long)B * H;
#pragma omp parallel
    {
        double *b = (double *)malloc(sizeof(double) * (size_t)dv);
#pragma omp for schedule(static)
        for (long sh = 0; sh < BH; ++sh)
            eager_one(op, (int)(sh % H), sh, dk, dv, X + sh * dk * dv,
                      q + sh * dk, k + sh * dk, v + sh * dv, beta, ld, u,
                      o + sh * dv, b);
        free(b);
    }
}

/* ------------------------------------------------------- DeltaLog model -- */

/*
 * Fold the n entries of one slot-head's log into its base (merge phase):
 *   Xb <- e^{Lam_n} (.)row Xb + sum_{j<n} (e^{Lam_n - Lam_j} (.) a_j) b_j^T
 */
static void fold_one(int dk, int dv, int M, int n, double *Xb,
                     const double *a, const double *bl, const double *L)
{
    const double *Ln = L + (long)(n - 1) * dk;
    for (int i = 0; i < dk; ++i) {
        double base_w = exp(Ln[i]);
        for (int j = 0; j < dv; ++j) {
            double x = base_w * Xb[(long)i * dv + j];
            for (int m = 0; m < n; ++m)
                x += exp(Ln[i] - L[(long)m * dk + i]) * a[(long)m * dk + i] *
                     bl[(long)m * dv + j];
            Xb[(long)i * dv + j] = x;
        }
    }
    (void)M;
}

static void dl_one(int op, int h, long sh, int dk, int dv, int M, int n,
                   double *Xb, double *a, double *bl, double *L,
                   const double *q, const double *k, const double *v,
                   const double *beta, const double *ld, const double *u,
                   double *o, double *work)
{
    double *Lnew = work;          /* [dk] cumulative log-decay after step t */
    double *wq = work + dk;       /* [dk] weights of the base read */
    double *cq = work + 2 * dk;   /* [M]  replay coefficients, q side */
    double *ck = cq + M;          /* [M]  replay coefficients, k side */
    double *bt = ck + M;          /* [dv] this step's value-side factor */

    for (int i = 0; i < dk; ++i) {
        double prev = n > 0 ? L[(long)(n - 1) * dk + i] : 0.0;
        double ell = log_decay(op, ld, sh, dk, i);
        Lnew[i] = prev + (ell < ORC_MIN_LOG_DECAY ? ORC_MIN_LOG_DECAY : ell);
    }

    if (op == ORC_RWKV6) {
        /* output from the logical state before this step (Lam_n), plus bonus */
        for (int i = 0; i < dk; ++i) {
            double prev = n > 0 ? L[(long)(n - 1) * dk + i] : 0.0;
            wq[i] = exp(prev) * q[i];
        }
        for (int m = 0; m < n; ++m) {
            double c = 0.0;
            for (int i = 0; i < dk; ++i)
                c += exp(L[(long)(n - 1) * dk + i] - L[(long)m * dk + i]) *
                     a[(long)m * dk + i] * q[i];
            cq[m] = c;
        }
        double mu = 0.0;
        for (int i = 0; i < dk; ++i)
            mu += q[i] * u[(long)h * dk + i] * k[i];
        for (int j = 0; j < dv; ++j) {
            double y = 0.0;
            for (int i = 0; i < dk; ++i)
                y += Xb[(long)i * dv + j] * wq[i];
            for (int m = 0; m < n; ++m)
                y += cq[m] * bl[(long)m * dv + j];
            o[j] = y + mu * v[j];
            bt[j] = v[j];
        }
    } else {
        /* replay of the decayed logical state X' = D_t X against q and k */
        for (int m = 0; m < n; ++m) {
            double c_q = 0.0, c_k = 0.0;
            for (int i = 0; i < dk; ++i) {
                double e = exp(Lnew[i] - L[(long)m * dk + i]) * a[(long)m * dk + i];
                c_q += e * q[i];
                c_k += e * k[i];
            }
            cq[m] = c_q;
            ck[m] = c_k;
        }
        double kappa = 0.0;
        for (int i = 0; i < dk; ++i)
            kappa += q[i] * k[i];
        for (int j = 0; j < dv; ++j) {
            double yq = 0.0, yk = 0.0;
            for (int i = 0; i < dk; ++i) {
                double e = exp(Lnew[i]) * Xb[(long)i * dv + j];
                yq += e * q[i];
                yk += e * k[i];
            }
            for (int m = 0; m < n; ++m) {
                yq += cq[m] * bl[(long)m * dv + j];
                yk += ck[m] * bl[(long)m * dv + j];
            }
            bt[j] = beta[sh] * (v[j] - yk); /* delta rule on X' */
            o[j] = yq + kappa * bt[j];      /* (X' + k b^T)^T q */
        }
    }

    /* append entry n: a = k, b = bt, Lam = Lnew */
    for (int i = 0; i < dk; ++i) {
        a[(long)n * dk + i] = k[i];
        L[(long)n * dk + i] = Lnew[i];
    }
    for (int j = 0; j < dv; ++j)
        bl[(long)n * dv + j] = bt[j];

    if (n + 1 == M)
        fold_one(dk, dv, M, M, Xb, a, bl, L);
}

/*
 * One DeltaLog decode step for all B*H slot-heads, which move in lockstep so
 * the log length n is shared.  Buffers:
 *   Xb  [B,H,dk,dv] base, in/out
 *   a   [B,H,M,dk], bl [B,H,M,dv], L [B,H,M,dk] log, in/out (entries < n used)
 * Other arguments as orc_eager_step.  Returns the log length after the step
 * (n+1, or 0 when the step merged).  Returns -1 on a bad n.
 */
int orc_dl_step(int op, int B, int H, int dk, int dv, int M, int n,
                double *Xb, double *a, double *bl, double *L,
                const double *q, const double *k, const double *v,
                const double *beta, const double *ld, const double *u,
                double *o)
{
    if (n < 0 || n >= M)
        return -1;
    long BH = (long)B * H;
#pragma omp parallel
    {
        double *work = (double *)malloc(sizeof(double) * (size_t)(2 * dk + 2 * M + dv));
#pragma omp for schedule(static)
        for (long sh = 0; sh < BH; ++sh)
            dl_one(op, (int)(sh % H), sh, dk, dv, M, n, Xb + sh * dk * dv,
                   a + sh * M * dk, bl + sh * M * dv, L + sh * M * dk,
                   q + sh * dk, k + sh * dk, v + sh * dv, beta, ld, u,
                   o + sh * dv, work);
        free(work);
    }
    return n + 1 == M ? 0 : n + 1;
}

/*
 * Forced merge: fold the n pending entries of every slot-head into its base
 * and return 0 (the new log length).  n == 0 leaves everything untouched.
 */
int orc_dl_merge(int B, int H, int dk, int dv, int M, int n, double *Xb,
                 const double *a, const double *bl, const double *L)
{
    if (n < 0 || n >= M)
        return -1;
    if (n == 0)
        return 0;
    long BH = (long)B * H;
#pragma omp parallel for schedule(static)
    for (long sh = 0; sh < BH; ++sh)
        fold_one(dk, dv, M, n, Xb + sh * dk * dv, a + sh * M * dk,
                 bl + sh * M * dv, L + sh * M * dk);
    return 0;
}

/* threads an OpenMP parallel region would use */
int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* set the thread count of later parallel regions (no-op without OpenMP) */
void orc_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}
