/*
 * deltalog.h -- C ABI of libdeltalog: the DeltaLog recurrent-state decode step
 * for linear attention (GDN, KDA, RWKV6) on AMD Instinct MI355X (gfx950).
 *
 * What it computes.  "DeltaLog: Deferred Materialization of Recurrent States
 * for Linear Attention Decoding" (arXiv 2608.15533; abstract on the fugumt.com
 * paper page, technical summary on gist.science).  Each (slot, head) keeps a
 * d_k x d_v fp32 state ("Problem" section: S_t is d_k x d_v, held as a
 * [B,H,d_k,d_v] tensor).  Eager decoding rewrites the whole state every token.
 * DeltaLog keeps a dense base S-bar plus a bounded log of compact factors
 * (a_t, b_t) and log-decay metadata Lambda ("Core mechanism: Base + Log"):
 * M-1 of every M steps only append to the log, the M-th merges the log into
 * S-bar with one dense write.  Outputs equal eager decoding's up to floating
 * point rounding (abstract: the model observes the same dense state).
 *
 * Operators ("Kernel implementation" section), per slot-head, with X the
 * d_k x d_v state (row i = key i, column j = value j), ell_t the log-decay
 * (<= 0; one per head for GDN, one per key for KDA/RWKV6), D_t = diag(e^ell_t):
 *   GDN, KDA (delta rule):  X' = D_t X;  b_t = beta_t (v_t - X'^T k_t);
 *                           X_t = X' + k_t b_t^T;  o_t = X_t^T q_t
 *   RWKV6 (raw update):     o_t = X_{t-1}^T r_t + (r_t . (u (.) k_t)) v_t;
 *                           X_t = D_t X_{t-1} + k_t v_t^T
 * (In the common S = X^T notation of GDN/KDA: S_t = S_{t-1} D_t +
 * beta_t (v_t - S_{t-1} D_t k_t) k_t^T, o_t = S_t q_t.)
 *
 * Log contents (the pages name a_t, b_t, Lambda without formulas; the reading
 * implemented here): a_t = k_t; b_t = the delta-rule b_t above (fp32), or v_t
 * for RWKV6 (input dtype); and ell_t, the step's log-decay.  The pages'
 * log-decay snapshot Lambda_t (the cumulative log-decay since the last merge)
 * is the running sum of the logged ell's; keeping the terms rather than their
 * running sum lets every decay factor be formed as a sum of consecutive
 * terms, exact to a few ulps even after repeated full forgetting.  Between
 * steps the logical state is
 *   X = e^{Lambda_n} (.)row S-bar + sum_{j<=n} (e^{Lambda_n - Lambda_j} (.) a_j) b_j^T.
 *
 * Memory layouts (all row-major, all device memory, all caller-owned):
 *   state / base   [B,H,d_k,d_v] fp32, 16-byte aligned
 *   q (r), k       [B,H,d_k]   input dtype          v  [B,H,d_v] input dtype
 *   beta           [B,H] fp32 (GDN, KDA; NULL for RWKV6)
 *   log_decay      GDN [B,H] fp32; KDA, RWKV6 [B,H,d_k] fp32 (natural log, <= 0).
 *                  -inf (full forgetting: the step erases the history) is
 *                  accepted.  Values below -112 act as -112, where e^ell is
 *                  already exactly 0 in fp32; this keeps every sum of logged
 *                  decays finite.
 *   u              RWKV6 bonus [H,d_k] fp32 (NULL for GDN, KDA)
 *   o              [B,H,d_v] fp32, 16-byte aligned
 *   workspace      dl_workspace_bytes() bytes, 256-byte aligned; holds the log,
 *                  the two-stage path's per-step coefficients and the per-slot
 *                  log phases; contents need no initialisation
 * Supported shapes: d_k, d_v in {16, 32, 64, 128}; 1 <= M <= 32; B, H >= 1
 * with B*H*d_k*d_v < 2^33 (a state of up to 32 GiB per handle; larger shapes
 * return DL_E_SHAPE).  All B slots step in lockstep (one shared log
 * length) unless per-slot logs are enabled (see the end of this file).
 *
 * Errors and ownership.  Every call returns a dl_status and never aborts or
 * throws.  Arguments are validated on the host before any HIP call (so bad
 * arguments are reported the same way with or without a GPU).  Kernel launch
 * failures return DL_E_HIP.  A buffer that a call writes (o; base and
 * workspace, through the handle; S of the eager step) must not overlap any
 * other buffer of the call, or the call returns DL_E_INVALID; the read-only
 * inputs may alias each other.  All calls are asynchronous on `stream` (a
 * hipStream_t; NULL = the default stream): a DL_OK return says the work was
 * queued, not that it finished.  The library never allocates or frees device
 * memory; the handle is host memory owned by the library (create/destroy).
 * A handle is not thread-safe; calls on one handle must be ordered on one
 * stream.
 */
#ifndef DELTALOG_H
#define DELTALOG_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { DL_OP_GDN = 0, DL_OP_KDA = 1, DL_OP_RWKV6 = 2 } dl_op;
typedef enum { DL_F32 = 0, DL_BF16 = 1 } dl_dtype;
typedef enum {
    DL_OK = 0,
    DL_E_INVALID = 1, /* null pointer, bad enum, B/H/M out of range, missing beta or u */
    DL_E_SHAPE = 2,   /* d_k or d_v not supported, or the state too large */
    DL_E_ALIGN = 3,   /* a pointer is not aligned as required above */
    DL_E_HIP = 4,     /* a HIP launch failed */
    DL_E_STATE = 5,   /* call out of order (e.g. append without replay prep) */
    DL_E_SCRATCH = 6  /* dl_decode_step_staged_noalloc: shape beyond its static scratch */
} dl_status;

typedef struct dl_state dl_state; /* opaque host-side handle */

/* Bytes of device workspace a handle of this shape needs (0 if the arguments
 * are invalid): the bounded log, M entries of O(d_k + d_v) factors per
 * slot-head ("Core mechanism: Base + Log": the log of compact factors and
 * log-decay metadata), plus the two-stage path's coefficients and the
 * per-slot phases. */
size_t dl_workspace_bytes(int B, int H, int d_k, int d_v, int M, dl_op op, dl_dtype in_dtype);

/* Create a handle over caller-owned device memory ("Problem": one d_k x d_v
 * state per slot and head, a [B,H,d_k,d_v] tensor; "Core mechanism: Base +
 * Log": that tensor becomes the dense base S-bar, beside a bounded log).
 * `base` holds the initial state S-bar_0 [B,H,d_k,d_v] fp32 and is updated
 * in place on merge steps; `workspace` has dl_workspace_bytes() bytes; `u`
 * is RWKV6's bonus [H,d_k] (NULL otherwise).  The log starts empty.  *out
 * receives the handle.  Errors: DL_E_INVALID (null or overlapping buffers,
 * B/H/M out of range, u missing for RWKV6), DL_E_SHAPE, DL_E_ALIGN. */
dl_status dl_state_create(int B, int H, int d_k, int d_v, int M, dl_op op, dl_dtype in_dtype,
                          float *base, void *workspace, const float *u, dl_state **out);

/* One decode step for all B*H slot-heads ("Core mechanism: Base + Log": the
 * append phase, which writes only the step's compact factors and log-decay,
 * on M-1 of every M steps; the merge phase, which folds the log into S-bar
 * with one dense write and empties it, on the step that brings the log to M
 * entries).  Writes o_t [B,H,d_v] fp32.
 * q is r for RWKV6.  beta may be NULL for RWKV6.  One kernel launch: each
 * value-tile workgroup also does its slot-head's ReplayPrep work.  Computes
 * the same step as dl_replay_prep followed by dl_append_decode (the results
 * agree up to floating-point summation order). */
dl_status dl_decode_step(dl_state *s, const void *q, const void *k, const void *v,
                         const float *beta, const float *log_decay, float *o, void *stream);

/* Stage 1 of a decode step ("Kernel implementation": the shared ReplayPrep
 * stage, once per slot-head): the replay coefficients of the n pending
 * entries against q_t and k_t (their decay factors e^{Lambda' - Lambda_j}
 * formed from the logged log-decays), q.k (RWKV6: r.(u (.) k)), and the
 * key-side append (a = k and this step's log-decay).  Must be followed by
 * dl_append_decode with the same q and k before any other call on s
 * (otherwise DL_E_STATE). */
dl_status dl_replay_prep(dl_state *s, const void *q, const void *k, const float *log_decay,
                         void *stream);

/* Stage 2 of a decode step ("Kernel implementation": AppendDecode, parallel
 * over value tiles, each owning a slice of S-bar and the matching value-side
 * log shard): streams S-bar, adds the replayed log, writes o_t and the
 * value-side factor b_t; on the M-th step also folds the whole log into S-bar
 * (one dense write).  DL_E_STATE unless dl_replay_prep ran just before. */
dl_status dl_append_decode(dl_state *s, const void *q, const void *k, const void *v,
                           const float *beta, float *o, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * two-stage step (dl_replay_prep then dl_append_decode) in one call whose
 * per-step replay coefficients live in a static device buffer of the library
 * instead of the workspace.  It allocates nothing; inputs, outputs and the
 * handle's base and workspace are as for dl_decode_step, and it leaves the
 * handle exactly as that pair of calls would (results agree bit for bit).
 * Limit: B*H*(2M+2) <= 2^20 floats (4 MiB; e.g. B*H = 8192 at M = 32),
 * otherwise DL_E_SCRATCH before any HIP call.  Each GPU has one such buffer,
 * shared by every call on it: calls that overlap in time on one GPU (on
 * different streams or host threads) race and must not be issued; calls
 * ordered on one stream are safe.  The calling thread's current device must
 * be the one that holds the handle's buffers and the stream.  The first call
 * on a device looks up the buffer's address (DL_E_HIP if that fails). */
dl_status dl_decode_step_staged_noalloc(dl_state *s, const void *q, const void *k, const void *v,
                                        const float *beta, const float *log_decay, float *o,
                                        void *stream);

/* Merge now ("Core mechanism: Base + Log", the merge phase, taken before its
 * M-th step): fold the n pending entries into S-bar with one dense write so
 * that `base` holds the logical state; empties the log.  No-op (DL_OK) when
 * the log is empty.  DL_E_STATE between dl_replay_prep and
 * dl_append_decode. */
dl_status dl_merge(dl_state *s, void *stream);

/* Empty the log without folding it (S-bar is left as is): drops the pending
 * updates.  For restarting a handle over a freshly written base. */
dl_status dl_state_reset(dl_state *s);

/* Number of pending log entries, 0..M-1 ("Core mechanism: Base + Log": the
 * log is bounded, holding at most M-1 entries between steps); -1 for a NULL
 * handle or a handle with per-slot logs (use dl_slot_log_len). */
int dl_log_len(const dl_state *s);

/* Set the number of pending entries to n (0..M-1) after the caller restored
 * base and workspace contents saved at that log length (exact mid-cycle
 * checkpoint/restore). */
dl_status dl_set_log_len(dl_state *s, int n);

/* Release the handle (host memory; the caller's device buffers are left as
 * they are, and the base holds S-bar, the logical state only if the log is
 * empty: see dl_merge).  NULL is accepted. */
dl_status dl_state_destroy(dl_state *s);

/* The same-GPU baseline ("Problem": eager decoding applies each token's update
 * to the whole state and writes the full [B,H,d_k,d_v] tensor back to HBM on
 * every step; the abstract's dense recurrent baselines): one eager step that
 * reads and rewrites S [B,H,d_k,d_v] in place and writes o [B,H,d_v].  u is
 * RWKV6's bonus [H,d_k] (NULL otherwise); beta may be NULL for RWKV6.
 * Errors as for dl_decode_step, plus DL_E_INVALID if S overlaps another
 * buffer. */
dl_status dl_eager_step(dl_op op, int B, int H, int d_k, int d_v, dl_dtype in_dtype, float *S,
                        const void *q, const void *k, const void *v, const float *beta,
                        const float *log_decay, const float *u, float *o, void *stream);

/* The merge interval M in [1, 32] that minimises the modelled HBM bytes per
 * decode step of dl_decode_step for this shape ("Traffic model" section of the
 * gist.science summary: appends of O(d_k + d_v) factors replace full writes,
 * one dense write every M steps, and a log replay that grows with M).  Per
 * slot-head, averaged over an M-cycle (mean log length (M-1)/2):
 *   bytes(M) = P (1 + 1/M)                  base read every step, write per merge
 *            + (M-1)/2 (E_key * tiles + E_val)   replay of the logged entries
 *            + (M-1)/M E_app                 appended entry (none on the merge)
 *            + (M-1)/M E_key (tiles_m - tiles)   the merge's extra key-side reads
 * with P = 4 d_k d_v, E_key = a_j + log-decay bytes (re-read by each value
 * tile: tiles_m = d_v/min(d_v, 64) tiles for a merge, and as many for an
 * append except KDA at d_v = 128, whose appends take whole rows: tiles = 1),
 * E_val = b_j bytes, E_app = E_key + E_val.
 * Returns 0 for invalid arguments. */
int dl_suggest_merge_interval(int B, int H, int d_k, int d_v, dl_op op, dl_dtype in_dtype);

/* The merge interval M in [1, max_M] that minimises the mean time per decode
 * step over a merge cycle, predicted from measured launch times (the
 * "Traffic model" trade-off of the gist.science summary, priced in measured
 * time instead of modelled bytes: M-1 appends whose log replay grows with
 * the log, then one merge whose dense write the M steps share):
 *   time(M) = ( append_us[0] + ... + append_us[M-2] + merge_us[M-1] ) / M.
 * append_us[n] is the time of one dl_decode_step launch that appends with n
 * entries in the log, merge_us[n] that of one that merges with n entries in
 * the log (folding n + 1), both for the caller's shape; each array holds
 * max_M host doubles (append_us[max_M-1] is not read).  A calibration takes
 * them by timing launches with the log held at each length (dl_set_log_len),
 * as `bench.py --choose-M` does.  The smallest such M on ties.  Returns 0 for
 * a NULL array, a negative or non-finite time, or max_M outside [1, 32]. */
int dl_choose_merge_interval(const double *append_us, const double *merge_us, int max_M);

/* ------------------------------------------------------------------------
 * Per-slot logs, for continuous batching.  The pages apply the schedule per
 * (slot, head) ("Kernel implementation": ReplayPrep runs per slot-head); with
 * per-slot logs each slot (a request) keeps its own log length, so requests
 * admitted at different steps merge at different steps.  Every decode step
 * still covers all B slots in one launch, in which each slot appends or, when
 * its log is full, merges.  None of these calls allocates, and all are
 * capturable into HIP graphs.
 * ------------------------------------------------------------------------ */

/* Switch a handle to per-slot logs.  Needs an empty log (a fresh handle, or
 * after dl_merge); every slot starts empty.  Afterwards dl_decode_step and
 * dl_merge act per slot; dl_replay_prep, dl_append_decode, dl_set_log_len and
 * dl_state_reset return DL_E_STATE.  Checkpoint of such a handle: dl_merge
 * (every active slot's log is then empty), save `base`; to restore, create a
 * handle over the saved base, enable per-slot logs and release the slots
 * that were released.  It continues exactly as the original would. */
dl_status dl_state_enable_slots(dl_state *s, void *stream);

/* Admit a new request into `slot` (also one released before): drop the
 * slot's pending log without folding it.  The caller writes the request's
 * initial state into the slot's rows of `base` ([slot, 0..H)) before the next
 * step (stream-ordered). */
dl_status dl_slot_admit(dl_state *s, int slot, void *stream);

/* Fold the pending entries of one slot into its rows of `base` (which then
 * hold that slot's logical state) and empty its log.  No-op when the slot's
 * log is empty or the slot is released.  Use before reading a finished
 * request's state. */
dl_status dl_slot_merge(dl_state *s, int slot, void *stream);

/* Release `slot` (its request finished; merge it first to keep its state):
 * until the next dl_slot_admit of this slot, decode steps and merges skip
 * it entirely (no reads, no writes; its rows of `base`, its outputs in `o`
 * and its log are left untouched), so empty slots cost no memory traffic. */
dl_status dl_slot_release(dl_state *s, int slot, void *stream);

/* Pending entries of one slot (the shared count on a lockstep handle; 0 for
 * a released slot), -1 for a bad handle or slot. */
int dl_slot_log_len(const dl_state *s, int slot);

/* Static description of a status code (never NULL; owned by the library). */
const char *dl_status_string(dl_status st);

#ifdef __cplusplus
}
#endif

#endif /* DELTALOG_H */
