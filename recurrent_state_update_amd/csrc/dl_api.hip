// dl_api.hip -- the C ABI of libdeltalog (include/deltalog.h): argument
// validation, the per-handle append/merge schedule, and kernel dispatch.
//
// Schedule ("Core mechanism: Base + Log" in the gist.science technical summary
// of DeltaLog): the host keeps the log length n of each handle.  A step with
// n + 1 < M is an append step (ReplayPrep, then AppendDecode without a state
// write); the step with n + 1 == M is the merge step (AppendDecode folds all M
// entries into S-bar and writes it once) and leaves n = 0.  The schedule is
// decided on the host from n alone, so no device-to-host read is ever needed.
//
// dl_decode_step runs the step as one launch of the fused kernel (the
// ReplayPrep work done inside each AppendDecode workgroup); dl_replay_prep +
// dl_append_decode run it as the two-stage split, ReplayPrep once per
// slot-head then AppendDecode per value tile.  Both compute the same step.
//
// This file is plain host code: kernels are reached only through the
// launchers declared in dl_internal.h (dl_gdn.hip, dl_kda.hip, dl_rwkv6.hip,
// dl_device.hip), so it also builds with a host compiler alone, as the
// sanitizer test does.
#include <new>

#include "deltalog.h"
#include "dl_internal.h"

struct dl_state {
    int B, H, dk, dv, M;
    dl_op op;
    dl_dtype dtype;
    float *base;
    char *ws;
    const float *u;
    dl::Layout lay;
    int n;        // pending log entries (lockstep schedule)
    bool prepped; // ReplayPrep ran for the step in progress
    // per-slot schedule (continuous batching): slot b holds (tm - t0[b]) mod M
    // entries, or is released (no request) when t0[b] < 0; t0 is mirrored
    // here and in the workspace
    bool per_slot;
    int tm;       // steps taken, mod M
    int *t0;      // host mirror [B]
};

namespace dl {

static size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

Layout workspace_layout(long B, long H, int dk, int dv, int M, int op, int dtype)
{
    const size_t es = dtype == BF16 ? 2 : 4; // input element size
    const long BH = B * H;
    Layout l{};
    l.cstride = 2 * M + 2;
    l.a_off = 0;
    l.b_off = round_up(l.a_off + (size_t)BH * M * dk * es, 256);
    const size_t bsz = op == RWKV6 ? es : 4;
    l.L_off = round_up(l.b_off + (size_t)BH * M * dv * bsz, 256);
    const size_t lsz = op == GDN ? (size_t)BH * M * 4 : (size_t)BH * M * dk * 4;
    l.c_off = round_up(l.L_off + lsz, 256);
    l.t_off = round_up(l.c_off + (size_t)BH * l.cstride * 4, 256);
    l.total = round_up(l.t_off + (size_t)B * 4, 256);
    return l;
}

} // namespace dl

namespace {

bool dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

dl_status check_shape(int B, int H, int dk, int dv, int M, int op, int dtype)
{
    if (op < DL_OP_GDN || op > DL_OP_RWKV6 || (dtype != DL_F32 && dtype != DL_BF16))
        return DL_E_INVALID;
    if (B <= 0 || H <= 0 || M < 1 || M > 32)
        return DL_E_INVALID;
    if (!dim_ok(dk) || !dim_ok(dv))
        return DL_E_SHAPE;
    // Every launch dispatches at most d_k*d_v/4 work-items per slot-head
    // (each step-kernel lane holds at least 4 state elements; ReplayPrep runs
    // 64, and d_k*d_v >= 256), and a dispatch counts its work-items in 32
    // bits: below 2^33 state elements (a 32 GiB fp32 state) every launch
    // stays under 2^31 of them.  Device offsets are 64-bit throughout.
    if ((long long)B * H * dk * dv >= (1LL << 33))
        return DL_E_SHAPE;
    return DL_OK;
}

// inputs of one step: q, k, v in the input dtype, beta/log-decay fp32, o fp32;
// the log-decay is checked only when the call reads it (need_ld)
dl_status check_step_ptrs(int op, int dtype, const void *q, const void *k, const void *v,
                          const float *beta, const float *ld, const float *o, bool need_ld)
{
    if (!q || !k || !v || !o || (need_ld && !ld))
        return DL_E_INVALID;
    if (op != DL_OP_RWKV6 && !beta)
        return DL_E_INVALID;
    const size_t es = dtype == DL_BF16 ? 2 : 4;
    if (!aligned(q, es) || !aligned(k, es) || !aligned(v, es) || (ld && !aligned(ld, 4)) ||
        (beta && !aligned(beta, 4)) || !aligned(o, 16))
        return DL_E_ALIGN;
    return DL_OK;
}

// Byte ranges of a call's buffers.  A buffer the call writes (o, the base,
// the workspace) must not overlap any other buffer of the call: kernels
// would read it while other workgroups write it.  Inputs may alias each
// other (all are read-only).
struct Span {
    const void *p;
    size_t bytes;
};

bool overlap(Span a, Span b)
{
    if (!a.p || !b.p || a.bytes == 0 || b.bytes == 0)
        return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a.p), y = reinterpret_cast<uintptr_t>(b.p);
    return x < y + b.bytes && y < x + a.bytes;
}

dl_status check_overlaps(const Span *writes, int nw, const Span *reads, int nr)
{
    for (int i = 0; i < nw; ++i) {
        for (int j = i + 1; j < nw; ++j)
            if (overlap(writes[i], writes[j]))
                return DL_E_INVALID;
        for (int j = 0; j < nr; ++j)
            if (overlap(writes[i], reads[j]))
                return DL_E_INVALID;
    }
    return DL_OK;
}

// The buffers of one step on a B x H x d_k x d_v shape.
struct StepSpans {
    Span q, k, v, beta, ld, u, o, base;
};

StepSpans step_spans(int op, int dtype, long B, long H, int dk, int dv, const void *q, const void *k,
                     const void *v, const float *beta, const float *ld, const float *u, const float *o,
                     const float *base)
{
    const size_t es = dtype == DL_BF16 ? 2 : 4, BH = (size_t)(B * H);
    StepSpans sp;
    sp.q = {q, BH * dk * es};
    sp.k = {k, BH * dk * es};
    sp.v = {v, BH * dv * es};
    sp.beta = {beta, BH * 4};
    sp.ld = {ld, (op == DL_OP_GDN ? BH : BH * dk) * 4};
    sp.u = {u, (size_t)H * dk * 4};
    sp.o = {o, BH * dv * 4};
    sp.base = {base, BH * dk * dv * 4};
    return sp;
}

dl::StepArgs make_args(const dl_state *s)
{
    dl::StepArgs a{};
    a.BH = s->B * s->H;
    a.H = s->H;
    a.M = s->M;
    a.n = s->n;
    a.u = s->u;
    a.base = s->base;
    a.alog = s->ws + s->lay.a_off;
    a.blog = s->ws + s->lay.b_off;
    a.Llog = reinterpret_cast<float *>(s->ws + s->lay.L_off);
    a.coef = reinterpret_cast<float *>(s->ws + s->lay.c_off);
    a.cstride = s->lay.cstride;
    a.tm = s->tm;
    a.t0 = reinterpret_cast<const int *>(s->ws + s->lay.t_off);
    a.slot = -1;
    return a;
}

int *slot_phases(const dl_state *s) { return reinterpret_cast<int *>(s->ws + s->lay.t_off); }

hipError_t launch_prep(int op, int dtype, int dk, const dl::StepArgs &a, hipStream_t st)
{
    switch (op) {
    case DL_OP_GDN: return dl::launch_prep_gdn(dtype, dk, a, st);
    case DL_OP_KDA: return dl::launch_prep_kda(dtype, dk, a, st);
    default: return dl::launch_prep_rwkv6(dtype, dk, a, st);
    }
}

hipError_t launch_step(int op, int dtype, int dk, int dv, int mode, const dl::StepArgs &a,
                       hipStream_t st)
{
    switch (op) {
    case DL_OP_GDN: return dl::launch_step_gdn(dtype, dk, dv, mode, a, st);
    case DL_OP_KDA: return dl::launch_step_kda(dtype, dk, dv, mode, a, st);
    default: return dl::launch_step_rwkv6(dtype, dk, dv, mode, a, st);
    }
}

// o, the base and the workspace against each other and against the step's
// inputs (ld may be NULL: the two-stage AppendDecode does not read it)
dl_status check_handle_step_overlaps(const dl_state *s, const void *q, const void *k, const void *v,
                                     const float *beta, const float *ld, const float *o)
{
    const StepSpans sp = step_spans(s->op, s->dtype, s->B, s->H, s->dk, s->dv, q, k, v, beta, ld, s->u, o,
                                    s->base);
    const Span w[3] = {sp.o, sp.base, {s->ws, s->lay.total}};
    const Span r[6] = {sp.q, sp.k, sp.v, sp.beta, sp.ld, sp.u};
    return check_overlaps(w, 3, r, 6);
}

} // namespace

extern "C" {

size_t dl_workspace_bytes(int B, int H, int d_k, int d_v, int M, dl_op op, dl_dtype in_dtype)
{
    if (check_shape(B, H, d_k, d_v, M, op, in_dtype) != DL_OK)
        return 0;
    return dl::workspace_layout(B, H, d_k, d_v, M, op, in_dtype).total;
}

dl_status dl_state_create(int B, int H, int d_k, int d_v, int M, dl_op op, dl_dtype in_dtype,
                          float *base, void *workspace, const float *u, dl_state **out)
{
    if (!out)
        return DL_E_INVALID;
    *out = nullptr;
    const dl_status st = check_shape(B, H, d_k, d_v, M, op, in_dtype);
    if (st != DL_OK)
        return st;
    if (!base || !workspace || (op == DL_OP_RWKV6 && !u))
        return DL_E_INVALID;
    if (!aligned(base, 16) || !aligned(workspace, 256) || (u && !aligned(u, 4)))
        return DL_E_ALIGN;
    {
        const StepSpans sp = step_spans(op, in_dtype, B, H, d_k, d_v, nullptr, nullptr, nullptr, nullptr,
                                        nullptr, op == DL_OP_RWKV6 ? u : nullptr, nullptr, base);
        const Span w[2] = {sp.base, {workspace, dl::workspace_layout(B, H, d_k, d_v, M, op, in_dtype).total}};
        if (check_overlaps(w, 2, &sp.u, 1) != DL_OK)
            return DL_E_INVALID;
    }
    dl_state *s = new (std::nothrow) dl_state;
    int *t0 = new (std::nothrow) int[B];
    if (!s || !t0) {
        delete s;
        delete[] t0;
        return DL_E_INVALID;
    }
    s->B = B;
    s->H = H;
    s->dk = d_k;
    s->dv = d_v;
    s->M = M;
    s->op = op;
    s->dtype = in_dtype;
    s->base = base;
    s->ws = static_cast<char *>(workspace);
    s->u = op == DL_OP_RWKV6 ? u : nullptr;
    s->lay = dl::workspace_layout(B, H, d_k, d_v, M, op, in_dtype);
    s->n = 0;
    s->prepped = false;
    s->per_slot = false;
    s->tm = 0;
    s->t0 = t0;
    for (int b = 0; b < B; ++b)
        t0[b] = 0;
    *out = s;
    return DL_OK;
}

dl_status dl_replay_prep(dl_state *s, const void *q, const void *k, const float *log_decay,
                         void *stream)
{
    if (!s || !q || !k || !log_decay)
        return DL_E_INVALID;
    if (s->prepped || s->per_slot)
        return DL_E_STATE;
    const size_t es = s->dtype == DL_BF16 ? 2 : 4;
    if (!aligned(q, es) || !aligned(k, es) || !aligned(log_decay, 4))
        return DL_E_ALIGN;
    {
        const StepSpans sp = step_spans(s->op, s->dtype, s->B, s->H, s->dk, s->dv, q, k, nullptr, nullptr,
                                        log_decay, nullptr, nullptr, nullptr);
        const Span w = {s->ws, s->lay.total};
        const Span r[3] = {sp.q, sp.k, sp.ld};
        if (check_overlaps(&w, 1, r, 3) != DL_OK)
            return DL_E_INVALID;
    }
    dl::StepArgs a = make_args(s);
    a.q = q;
    a.k = k;
    a.ld = log_decay;
    if (launch_prep(s->op, s->dtype, s->dk, a, static_cast<hipStream_t>(stream)) != hipSuccess)
        return DL_E_HIP;
    s->prepped = true;
    return DL_OK;
}

dl_status dl_append_decode(dl_state *s, const void *q, const void *k, const void *v,
                           const float *beta, float *o, void *stream)
{
    if (!s)
        return DL_E_INVALID;
    if (!s->prepped || s->per_slot)
        return DL_E_STATE;
    // this stage does not read the log-decay: ReplayPrep stored Lam'
    dl_status st = check_step_ptrs(s->op, s->dtype, q, k, v, beta, nullptr, o, false);
    if (st == DL_OK)
        st = check_handle_step_overlaps(s, q, k, v, beta, nullptr, o);
    if (st != DL_OK)
        return st;
    dl::StepArgs a = make_args(s);
    a.q = q;
    a.k = k;
    a.v = v;
    a.beta = beta;
    a.o = o;
    const bool merge = s->n + 1 == s->M;
    if (launch_step(s->op, s->dtype, s->dk, s->dv, merge ? dl::MERGE : dl::APPEND, a,
                     static_cast<hipStream_t>(stream)) != hipSuccess)
        return DL_E_HIP;
    s->prepped = false;
    s->n = merge ? 0 : s->n + 1;
    return DL_OK;
}

dl_status dl_decode_step(dl_state *s, const void *q, const void *k, const void *v,
                         const float *beta, const float *log_decay, float *o, void *stream)
{
    if (!s)
        return DL_E_INVALID;
    if (s->prepped)
        return DL_E_STATE;
    dl_status st = check_step_ptrs(s->op, s->dtype, q, k, v, beta, log_decay, o, true);
    if (st == DL_OK)
        st = check_handle_step_overlaps(s, q, k, v, beta, log_decay, o);
    if (st != DL_OK)
        return st;
    dl::StepArgs a = make_args(s);
    a.q = q;
    a.k = k;
    a.v = v;
    a.beta = beta;
    a.ld = log_decay;
    a.o = o;
    if (s->per_slot) { // every slot appends or merges by its own phase
        if (launch_step(s->op, s->dtype, s->dk, s->dv, dl::SSTEP, a, static_cast<hipStream_t>(stream)) !=
            hipSuccess)
            return DL_E_HIP;
        s->tm = (s->tm + 1) % s->M;
        return DL_OK;
    }
    const bool merge = s->n + 1 == s->M;
    if (launch_step(s->op, s->dtype, s->dk, s->dv, merge ? dl::FMERGE : dl::FAPPEND, a,
                    static_cast<hipStream_t>(stream)) !=
        hipSuccess)
        return DL_E_HIP;
    s->n = merge ? 0 : s->n + 1;
    return DL_OK;
}

dl_status dl_decode_step_staged_noalloc(dl_state *s, const void *q, const void *k, const void *v,
                                        const float *beta, const float *log_decay, float *o,
                                        void *stream)
{
    if (!s)
        return DL_E_INVALID;
    if (s->prepped || s->per_slot)
        return DL_E_STATE;
    dl_status st = check_step_ptrs(s->op, s->dtype, q, k, v, beta, log_decay, o, true);
    if (st == DL_OK)
        st = check_handle_step_overlaps(s, q, k, v, beta, log_decay, o);
    if (st != DL_OK)
        return st;
    if ((size_t)s->B * s->H * s->lay.cstride > dl::kScratchFloats)
        return DL_E_SCRATCH;
    float *coef = nullptr;
    if (dl::scratch_on_current_device(&coef) != hipSuccess)
        return DL_E_HIP;
    dl::StepArgs a = make_args(s);
    a.coef = coef; // the coefficient rows live in the static scratch, not the workspace
    a.q = q;
    a.k = k;
    a.v = v;
    a.beta = beta;
    a.ld = log_decay;
    a.o = o;
    const hipStream_t hs = static_cast<hipStream_t>(stream);
    const bool merge = s->n + 1 == s->M;
    if (launch_prep(s->op, s->dtype, s->dk, a, hs) != hipSuccess ||
        launch_step(s->op, s->dtype, s->dk, s->dv, merge ? dl::MERGE : dl::APPEND, a, hs) != hipSuccess)
        return DL_E_HIP;
    s->n = merge ? 0 : s->n + 1;
    return DL_OK;
}

dl_status dl_merge(dl_state *s, void *stream)
{
    if (!s)
        return DL_E_INVALID;
    if (s->prepped)
        return DL_E_STATE;
    if (s->per_slot) {
        dl::StepArgs a = make_args(s);
        const hipStream_t st = static_cast<hipStream_t>(stream);
        if (launch_step(s->op, s->dtype, s->dk, s->dv, dl::SFOLD, a, st) != hipSuccess ||
            dl::launch_slot_phase(slot_phases(s), s->B, -1, s->tm, true, st) != hipSuccess)
            return DL_E_HIP;
        for (int b = 0; b < s->B; ++b)
            if (s->t0[b] >= 0)
                s->t0[b] = s->tm;
        return DL_OK;
    }
    if (s->n == 0)
        return DL_OK;
    dl::StepArgs a = make_args(s);
    if (launch_step(s->op, s->dtype, s->dk, s->dv, dl::FOLD, a, static_cast<hipStream_t>(stream)) !=
        hipSuccess)
        return DL_E_HIP;
    s->n = 0;
    return DL_OK;
}

dl_status dl_state_reset(dl_state *s)
{
    if (!s)
        return DL_E_INVALID;
    if (s->per_slot)
        return DL_E_STATE;
    s->n = 0;
    s->prepped = false;
    return DL_OK;
}

int dl_log_len(const dl_state *s) { return (s && !s->per_slot) ? s->n : -1; }

dl_status dl_set_log_len(dl_state *s, int n)
{
    if (!s)
        return DL_E_INVALID;
    if (n < 0 || n >= s->M)
        return DL_E_INVALID;
    if (s->prepped || s->per_slot)
        return DL_E_STATE;
    s->n = n;
    return DL_OK;
}

dl_status dl_state_destroy(dl_state *s)
{
    if (s)
        delete[] s->t0;
    delete s;
    return DL_OK;
}

dl_status dl_state_enable_slots(dl_state *s, void *stream)
{
    if (!s)
        return DL_E_INVALID;
    if (s->prepped || s->n != 0 || s->per_slot)
        return DL_E_STATE;
    if (dl::launch_slot_phase(slot_phases(s), s->B, -1, 0, false, static_cast<hipStream_t>(stream)) !=
        hipSuccess)
        return DL_E_HIP;
    s->per_slot = true;
    s->tm = 0;
    for (int b = 0; b < s->B; ++b)
        s->t0[b] = 0;
    return DL_OK;
}

dl_status dl_slot_admit(dl_state *s, int slot, void *stream)
{
    if (!s || slot < 0 || slot >= s->B)
        return DL_E_INVALID;
    if (!s->per_slot)
        return DL_E_STATE;
    if (dl::launch_slot_phase(slot_phases(s), s->B, slot, s->tm, false, static_cast<hipStream_t>(stream)) !=
        hipSuccess)
        return DL_E_HIP;
    s->t0[slot] = s->tm;
    return DL_OK;
}

dl_status dl_slot_release(dl_state *s, int slot, void *stream)
{
    if (!s || slot < 0 || slot >= s->B)
        return DL_E_INVALID;
    if (!s->per_slot)
        return DL_E_STATE;
    if (dl::launch_slot_phase(slot_phases(s), s->B, slot, -1, false, static_cast<hipStream_t>(stream)) !=
        hipSuccess)
        return DL_E_HIP;
    s->t0[slot] = -1;
    return DL_OK;
}

dl_status dl_slot_merge(dl_state *s, int slot, void *stream)
{
    if (!s || slot < 0 || slot >= s->B)
        return DL_E_INVALID;
    if (!s->per_slot)
        return DL_E_STATE;
    if (dl_slot_log_len(s, slot) == 0) // nothing pending, or a released slot
        return DL_OK;
    dl::StepArgs a = make_args(s);
    a.slot = slot;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (launch_step(s->op, s->dtype, s->dk, s->dv, dl::SFOLD, a, st) != hipSuccess ||
        dl::launch_slot_phase(slot_phases(s), s->B, slot, s->tm, false, st) != hipSuccess)
        return DL_E_HIP;
    s->t0[slot] = s->tm;
    return DL_OK;
}

int dl_slot_log_len(const dl_state *s, int slot)
{
    if (!s || slot < 0 || slot >= s->B)
        return -1;
    if (!s->per_slot)
        return s->n;
    if (s->t0[slot] < 0) // released: no request, nothing pending
        return 0;
    return (s->tm - s->t0[slot] + s->M) % s->M;
}

dl_status dl_eager_step(dl_op op, int B, int H, int d_k, int d_v, dl_dtype in_dtype, float *S,
                        const void *q, const void *k, const void *v, const float *beta,
                        const float *log_decay, const float *u, float *o, void *stream)
{
    dl_status st = check_shape(B, H, d_k, d_v, 1, op, in_dtype);
    if (st != DL_OK)
        return st;
    if (!S || (op == DL_OP_RWKV6 && !u))
        return DL_E_INVALID;
    st = check_step_ptrs(op, in_dtype, q, k, v, beta, log_decay, o, true);
    if (st != DL_OK)
        return st;
    if (!aligned(S, 16) || (u && !aligned(u, 4)))
        return DL_E_ALIGN;
    {
        const StepSpans sp = step_spans(op, in_dtype, B, H, d_k, d_v, q, k, v, beta, log_decay,
                                        op == DL_OP_RWKV6 ? u : nullptr, o, S);
        const Span w[2] = {sp.o, sp.base};
        const Span r[6] = {sp.q, sp.k, sp.v, sp.beta, sp.ld, sp.u};
        if (check_overlaps(w, 2, r, 6) != DL_OK)
            return DL_E_INVALID;
    }
    dl::StepArgs a{};
    a.BH = B * H;
    a.H = H;
    a.M = 1;
    a.n = 0;
    a.q = q;
    a.k = k;
    a.v = v;
    a.beta = beta;
    a.ld = log_decay;
    a.u = op == DL_OP_RWKV6 ? u : nullptr;
    a.base = S;
    a.o = o;
    if (launch_step(op, in_dtype, d_k, d_v, dl::EAGER, a, static_cast<hipStream_t>(stream)) !=
        hipSuccess)
        return DL_E_HIP;
    return DL_OK;
}

int dl_suggest_merge_interval(int B, int H, int d_k, int d_v, dl_op op, dl_dtype in_dtype)
{
    if (check_shape(B, H, d_k, d_v, 1, op, in_dtype) != DL_OK)
        return 0;
    const double es = in_dtype == DL_BF16 ? 2.0 : 4.0;
    const double P = 4.0 * d_k * d_v;
    const double lsz = op == DL_OP_GDN ? 4.0 : 4.0 * d_k;
    const double e_key = d_k * es + lsz;
    const double e_val = d_v * (op == DL_OP_RWKV6 ? es : 4.0);
    // value tiles per slot-head, each re-reading the key side: 64-column
    // tiles, except KDA's appends at d_v = 128, which take whole rows (as the
    // step kernel does); a merge always takes 64-column tiles
    const double tiles_merge = d_v / (double)(d_v < 64 ? d_v : 64);
    const double tiles = (op == DL_OP_KDA && d_v == 128) ? 1.0 : tiles_merge;
    int best = 1;
    double best_bytes = 0.0;
    for (int M = 1; M <= 32; ++M) {
        const double bytes = P * (1.0 + 1.0 / M) + 0.5 * (M - 1) * (e_key * tiles + e_val) +
                             (double)(M - 1) / M * (e_key + e_val) +
                             (tiles_merge - tiles) * (double)(M - 1) / M * e_key; // the merge's extra reads
        if (M == 1 || bytes < best_bytes) {
            best = M;
            best_bytes = bytes;
        }
    }
    return best;
}

int dl_choose_merge_interval(const double *append_us, const double *merge_us, int max_M)
{
    if (!append_us || !merge_us || max_M < 1 || max_M > 32)
        return 0;
    for (int n = 0; n < max_M; ++n) {
        const double a = n + 1 < max_M ? append_us[n] : 0.0, m = merge_us[n];
        if (!(a >= 0.0) || !(m >= 0.0) || a > 1e30 || m > 1e30) // NaN fails >= 0
            return 0;
    }
    int best = 1;
    double best_t = 0.0, appends = 0.0; // appends = sum of append_us[0..M-2]
    for (int M = 1; M <= max_M; ++M) {
        if (M >= 2)
            appends += append_us[M - 2];
        const double t = (appends + merge_us[M - 1]) / M;
        if (M == 1 || t < best_t) {
            best = M;
            best_t = t;
        }
    }
    return best;
}

const char *dl_status_string(dl_status st)
{
    switch (st) {
    case DL_OK: return "ok";
    case DL_E_INVALID: return "invalid argument";
    case DL_E_SHAPE: return "unsupported shape";
    case DL_E_ALIGN: return "misaligned pointer";
    case DL_E_HIP: return "HIP launch failed";
    case DL_E_STATE: return "call out of order";
    case DL_E_SCRATCH: return "shape needs more scratch than the library's static buffer holds";
    }
    return "unknown status";
}

} // extern "C"
