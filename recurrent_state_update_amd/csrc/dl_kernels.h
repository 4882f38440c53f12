// dl_kernels.h -- the HIP kernels of libdeltalog for gfx950 (CDNA4, wave64),
// as templates instantiated once per operator in dl_gdn.hip / dl_kda.hip /
// dl_rwkv6.hip.
//
// Method: DeltaLog (arXiv 2608.15533).  The gist.science technical summary,
// section "Kernel implementation", splits the step into a ReplayPrep stage run
// once per slot-head (coefficients shared by every value tile) and an
// AppendDecode stage that is parallel over tiles of the value dimension d_v,
// each tile owning a slice of the dense base and the matching value-side log
// shard; "Core mechanism: Base + Log" gives the append and merge phases.
//
// Notation (one slot-head): X-bar is the d_k x d_v fp32 base, row i = key i.
// Log entry j < n holds a_j = k_j (input dtype), b_j (fp32 for the delta rule,
// input dtype for RWKV6) and Lam_j, the cumulative log-decay since the last
// merge (one float for GDN, d_k floats for KDA and RWKV6).  Lam' = Lam_{n-1} +
// ell_t (Lam_{-1} = 0).  The logical state after entries 0..n-1 is
//   X = e^{Lam_{n-1}} (.)row X-bar + sum_j (e^{Lam_{n-1} - Lam_j} (.) a_j) b_j^T.
// Decayed state X' = D_t X, so for the delta rule
//   X'^T k = X-bar^T (e^{Lam'} (.) k) + sum_j c^k_j b_j,
//   c^k_j = sum_i e^{Lam'_i - Lam_j,i} a_j,i k_i       (same for q),
//   b_t = beta (v - X'^T k),  o_t = X'^T q + (q.k) b_t.
// RWKV6 reads the state before the step: o_t = X-bar^T (e^{Lam_{n-1}} (.) r)
// + sum_j c^r_j b_j + (r.(u (.) k)) v.  A merge folds entries to
//   X-bar <- e^{Lam_f} (.)row X-bar + sum_j (e^{Lam_f - Lam_j} (.) a_j) b_j^T.
// Only exponents <= 0 are ever taken (differences of cumulative log-decays).
//
// Hardware mapping.  The step is a matrix-vector product plus (on merges) a
// rank-M update: ~1-2 flop per state byte, far under the fp32 balance, so it is
// HBM-bound and uses no MFMA.  Each workgroup owns one (slot-head, value tile
// of T columns).  A lane owns 4 adjacent columns (one 128-bit load per row) and
// P rows; a row of T columns is read by T/4 adjacent lanes, so a wave's load
// covers whole contiguous row segments.  All P row loads are issued before any
// use.  Column sums over rows reduce across lanes with xor-shuffles and across
// waves through LDS; the small per-step metadata (value-side log shard,
// coefficients, fold table) is staged in LDS while the base loads are in
// flight.  Workgroups of one slot-head are placed on the same XCD.
#pragma once

#include "dl_internal.h"

#ifndef DL_TILE_MAX
#define DL_TILE_MAX 64 // widest value tile (columns) per workgroup
#endif
#ifndef DL_THREADS_MAX
#define DL_THREADS_MAX 256 // threads per workgroup of the state kernel
#endif

namespace dl {

// ------------------------------------------------------------------ helpers --

template <typename TIn> __device__ __forceinline__ float load_in(const TIn *p, long i);
template <> __device__ __forceinline__ float load_in<float>(const float *p, long i) { return p[i]; }
// bf16 held as its 16 raw bits: the fp32 with the same upper half
template <> __device__ __forceinline__ float load_in<uint16_t>(const uint16_t *p, long i)
{
    return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}

// Sum over the lanes of a wave64 whose lane ids differ only in bits >= log2(FROM).
template <int FROM> __device__ __forceinline__ float wave_sum_from(float x)
{
#pragma unroll
    for (int off = FROM; off < 64; off <<= 1)
        x += __shfl_xor(x, off, 64);
    return x;
}

// Workgroup b of a 1-D grid is dispatched to XCD b % 8.  Renumber so each XCD
// works on a contiguous range of logical tiles (tiles of one slot-head then
// share that XCD's L2 for their common metadata).  Bijective on [0, G).
__device__ __forceinline__ int xcd_remap(int b, int G)
{
    constexpr int NX = 8;
    const int per = G / NX;
    if (b >= per * NX)
        return b;
    return (b % NX) * per + b / NX;
}

template <int DK, int DV> struct TileCfg {
    static constexpr int T = DV < DL_TILE_MAX ? DV : DL_TILE_MAX;            // tile columns
    static constexpr int NT = DK * T / 4 < DL_THREADS_MAX ? DK * T / 4 : DL_THREADS_MAX; // threads
    static constexpr int LPR = T / 4;     // lanes per row
    static constexpr int RPP = NT / LPR;  // rows per pass of the workgroup
    static constexpr int P = DK / RPP;    // rows per lane
    static constexpr int NTILE = DV / T;
    static constexpr int NW = (NT + 63) / 64;
    static_assert(P * RPP == DK && LPR <= 32 && NT % LPR == 0, "tile shape");
};

// Rows of the staged value-side factors and of the fold table for a launch.
__host__ __device__ constexpr int bt_rows(int mode, int n)
{
    return mode == FOLD ? n : mode == EAGER ? 1 : n + 1;
}
__host__ __device__ constexpr int fold_rows(int mode, int n)
{
    return mode == MERGE ? n + 1 : mode == EAGER ? 1 : mode == FOLD ? n : 0;
}
// Dynamic LDS floats: Bt [bt_rows][T], F [fold_rows][DK], coefficients [2n+1].
__host__ __device__ constexpr int dyn_floats(int mode, int n, int DK, int T)
{
    return bt_rows(mode, n) * T + fold_rows(mode, n) * DK +
           ((mode == APPEND || mode == MERGE) ? 2 * n + 1 : 0);
}

// ------------------------------------------------------------- ReplayPrep --
//
// One wave64 per slot-head, four slot-heads per workgroup.  Per slot-head:
// Lam' = Lam_{n-1} + ell_t; coefficients c^q_j, c^k_j (RWKV6: c^r_j against
// Lam_{n-1}) for the n logged entries; kappa = q.k (RWKV6: r.(u (.) k)); then
// the key-side append a_n = k, Lam_n = Lam'.  coef row: [c^q_0..M-1,
// c^k_0..M-1, kappa].
template <int OP, typename TIn, int DK>
__global__ __launch_bounds__(256) void replay_prep_kernel(StepArgs a)
{
    constexpr int KPL = (DK + 63) / 64; // keys per lane
    const int lane = threadIdx.x & 63;
    const int sh = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (sh >= a.BH)
        return; // whole wave leaves together
    const int n = a.n, M = a.M;
    const TIn *q = static_cast<const TIn *>(a.q) + (long)sh * DK;
    const TIn *k = static_cast<const TIn *>(a.k) + (long)sh * DK;
    const TIn *alog = static_cast<const TIn *>(a.alog) + (long)sh * M * DK;
    float *L = a.Llog + (OP == GDN ? (long)sh * M : (long)sh * M * DK);

    float qv[KPL], kv[KPL], lp[KPL], lw[KPL];
#pragma unroll
    for (int c = 0; c < KPL; ++c) {
        const int i = lane + 64 * c;
        const bool ok = i < DK;
        qv[c] = ok ? load_in(q, i) : 0.f;
        kv[c] = ok ? load_in(k, i) : 0.f;
        if (OP == GDN) {
            lp[c] = n > 0 ? L[n - 1] : 0.f;
            lw[c] = lp[c] + a.ld[sh];
        } else {
            lp[c] = (ok && n > 0) ? L[(long)(n - 1) * DK + i] : 0.f;
            lw[c] = lp[c] + (ok ? a.ld[(long)sh * DK + i] : 0.f);
        }
    }

    float *coef = a.coef + (long)sh * a.cstride;
    for (int m = 0; m < n; ++m) {
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int c = 0; c < KPL; ++c) {
            const int i = lane + 64 * c;
            if (i < DK) {
                const float am = load_in(alog, (long)m * DK + i);
                float e;
                if (OP == GDN)
                    e = am; // scalar decay factor applied after the sum
                else if (OP == KDA)
                    e = expf(lw[c] - L[(long)m * DK + i]) * am;
                else
                    e = expf(lp[c] - L[(long)m * DK + i]) * am;
                sq += e * qv[c];
                sk += e * kv[c];
            }
        }
        sq = wave_sum_from<1>(sq);
        if (OP != RWKV6)
            sk = wave_sum_from<1>(sk);
        if (OP == GDN) {
            const float s = expf(lw[0] - L[m]);
            sq *= s;
            sk *= s;
        }
        if (lane == 0) {
            coef[m] = sq;
            if (OP != RWKV6)
                coef[M + m] = sk;
        }
    }

    float kap = 0.f;
#pragma unroll
    for (int c = 0; c < KPL; ++c) {
        const int i = lane + 64 * c;
        if (i < DK)
            kap += OP == RWKV6 ? qv[c] * a.u[(long)(sh % a.H) * DK + i] * kv[c] : qv[c] * kv[c];
    }
    kap = wave_sum_from<1>(kap);
    if (lane == 0)
        coef[2 * M] = kap;

    // key-side append of entry n
    TIn *an = static_cast<TIn *>(a.alog) + ((long)sh * M + n) * DK;
#pragma unroll
    for (int c = 0; c < KPL; ++c) {
        const int i = lane + 64 * c;
        if (i < DK) {
            an[i] = k[i];
            if (OP != GDN)
                L[(long)n * DK + i] = lw[c];
        }
    }
    if (OP == GDN && lane == 0)
        L[n] = lw[0];
}

// ------------------------------------------------------------ state kernel --
//
// AppendDecode (APPEND, MERGE), the eager baseline (EAGER) and the standalone
// merge (FOLD) share this body; MODE selects which parts run.
//   reads   (APPEND, MERGE, EAGER): y = X-bar^T w over the tile, outputs o_t
//           and the value-side factor b_t of this step;
//   writes  (MERGE, EAGER, FOLD):   fold entries into the tile, one store.
template <int OP, typename TIn, int DK, int DV, int MODE>
__global__ __launch_bounds__((TileCfg<DK, DV>::NT)) void state_kernel(StepArgs a)
{
    using C = TileCfg<DK, DV>;
    constexpr int T = C::T, NT = C::NT, LPR = C::LPR, RPP = C::RPP, P = C::P;
    constexpr int NTILE = C::NTILE, NW = C::NW;
    constexpr bool DELTA = OP != RWKV6;
    constexpr bool READS = MODE != FOLD;
    constexpr bool WRITES = MODE != APPEND;
    constexpr bool LOGGED = MODE == APPEND || MODE == MERGE; // uses ReplayPrep's output
    constexpr int NV = 9; // reduced values per column group: 4 yq, 4 yk, kappa

    extern __shared__ float4 dyn4[];
    float *dyn = reinterpret_cast<float *>(dyn4);
    __shared__ float red[NW][LPR][NV];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int c4 = tid % LPR, r0 = tid / LPR;
    const int blk = xcd_remap(blockIdx.x, gridDim.x);
    const int sh = blk / NTILE, tile = blk % NTILE;
    const int col = tile * T + 4 * c4;
    const int M = a.M, n = a.n;

    // 1. issue the whole tile's loads: P rows x 128 bits per lane
    float *S = a.base + (long)sh * DK * DV;
    float4 x[P];
#pragma unroll
    for (int p = 0; p < P; ++p)
        x[p] = *reinterpret_cast<const float4 *>(S + (long)(r0 + p * RPP) * DV + col);

    const TIn *q = static_cast<const TIn *>(a.q) + (long)sh * DK;
    const TIn *k = static_cast<const TIn *>(a.k) + (long)sh * DK;
    const float *L = a.Llog + (OP == GDN ? (long)sh * M : (long)sh * M * DK);

    const int nb = bt_rows(MODE, n), nf = fold_rows(MODE, n);
    float *Bt = dyn;                                  // [nb][T] value-side factors, this tile
    float *F = Bt + nb * T;                           // [nf][DK] key-side fold coefficients
    float *cf = F + (WRITES ? nf * DK : 0);           // [2n+1] c^q, c^k, kappa

    // 2. stage the value-side log shard of this tile (entries < n) in LDS
    const int nlog = (MODE == EAGER) ? 0 : n;
    for (int idx = tid; idx < nlog * (T / 4); idx += NT) {
        const int m = idx / (T / 4), j4 = idx % (T / 4);
        const long off = ((long)sh * M + m) * DV + tile * T + 4 * j4;
        float4 b;
        if (DELTA) {
            b = *reinterpret_cast<const float4 *>(static_cast<const float *>(a.blog) + off);
        } else {
            const TIn *bl = static_cast<const TIn *>(a.blog);
            b = make_float4(load_in(bl, off), load_in(bl, off + 1), load_in(bl, off + 2),
                            load_in(bl, off + 3));
        }
        *reinterpret_cast<float4 *>(Bt + m * T + 4 * j4) = b;
    }
    if (LOGGED) {
        const float *coef = a.coef + (long)sh * a.cstride;
        for (int idx = tid; idx < 2 * n + 1; idx += NT)
            cf[idx] = idx < n ? coef[idx] : idx < 2 * n ? coef[M + idx - n] : coef[2 * M];
    }
    // 3. fold table: F[m][i] = e^{Lam_f,i - Lam_m,i} a_m,i for logged entries,
    //    k_i for this step's entry (MERGE, EAGER)
    if (WRITES) {
        const TIn *alog = static_cast<const TIn *>(a.alog) + (long)sh * M * DK;
        const int lf = MODE == FOLD ? n - 1 : n;
        for (int idx = tid; idx < nf * DK; idx += NT) {
            const int m = idx / DK, i = idx % DK;
            float f;
            if (MODE == EAGER || (MODE == MERGE && m == n)) {
                f = load_in(k, i);
            } else {
                const float lfv = OP == GDN ? L[lf] : L[(long)lf * DK + i];
                const float lm = OP == GDN ? L[m] : L[(long)m * DK + i];
                f = expf(lfv - lm) * load_in(alog, (long)m * DK + i);
            }
            F[idx] = f;
        }
    }
    // prefetch what the finalising lanes need
    float4 vv = make_float4(0.f, 0.f, 0.f, 0.f);
    float bet = 0.f;
    if (READS && tid < LPR) {
        const TIn *v = static_cast<const TIn *>(a.v) + (long)sh * DV + col;
        vv = make_float4(load_in(v, 0), load_in(v, 1), load_in(v, 2), load_in(v, 3));
        if (DELTA)
            bet = a.beta[sh];
    }

    // 4. column sums y_q = X-bar^T w_q, y_k = X-bar^T w_k over this lane's rows
    float rowf[P]; // per-row base factor for the fold (KDA, RWKV6)
    if (READS) {
        float yq[4] = {0.f, 0.f, 0.f, 0.f}, yk[4] = {0.f, 0.f, 0.f, 0.f}, kap = 0.f;
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int r = r0 + p * RPP;
            const float qr = load_in(q, r), kr = load_in(k, r);
            float wq = qr, wk = kr;
            if (OP == KDA) {
                const float lnew = MODE == EAGER ? a.ld[(long)sh * DK + r] : L[(long)n * DK + r];
                const float e = expf(lnew);
                wq *= e;
                wk *= e;
                rowf[p] = e;
            } else if (OP == RWKV6) {
                const float lprev = (MODE == EAGER || n == 0) ? 0.f : L[(long)(n - 1) * DK + r];
                wq *= expf(lprev);
                if (WRITES)
                    rowf[p] = expf(MODE == EAGER ? a.ld[(long)sh * DK + r] : L[(long)n * DK + r]);
            }
            if (MODE == EAGER && c4 == 0)
                kap += DELTA ? qr * kr : qr * a.u[(long)(sh % a.H) * DK + r] * kr;
            const float xs[4] = {x[p].x, x[p].y, x[p].z, x[p].w};
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                yq[c] = fmaf(wq, xs[c], yq[c]);
                if (DELTA)
                    yk[c] = fmaf(wk, xs[c], yk[c]);
            }
        }
        float vals[NV] = {yq[0], yq[1], yq[2], yq[3], yk[0], yk[1], yk[2], yk[3], kap};
#pragma unroll
        for (int c = 0; c < NV; ++c) {
            if (!DELTA && c >= 4 && c < 8)
                continue;
            if (MODE != EAGER && c == 8)
                continue;
            vals[c] = wave_sum_from<LPR>(vals[c]);
        }
        if (lane < LPR) {
#pragma unroll
            for (int c = 0; c < NV; ++c)
                red[wave][lane][c] = vals[c];
        }
    } else if (OP != GDN) {
        // FOLD: per-row base factor e^{Lam_{n-1}}
#pragma unroll
        for (int p = 0; p < P; ++p)
            rowf[p] = expf(L[(long)(n - 1) * DK + r0 + p * RPP]);
    }
    __syncthreads();

    // 5. finalise this tile's outputs (one lane per 4 columns)
    if (READS) {
        if (tid < LPR) {
            float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            float kap = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
#pragma unroll
                for (int c = 0; c < 8; ++c)
                    y[c] += red[w][tid][c];
                kap += red[w][0][8];
            }
            if (OP == GDN) {
                const float s = expf(MODE == EAGER ? a.ld[sh] : L[n]);
#pragma unroll
                for (int c = 0; c < 8; ++c)
                    y[c] *= s;
            }
            float rq[4] = {0.f, 0.f, 0.f, 0.f}, rk[4] = {0.f, 0.f, 0.f, 0.f};
            if (LOGGED) {
                kap = cf[2 * n];
                for (int m = 0; m < n; ++m) {
                    const float4 b = *reinterpret_cast<const float4 *>(Bt + m * T + 4 * c4);
                    const float bs[4] = {b.x, b.y, b.z, b.w};
                    const float cq = cf[m], ck = cf[n + m];
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        rq[c] = fmaf(cq, bs[c], rq[c]);
                        if (DELTA)
                            rk[c] = fmaf(ck, bs[c], rk[c]);
                    }
                }
            }
            const float vs[4] = {vv.x, vv.y, vv.z, vv.w};
            float bt[4], ov[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if (DELTA) {
                    bt[c] = bet * (vs[c] - y[4 + c] - rk[c]);
                    ov[c] = y[c] + rq[c] + kap * bt[c];
                } else {
                    bt[c] = vs[c];
                    ov[c] = y[c] + rq[c] + kap * vs[c];
                }
            }
            *reinterpret_cast<float4 *>(a.o + (long)sh * DV + col) = make_float4(ov[0], ov[1], ov[2], ov[3]);
            if (LOGGED) { // value-side append of entry n
                const long off = ((long)sh * M + n) * DV + col;
                if (DELTA) {
                    *reinterpret_cast<float4 *>(static_cast<float *>(a.blog) + off) =
                        make_float4(bt[0], bt[1], bt[2], bt[3]);
                } else {
                    const TIn *v = static_cast<const TIn *>(a.v) + (long)sh * DV + col;
                    TIn *bl = static_cast<TIn *>(a.blog) + off;
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        bl[c] = v[c];
                }
            }
            if (WRITES)
                *reinterpret_cast<float4 *>(Bt + (nb - 1) * T + 4 * c4) = make_float4(bt[0], bt[1], bt[2], bt[3]);
        }
        if (WRITES)
            __syncthreads();
    }

    // 6. fold and write the tile once
    if (WRITES) {
        float gs = 1.f; // GDN: scalar base factor e^{Lam_f}
        if (OP == GDN)
            gs = expf(MODE == EAGER ? a.ld[sh] : MODE == FOLD ? L[n - 1] : L[n]);
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int r = r0 + p * RPP;
            const float bf = OP == GDN ? gs : rowf[p];
            float4 acc = make_float4(bf * x[p].x, bf * x[p].y, bf * x[p].z, bf * x[p].w);
            for (int m = 0; m < nf; ++m) {
                const float f = F[m * DK + r];
                const float4 b = *reinterpret_cast<const float4 *>(Bt + m * T + 4 * c4);
                acc.x = fmaf(f, b.x, acc.x);
                acc.y = fmaf(f, b.y, acc.y);
                acc.z = fmaf(f, b.z, acc.z);
                acc.w = fmaf(f, b.w, acc.w);
            }
            *reinterpret_cast<float4 *>(S + (long)r * DV + col) = acc;
        }
    }
}

// ---------------------------------------------------------------- launchers --

template <int OP, typename TIn, int DK>
hipError_t launch_prep_t(const StepArgs &a, hipStream_t st)
{
    const dim3 grid((a.BH + 3) / 4);
    hipLaunchKernelGGL((replay_prep_kernel<OP, TIn, DK>), grid, dim3(256), 0, st, a);
    return hipGetLastError();
}

template <int OP>
hipError_t launch_prep(int dtype, int dk, const StepArgs &a, hipStream_t st)
{
#define DL_PREP_CASE(D)                                                                \
    case D:                                                                            \
        return dtype == BF16 ? launch_prep_t<OP, uint16_t, D>(a, st)                   \
                             : launch_prep_t<OP, float, D>(a, st);
    switch (dk) {
        DL_PREP_CASE(16)
        DL_PREP_CASE(32)
        DL_PREP_CASE(64)
        DL_PREP_CASE(128)
    }
#undef DL_PREP_CASE
    return hipErrorInvalidValue;
}

template <int OP, typename TIn, int DK, int DV, int MODE>
hipError_t launch_state_t(const StepArgs &a, hipStream_t st)
{
    using C = TileCfg<DK, DV>;
    const dim3 grid((unsigned)a.BH * C::NTILE);
    const size_t lds = sizeof(float) * (size_t)dyn_floats(MODE, a.n, DK, C::T);
    hipLaunchKernelGGL((state_kernel<OP, TIn, DK, DV, MODE>), grid, dim3(C::NT), lds, st, a);
    return hipGetLastError();
}

template <int OP, typename TIn, int DK, int DV>
hipError_t launch_state_mode(int mode, const StepArgs &a, hipStream_t st)
{
    switch (mode) {
    case APPEND: return launch_state_t<OP, TIn, DK, DV, APPEND>(a, st);
    case MERGE: return launch_state_t<OP, TIn, DK, DV, MERGE>(a, st);
    case EAGER: return launch_state_t<OP, TIn, DK, DV, EAGER>(a, st);
    case FOLD: return launch_state_t<OP, TIn, DK, DV, FOLD>(a, st);
    }
    return hipErrorInvalidValue;
}

template <int OP, typename TIn, int DK>
hipError_t launch_state_dv(int dv, int mode, const StepArgs &a, hipStream_t st)
{
    switch (dv) {
    case 16: return launch_state_mode<OP, TIn, DK, 16>(mode, a, st);
    case 32: return launch_state_mode<OP, TIn, DK, 32>(mode, a, st);
    case 64: return launch_state_mode<OP, TIn, DK, 64>(mode, a, st);
    case 128: return launch_state_mode<OP, TIn, DK, 128>(mode, a, st);
    }
    return hipErrorInvalidValue;
}

template <int OP, typename TIn>
hipError_t launch_state_dk(int dk, int dv, int mode, const StepArgs &a, hipStream_t st)
{
    switch (dk) {
    case 16: return launch_state_dv<OP, TIn, 16>(dv, mode, a, st);
    case 32: return launch_state_dv<OP, TIn, 32>(dv, mode, a, st);
    case 64: return launch_state_dv<OP, TIn, 64>(dv, mode, a, st);
    case 128: return launch_state_dv<OP, TIn, 128>(dv, mode, a, st);
    }
    return hipErrorInvalidValue;
}

template <int OP>
hipError_t launch_state(int dtype, int dk, int dv, int mode, const StepArgs &a, hipStream_t st)
{
    return dtype == BF16 ? launch_state_dk<OP, uint16_t>(dk, dv, mode, a, st)
                         : launch_state_dk<OP, float>(dk, dv, mode, a, st);
}

} // namespace dl
