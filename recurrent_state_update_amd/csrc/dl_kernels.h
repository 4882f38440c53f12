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
// input dtype for RWKV6) and ell_j, the log-decay of the step that appended it
// (one float for GDN, d_k floats for KDA and RWKV6).  The pages' log-decay
// snapshot is their running sum Lam_j = ell_0 + ... + ell_j, the cumulative
// log-decay since the last merge; Lam' = Lam_{n-1} + ell_t (Lam_{-1} = 0).
// The logical state after entries 0..n-1 is
//   X = e^{Lam_{n-1}} (.)row X-bar + sum_j (e^{Lam_{n-1} - Lam_j} (.) a_j) b_j^T.
// Decayed state X' = D_t X, so for the delta rule
//   X'^T k = X-bar^T (e^{Lam'} (.) k) + sum_j c^k_j b_j,
//   c^k_j = sum_i e^{Lam'_i - Lam_j,i} a_j,i k_i       (same for q),
//   b_t = beta (v - X'^T k),  o_t = X'^T q + (q.k) b_t.
// RWKV6 reads the state before the step: o_t = X-bar^T (e^{Lam_{n-1}} (.) r)
// + sum_j c^r_j b_j + (r.(u (.) k)) v.  A merge folds entries to
//   X-bar <- e^{Lam_f} (.)row X-bar + sum_j (e^{Lam_f - Lam_j} (.) a_j) b_j^T.
// Every exponent is a sum of consecutive ell's, Lam_{n-1} - Lam_j = ell_{j+1}
// + ... + ell_{n-1}, formed by adding the logged ell's directly (suffix sums),
// never as the difference of two cumulative values: all terms are <= 0, so
// the sums are exact to a few ulps of their own size and exponents are <= 0.
//
// Hardware mapping.  The step is a matrix-vector product plus (on merges) a
// rank-M update: ~1-2 flop per state byte, far under the fp32 balance, so it is
// HBM-bound and uses no MFMA.  Each workgroup owns one (slot-head, value tile
// of T columns).  A lane owns 4 adjacent columns (one 128-bit load per row) and
// P rows; a row of T columns is read by T/4 adjacent lanes, so a wave's load
// covers whole contiguous row segments.  All loads of a workgroup are issued
// before any is used: the small ones (row metadata, the tile's log shard,
// coefficients) first, then the P base rows, so the workgroup waits on memory
// once.  Loads that a lane does not need are pointed past the end of a
// bounds-limited buffer resource: they return zero without touching memory,
// which keeps the code branch-free (no load gets sunk behind a wait) and adds
// no traffic.  Column sums reduce across lanes in registers (DPP row rotations
// and the permlane swaps) and across waves through LDS.  Register use is kept
// at or under 64 VGPRs on the hot modes where it can be, which lets eight
// waves share a SIMD.
#pragma once

#include <hip/hip_runtime.h>

#include "dl_internal.h"

#ifndef DL_TILE_MAX
#define DL_TILE_MAX 64 // widest value tile (columns) per workgroup
#endif
#ifndef DL_MAX_M
#define DL_MAX_M 32 // largest merge interval
#endif
#ifndef DL_THREADS_MAX
#define DL_THREADS_MAX 256 // threads per workgroup of the step kernel
#endif

namespace dl {

// ------------------------------------------------------------------ helpers --

// Sum over the lanes of a wave64 whose lane ids differ only in bits >= log2(FROM)
// (FROM a power of two), left in every lane.  Everything stays in registers:
//   - within a 16-lane row, adding the row rotated by FROM, 2 FROM, ..., 8
//     (DPP row_ror) leaves each lane the sum of the lanes of its row that share
//     its low bits;
//   - across rows, v_permlane16_swap applied to two copies of x returns rows
//     (r0, r0, r2, r2) and (r1, r1, r3, r3), whose sum is the xor-16 sum, and
//     v_permlane32_swap likewise gives the xor-32 sum.
// Call with the whole wave active.
template <int ROR> __device__ __forceinline__ float add_row_ror(float x)
{
    return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + ROR, 0xF, 0xF, false));
}
template <int FROM> __device__ __forceinline__ float wave_sum_from(float x)
{
    static_assert(FROM >= 1 && FROM <= 32 && (FROM & (FROM - 1)) == 0, "power of two");
    if constexpr (FROM <= 1) x = add_row_ror<1>(x);
    if constexpr (FROM <= 2) x = add_row_ror<2>(x);
    if constexpr (FROM <= 4) x = add_row_ror<4>(x);
    if constexpr (FROM <= 8) x = add_row_ror<8>(x);
    if constexpr (FROM <= 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
    }
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Full forgetting.  A log-decay of -inf (e^ell = 0: the step erases the
// history) would make the cumulative Lam infinite, and a later difference
// Lam' - Lam_j would be -inf - (-inf), which is undefined.  Every log-decay is
// therefore taken at no less than kMinLogDecay.  At that value e^ell is
// already exactly 0 in fp32, so such a step still erases every older term
// exactly, while Lam stays finite.  A NaN passes through unchanged.
constexpr float kMinLogDecay = -112.f;
__device__ __forceinline__ float floor_log_decay(float x) { return x < kMinLogDecay ? kMinLogDecay : x; }

// Raw buffer resources: a base, a size in bytes, and loads at a 32-bit byte
// offset (per lane) plus a wave-uniform offset.  An access at or past the size
// reads zero and touches no memory; stores there are dropped.
using rsrc_t = __amdgpu_buffer_rsrc_t;
using u32x2 = unsigned int __attribute__((ext_vector_type(2)));
using u32x4 = unsigned int __attribute__((ext_vector_type(4)));
constexpr int kBufferDword3 = 0x00020000;   // raw buffer, 32-bit data format (CDNA)
constexpr unsigned kSkip = 0x80000000u;     // a byte offset past every resource here
constexpr unsigned kSkipElem = 0x20000000u; // an element index past every resource here
                                            // (x4 bytes still fits 32 bits)

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, unsigned bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, kBufferDword3);
}
__device__ __forceinline__ float4 buf_ld4(rsrc_t r, unsigned off, unsigned soff = 0)
{
    return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0));
}
// Streaming form for the state tile, which each step reads exactly once: the
// non-temporal hint (cache-policy bit "nt") keeps it from displacing the
// reused data (log entries, inputs) in the caches; measured ~12% faster per
// step on MI355X.
constexpr int kNonTemporal = 2;
__device__ __forceinline__ float4 buf_ld4_stream(rsrc_t r, unsigned off, unsigned soff)
{
    return __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, kNonTemporal));
}
__device__ __forceinline__ void buf_st4(rsrc_t r, unsigned off, unsigned soff, float4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, soff, 0);
}
// Streaming store of a state tile: used by the eager step, which rewrites the
// whole state every step (measured ~10% faster per eager step).  The DeltaLog
// merge keeps the default policy: the hint sped up back-to-back merges but not
// a merge cycle, whose appends otherwise absorb the write-back.
__device__ __forceinline__ void buf_st4_stream(rsrc_t r, unsigned off, unsigned soff, float4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, soff, kNonTemporal);
}
__device__ __forceinline__ float buf_ldf(rsrc_t r, unsigned off)
{
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
// One input element (fp32, or bf16 as its 16 raw bits) at element index e.
template <typename TIn> __device__ __forceinline__ float buf_ld_in(rsrc_t r, unsigned e);
template <> __device__ __forceinline__ float buf_ld_in<float>(rsrc_t r, unsigned e)
{
    return buf_ldf(r, e * 4u);
}
template <> __device__ __forceinline__ float buf_ld_in<uint16_t>(rsrc_t r, unsigned e)
{
    const unsigned short h = __builtin_amdgcn_raw_buffer_load_b16(r, e * 2u, 0, 0);
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
// Four consecutive input elements at element index e (a multiple of 4).
template <typename TIn> __device__ __forceinline__ float4 buf_ld4_in(rsrc_t r, unsigned e);
template <> __device__ __forceinline__ float4 buf_ld4_in<float>(rsrc_t r, unsigned e)
{
    return buf_ld4(r, e * 4u);
}
template <> __device__ __forceinline__ float4 buf_ld4_in<uint16_t>(rsrc_t r, unsigned e)
{
    const u32x2 h = __builtin_amdgcn_raw_buffer_load_b64(r, e * 2u, 0, 0);
    return make_float4(__uint_as_float(h[0] << 16), __uint_as_float(h[0] & 0xffff0000u),
                       __uint_as_float(h[1] << 16), __uint_as_float(h[1] & 0xffff0000u));
}
// An input-dtype value back from a float that holds one exactly.
template <typename TIn> __device__ __forceinline__ TIn to_in(float x);
template <> __device__ __forceinline__ float to_in<float>(float x) { return x; }
template <> __device__ __forceinline__ uint16_t to_in<uint16_t>(float x)
{
    return static_cast<uint16_t>(__float_as_uint(x) >> 16);
}

// Raw forms of the element loads: the bits are returned untouched and
// converted later, so a load inside a branch does not force a wait there
// (a conversion next to the load would).
// Raw bits of one element, always as a 32-bit word: fp32 loads the element;
// bf16 loads the aligned word that holds it (two adjacent lanes share a word,
// so the access stays coalesced) and cvt1 picks the half from the element
// index's parity.  Keeping 32-bit raw words means no zero-extension or
// packing has to sit next to the load.
template <typename TIn> __device__ __forceinline__ unsigned buf_raw1(rsrc_t r, unsigned e)
{
    if constexpr (sizeof(TIn) == 4)
        return __builtin_amdgcn_raw_buffer_load_b32(r, e * 4u, 0, 0);
    else
        return __builtin_amdgcn_raw_buffer_load_b32(r, (e & ~1u) * 2u, 0, 0);
}
template <typename TIn> __device__ __forceinline__ float cvt1(unsigned raw, unsigned e)
{
    if constexpr (sizeof(TIn) == 4)
        return __uint_as_float(raw);
    else
        return __uint_as_float((e & 1u) ? (raw & 0xffff0000u) : (raw << 16));
}
template <typename TIn> __device__ __forceinline__ u32x4 buf_raw4(rsrc_t r, unsigned e)
{
    if constexpr (sizeof(TIn) == 4) {
        return __builtin_amdgcn_raw_buffer_load_b128(r, e * 4u, 0, 0);
    } else {
        const u32x2 h = __builtin_amdgcn_raw_buffer_load_b64(r, e * 2u, 0, 0);
        return u32x4{h[0], h[1], 0u, 0u};
    }
}
template <typename TIn> __device__ __forceinline__ float4 cvt4(u32x4 raw)
{
    if constexpr (sizeof(TIn) == 4)
        return __builtin_bit_cast(float4, raw);
    else
        return make_float4(__uint_as_float(raw[0] << 16), __uint_as_float(raw[0] & 0xffff0000u),
                           __uint_as_float(raw[1] << 16), __uint_as_float(raw[1] & 0xffff0000u));
}

// The value tile of one launch: 64 columns, with 256 threads (8 rows per lane
// at d_k = 128) or 512 (4 rows per lane), except where whole rows (128
// columns, 512 threads, d_v = 128) measured faster.  Per decode step, with 4
// rotating states:
//   - KDA's appends, per-slot steps and standalone folds take whole rows:
//     KDA's per-key log-decays make each logged entry's key side (a_j and
//     ell_j) 768 bytes, and the two 64-column tiles of a slot-head run on
//     different XCDs, so each would fetch it; whole rows read it once (1%
//     faster at B=64, 2.2% at B=256);
//   - merges (every operator) take 64-column tiles with 512 threads: 0.1-0.4%
//     faster than whole rows at B=64, 1.1-1.5% at B=256 (GDN, KDA);
//   - GDN's appends (a 260-byte key side) take 64-column tiles with 256
//     threads; 512 threads are 0.1-0.3 us slower;
//   - the eager step takes 64-column tiles, with 512 threads at d_k = 128 up
//     to a batch size chosen at launch (THREADS), 256 beyond.
// THREADS, when set, asks for that many threads per tile.
template <int OP, int MODE, int DK, int DV, int THREADS = 0> struct TileCfg {
    static constexpr bool MERGES = MODE == MERGE || MODE == FMERGE;
    static constexpr bool WIDE = DV == 128 && OP == KDA && MODE != EAGER && !MERGES;
    static constexpr int TMAX = WIDE ? 128 : DL_TILE_MAX;
    static constexpr int THR = THREADS ? THREADS : (WIDE || (MERGES && DV >= 64)) ? 512 : DL_THREADS_MAX;
    static constexpr int T = DV < TMAX ? DV : TMAX;                  // tile columns
    static constexpr int NT = DK * T / 4 < THR ? DK * T / 4 : THR;  // threads
    static constexpr int LPR = T / 4;     // lanes per row
    static constexpr int RPP = NT / LPR;  // rows per pass of the workgroup
    static constexpr int P = DK / RPP;    // rows per lane
    static constexpr int NTILE = DV / T;
    static constexpr int NW = NT / 64;
    static_assert(P * RPP == DK && LPR <= 32 && NT % LPR == 0 && NT % 64 == 0, "tile shape");
};

__host__ __device__ constexpr bool mode_fused(int mode)
{
    return mode == FAPPEND || mode == FMERGE || mode == SSTEP;
}
__host__ __device__ constexpr bool mode_fold(int mode) { return mode == FOLD || mode == SFOLD; }
__host__ __device__ constexpr bool mode_logged(int mode)
{
    return mode == APPEND || mode == MERGE || mode_fused(mode);
}
// Rows of the staged value-side factors and of the fold table for a launch.
// (SSTEP is sized for a merge at the longest log, the host passing n = M-1.)
__host__ __device__ constexpr int bt_rows(int mode, int n)
{
    return mode_fold(mode) ? n : mode == EAGER ? 1 : n + 1;
}
__host__ __device__ constexpr int fold_rows(int mode, int n)
{
    return (mode == MERGE || mode == FMERGE || mode == SSTEP) ? n + 1
         : mode == EAGER ? 1 : mode_fold(mode) ? n : 0;
}
constexpr int kRowTables = 8;
// Floats per row table: d_k entries and a pad slot, rounded to 16 bytes.
__host__ __device__ constexpr int row_table_stride(int DK) { return DK + 4; }
// Modes that read the log's decays: every mode but the eager step.
__host__ __device__ constexpr bool mode_has_log(int mode) { return mode_logged(mode) || mode_fold(mode); }
// Rows of the per-key table [rows][DK]: the fold rows of the merging modes,
// and for a per-key decay (KDA, RWKV6) at least the n logged entries, whose
// log-decays are staged there and turned into suffix sums in place (a fold
// row m then overwrites suffix-sum row m).
__host__ __device__ constexpr int key_rows(int op, int mode, int n)
{
    return (op != GDN && mode_has_log(mode) && n > fold_rows(mode, n)) ? n : fold_rows(mode, n);
}
// Dynamic LDS floats of the step kernel: eight per-row tables [DK], Bt
// [bt_rows][T], the per-key table [key_rows][DK], coefficients [2n+1], GDN's
// n suffix sums, then a 16-byte aligned junk slot: lanes with nothing to
// publish store there, which keeps the publishing stores unconditional.
__host__ __device__ constexpr int dyn_floats(int op, int mode, int n, int DK, int T)
{
    return kRowTables * row_table_stride(DK) + bt_rows(mode, n) * T + key_rows(op, mode, n) * DK +
           (mode_logged(mode) ? 2 * n + 1 : 0) + (op == GDN && mode_has_log(mode) ? n : 0) + 3 + 4;
}

// ------------------------------------------------------------- ReplayPrep --
//
// One wave64 per slot-head, four slot-heads per workgroup.  Per slot-head:
// coefficients c^q_j, c^k_j (RWKV6: c^r_j) of the n logged entries, with the
// factor e^{Lam' - Lam_j} (RWKV6: e^{Lam_{n-1} - Lam_j}) formed as e^{S_j +
// ell_t} (RWKV6: e^{S_j}) from the suffix sum S_j of the logged log-decays
// after entry j, accumulated newest entry first; kappa = q.k (RWKV6:
// r.(u (.) k)); then the key-side append a_n = k, ell_n = ell_t.  coef row:
// [c^q_0..M-1, c^k_0..M-1, kappa].
template <int OP, typename TIn, int DK>
__global__ __launch_bounds__(256) void replay_prep_kernel(StepArgs a)
{
    constexpr int KPL = (DK + 63) / 64; // keys per lane
    constexpr int EB = 8;               // log entries whose loads are issued together
    const int lane = threadIdx.x & 63;
    // the wave's slot-head, uniform over the wave: read from the first lane so
    // that the compiler keeps it (and the buffer resources built from it) in
    // scalar registers; otherwise every buffer load becomes a loop over the
    // lanes' resources, each iteration waiting for its load
    const int sh = blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (sh >= a.BH)
        return; // whole wave leaves together
    const int n = a.n, M = a.M;
    float *L = a.Llog + (OP == GDN ? (long)sh * M : (long)sh * M * DK);
    // the n logged entries of this slot-head (loads past them read zero)
    const rsrc_t ar = make_rsrc(static_cast<const TIn *>(a.alog) + (long)sh * M * DK, n * DK * sizeof(TIn));
    const rsrc_t lr = make_rsrc(L, (OP == GDN ? n : n * DK) * 4);

    // batch b holds entries top - e, e < EB, top = n - 1 - b EB (newest first)
    float am[EB][KPL], lm[EB][KPL], gm[EB];
    auto load_batch = [&](int top) {
#pragma unroll
        for (int e = 0; e < EB; ++e) {
            const int m = top - e;
            gm[e] = OP == GDN ? buf_ldf(lr, m >= 0 ? (unsigned)m * 4u : kSkip) : 0.f;
#pragma unroll
            for (int c = 0; c < KPL; ++c) {
                const int i = lane + 64 * c;
                const unsigned ei = (m >= 0 && i < DK) ? (unsigned)(m * DK + i) : kSkipElem;
                am[e][c] = buf_ld_in<TIn>(ar, ei);
                lm[e][c] = OP != GDN ? buf_ld_in<float>(lr, ei) : 0.f;
            }
        }
    };
    load_batch(n - 1); // first batch of entry loads, ahead of everything else
    const rsrc_t qr = make_rsrc(static_cast<const TIn *>(a.q) + (long)sh * DK, DK * sizeof(TIn));
    const rsrc_t kr = make_rsrc(static_cast<const TIn *>(a.k) + (long)sh * DK, DK * sizeof(TIn));
    const rsrc_t ur = make_rsrc(a.u + (long)(sh % a.H) * DK, OP == RWKV6 ? DK * 4 : 0);
    float qv[KPL], kv[KPL], uv[KPL], ell[KPL], sfx[KPL];
#pragma unroll
    for (int c = 0; c < KPL; ++c) {
        const int i = lane + 64 * c;
        const unsigned ei = i < DK ? (unsigned)i : kSkipElem;
        qv[c] = buf_ld_in<TIn>(qr, ei);
        kv[c] = buf_ld_in<TIn>(kr, ei);
        uv[c] = OP == RWKV6 ? buf_ld_in<float>(ur, ei) : 0.f; // RWKV6's bonus u
        ell[c] = floor_log_decay(OP == GDN ? a.ld[sh] : (i < DK ? a.ld[(long)sh * DK + i] : 0.f));
        sfx[c] = 0.f; // running suffix sum of the logged per-key log-decays
    }
    float gsfx = 0.f; // GDN: the same for its scalar log-decays
    // Lane m keeps entry m's coefficients (M <= 32 lanes), stored once after
    // the walk.  A store inside the walk would sit in a lane-0 branch, and the
    // wait for the next entry's loads would then also wait for that store
    // (the memory counter counts both, and the branch hides how many are in
    // flight): one store round trip per entry.
    float cq_m = 0.f, ck_m = 0.f;

    float *coef = a.coef + (long)sh * a.cstride;
    for (int top = n - 1; top >= 0; top -= EB) {
        if (top < n - 1)
            load_batch(top);
#pragma unroll
        for (int e = 0; e < EB; ++e) {
            const int m = top - e;
            if (m < 0)
                break; // uniform over the wave
            // GDN: the entry's scalar factor e^{S_m + ell_t}, applied after the sum
            const float g = OP == GDN ? expf(gsfx + ell[0]) : 1.f;
            if (OP == GDN)
                gsfx += gm[e];
            float sq = 0.f, sk = 0.f;
#pragma unroll
            for (int c = 0; c < KPL; ++c) {
                if (lane + 64 * c >= DK)
                    continue;
                float f;
                if (OP == GDN)
                    f = am[e][c];
                else if (OP == KDA)
                    f = expf(sfx[c] + ell[c]) * am[e][c];
                else
                    f = expf(sfx[c]) * am[e][c];
                sq = fmaf(f, qv[c], sq);
                sk = fmaf(f, kv[c], sk);
                if (OP != GDN)
                    sfx[c] += lm[e][c];
            }
            sq = wave_sum_from<1>(sq);
            if (OP != RWKV6)
                sk = wave_sum_from<1>(sk);
            // every lane holds the sums; lane m keeps them
            cq_m = lane == m ? sq * g : cq_m;
            ck_m = lane == m ? sk * g : ck_m;
        }
    }

    float kap = 0.f;
#pragma unroll
    for (int c = 0; c < KPL; ++c) {
        const int i = lane + 64 * c;
        if (i < DK)
            kap += OP == RWKV6 ? qv[c] * uv[c] * kv[c] : qv[c] * kv[c];
    }
    kap = wave_sum_from<1>(kap);

    // Every store last, after every load has been used (a wait for a load
    // issued before a store would also wait for the store).  The key-side
    // append of entry n first: it is the last use of the step's log-decay.
    TIn *an = static_cast<TIn *>(a.alog) + ((long)sh * M + n) * DK;
#pragma unroll
    for (int c = 0; c < KPL; ++c) {
        const int i = lane + 64 * c;
        if (i < DK) {
            an[i] = to_in<TIn>(kv[c]);
            if (OP != GDN)
                L[(long)n * DK + i] = ell[c];
        }
    }
    if (OP == GDN && lane == 0)
        L[n] = ell[0];
    if (lane < n) {
        coef[lane] = cq_m;
        if (OP != RWKV6)
            coef[M + lane] = ck_m;
    }
    if (lane == 0)
        coef[2 * M] = kap;
}

// Waves per SIMD the compiler must leave room for: 8 (64 VGPRs) for the
// per-slot step with bf16 inputs, which fits them with no spill but left to
// itself takes a few more and drops to 7; the compiler's own choice elsewhere.
template <typename TIn> __host__ __device__ constexpr int min_waves(int mode)
{
    return (mode == SSTEP && sizeof(TIn) == 2) ? 8 : 1;
}

// -------------------------------------------------------------- step kernel --
//
// One body for every launch on the state, MODE selecting the parts:
//   APPEND, MERGE    AppendDecode of the two-stage path: replay coefficients
//                    and the key-side append come from ReplayPrep;
//   FAPPEND, FMERGE  the one-launch path: each workgroup also computes its
//                    slot-head's replay coefficients (wave w takes log entries
//                    w, w+NW, ...) and tile 0 performs the key-side append;
//   EAGER            the eager baseline: decay, delta rule or raw update,
//                    rank-1 fold of this step only;
//   FOLD             standalone merge of the n pending entries;
//   SSTEP, SFOLD     the one-launch step and the standalone merge for a handle
//                    whose slots keep separate logs (continuous batching):
//                    each workgroup derives its slot's log length from the
//                    slot's phase, and an SSTEP workgroup merges exactly when
//                    its slot's log is full, so one launch mixes append and
//                    merge workgroups.
// Merging launches end with the fold and the single dense write.
template <int OP, typename TIn, int DK, int DV, int MODE, int THREADS = 0>
__global__ __launch_bounds__((TileCfg<OP, MODE, DK, DV, THREADS>::NT))
__attribute__((amdgpu_waves_per_eu(min_waves<TIn>(MODE)))) void step_kernel(StepArgs a)
{
    using C = TileCfg<OP, MODE, DK, DV, THREADS>;
    constexpr int T = C::T, NT = C::NT, LPR = C::LPR, RPP = C::RPP, P = C::P;
    constexpr int NTILE = C::NTILE, NW = C::NW;
    constexpr bool DELTA = OP != RWKV6;
    constexpr bool FUSED = mode_fused(MODE);
    constexpr bool STAGED = MODE == APPEND || MODE == MERGE;
    constexpr bool LOGGED = FUSED || STAGED;               // a step of the DeltaLog schedule
    constexpr bool FOLDS = mode_fold(MODE);                // standalone merge
    constexpr bool SLOTS = MODE == SSTEP || MODE == SFOLD; // per-slot logs
    constexpr bool READS = !FOLDS;                         // computes o_t and b_t
    constexpr bool MAY_WRITE = !(MODE == APPEND || MODE == FAPPEND);
    constexpr bool KAPPA_HERE = FUSED || MODE == EAGER;    // q.k summed in this kernel
    constexpr int ES = sizeof(TIn);
    constexpr int BS = DELTA ? 4 : ES;                     // b-log element size
    constexpr int NV = 9;                                  // 4 yq, 4 yk, kappa
    constexpr int RW = (DK + NT - 1) / NT;                 // row-table rows per lane
    // log-shard float4 per lane: staged ahead of the tile's rows for the first
    // NT/(T/4) entries (16 with 64-column tiles); longer logs take a second pass
    constexpr int SB = ((DL_MAX_M - 1) * (T / 4) + NT - 1) / NT;
    constexpr int KPL = (DK + 63) / 64;                    // keys per lane, coefficient pass
    constexpr int EW = (8 + NW - 1) / NW;                  // entries per wave, coefficient pass

    extern __shared__ float4 dyn4[];
    float *dyn = reinterpret_cast<float *>(dyn4);
    __shared__ float red[NW][LPR][NV];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6); // uniform: scalar registers
    const int c4 = tid % LPR, r0 = tid / LPR;
    // Natural block order: consecutive workgroups (dispatched round-robin over
    // the 8 XCDs) read adjacent tiles, which streams HBM faster than giving
    // each XCD a contiguous slab of the state (measured).
    const int sh = (SLOTS && a.slot >= 0 ? a.slot * a.H : 0) + blockIdx.x / NTILE;
    const int tile = blockIdx.x % NTILE;
    const int col = tile * T + 4 * c4;
    const int M = a.M;
    // log length: shared by all slots, or this slot's own (wave-uniform); a
    // released slot (phase < 0) holds no request, so its workgroups leave
    // before any load
    const int phase = SLOTS ? a.t0[sh / a.H] : 0;
    if (SLOTS && phase < 0)
        return;
    const int n = SLOTS ? (a.tm - phase + M) % M : a.n;
    if (MODE == SFOLD && n == 0)
        return; // nothing pending for this slot (whole workgroup leaves)
    const bool merging = MODE == MERGE || MODE == FMERGE || (MODE == SSTEP && n == M - 1);
    const bool writes = merging || MODE == EAGER || FOLDS;

    float *S = a.base + (long)sh * DK * DV;
    float *L = a.Llog + (OP == GDN ? (long)sh * M : (long)sh * M * DK);

    const int nb = bt_rows(MODE, n);
    const int nf = merging ? n + 1 : MODE == EAGER ? 1 : FOLDS ? n : 0;
    // The log holds each entry's own step log-decay ell_j (floored); the
    // cumulative Lam_j is their running sum.  Every factor a step needs is
    // e^(a sum of consecutive ell's): with Lam_{n-1} = T = sum_j ell_j and
    // S_m = sum_{j>m} ell_j, the base weights are e^(T + offset) and entry m's
    // factors e^(S_m + offset), offset = ell_t or 0.  Summing the ell's
    // directly (all <= 0) keeps these exact to a few ulps even after full
    // forgetting: a wiped step (-112) makes every sum across it <= -112,
    // whose exponential is 0, and no difference of two large cumulative
    // values is ever formed.
    constexpr bool KEYLOG = OP != GDN && mode_has_log(MODE); // per-key decays of logged entries
    const bool scan = KEYLOG && n > 0;                       // uniform over the workgroup
    const int kr = KEYLOG && n > nf ? n : nf;                // rows of the per-key table
    // Per-row tables, each TS = d_k + 4 floats: entry d_k is a pad slot that
    // lanes past d_k write to, so one row index addresses every table.
    constexpr int TS = row_table_stride(DK);
    float *Wq = dyn;             // read weights, q side
    float *Wk = dyn + TS;        // read weights, k side
    float *Rf = dyn + 2 * TS;    // fold base factor e^{Lam_f}
    float *Lf = dyn + 3 * TS;    // fold offset: Lam_f - Lam_{n-1}
    float *Qk = dyn + 4 * TS;    // q.k (RWKV6: r.(u (.) k)) terms
    float *Qr = dyn + 5 * TS;    // raw q (FUSED coefficient pass)
    float *Kr = dyn + 6 * TS;    // raw k (FUSED)
    float *Lx = dyn + 7 * TS;    // read offset: Lam' - Lam_{n-1} (delta) / 0 (RWKV6) (FUSED)
    float *Bt = dyn + kRowTables * TS;         // [nb][T] value-side factors of this tile
    float *F = Bt + nb * T;                    // [kr][DK] per-key table: logged decays, turned
                                               // into suffix sums in place, then fold rows
    float *cf = F + kr * DK;                   // [2n+1] (c^q_m, c^k_m) pairs, kappa (LOGGED)
    float *gsum = cf + (LOGGED ? 2 * n + 1 : 0); // GDN: [n] suffix sums S_m
    float *junk = dyn + ((kRowTables * TS + nb * T + kr * DK + (LOGGED ? 2 * n + 1 : 0) +
                          (OP == GDN && mode_has_log(MODE) ? n : 0) + 3) & ~3);

    // ------------------------------------------------------ 0. small loads --
    // Row metadata for rows i = tid + j*NT (lanes past d_k skip).
    const rsrc_t q_r = make_rsrc(static_cast<const TIn *>(a.q) + (long)sh * DK, READS ? DK * ES : 0);
    const rsrc_t k_r = make_rsrc(static_cast<const TIn *>(a.k) + (long)sh * DK, READS ? DK * ES : 0);
    // the log-decay log: entry j's ell_j at [j] (GDN) or [j][DK]; entry n holds
    // this step's, appended by ReplayPrep on the two-stage path
    const rsrc_t L_r = make_rsrc(L, MODE == EAGER ? 0 : (OP == GDN ? M : M * DK) * 4);
    const rsrc_t ld_r = make_rsrc(a.ld + (OP == GDN ? sh : (long)sh * DK),
                                  (MODE == EAGER || FUSED) ? (OP == GDN ? 1 : DK) * 4 : 0);
    const rsrc_t u_r = make_rsrc(a.u + (long)(sh % a.H) * DK, (OP == RWKV6 && KAPPA_HERE) ? DK * 4 : 0);
    // Loads are skipped outright (wave-uniform branches) where a whole wave
    // needs none of them, and pointed past the resource end where only some
    // of its lanes do.
    unsigned rq_[RW], rk_[RW], rell[RW], ru[RW]; // raw words
#pragma unroll
    for (int j = 0; j < RW; ++j) {
        const int i = tid + j * NT;
        const unsigned ei = i < DK ? (unsigned)i : kSkipElem;
        // skipped loads leave an unused, non-constant placeholder (a constant
        // would let the compiler fold the later conversion into the branch)
        rq_[j] = rk_[j] = rell[j] = ru[j] = (unsigned)tid;
        if (wave * 64 + j * NT < DK) { // this wave holds rows of the tables
            if (READS) {
                rq_[j] = buf_raw1<TIn>(q_r, ei);
                rk_[j] = buf_raw1<TIn>(k_r, ei);
            }
            // this step's per-key log-decay: the input, or entry n of the log
            if (OP != GDN) {
                if (STAGED)
                    rell[j] = buf_raw1<float>(L_r, i < DK ? (unsigned)(n * DK + i) : kSkipElem);
                else if (MODE == EAGER || FUSED)
                    rell[j] = buf_raw1<float>(ld_r, ei);
            }
            if (OP == RWKV6 && KAPPA_HERE)
                ru[j] = buf_raw1<float>(u_r, ei);
        }
    }
    // GDN: this step's scalar log-decay (wave-uniform) and the n logged ones,
    // lane j holding ell_j
    float gell = 0.f;
    unsigned glog = (unsigned)tid; // placeholder
    if (OP == GDN) {
        gell = (MODE == EAGER || FUSED) ? floor_log_decay(a.ld[sh]) : STAGED ? L[n] : 0.f;
        if (MODE != EAGER && n > 0)
            glog = __builtin_amdgcn_raw_buffer_load_b32(L_r, lane < n ? (unsigned)lane * 4u : kSkip, 0, 0);
    }
    // KDA, RWKV6: the n logged per-key log-decays [n][DK], one float4 per
    // thread ahead of the tile's rows (the first NT*4/DK entries; longer logs
    // take a second pass)
    const int nlg4 = KEYLOG ? n * (DK / 4) : 0;
    auto lg_load = [&](int s) {
        const int idx = tid + s * NT;
        return buf_raw4<float>(L_r, idx < nlg4 ? (unsigned)(4 * idx) : kSkipElem);
    };
    u32x4 lst = u32x4{(unsigned)tid, 0u, 0u, 0u}; // placeholder, stored to the junk slot
    if (KEYLOG && wave * 64 < nlg4)
        lst = lg_load(0);
    // This tile's shard of the n logged value-side factors.
    const rsrc_t b_r = make_rsrc(static_cast<const char *>(a.blog) + (long)sh * M * DV * BS,
                                 MODE == EAGER ? 0 : n * DV * BS);
    auto shard_load = [&](int s) { // slot idx = tid + s NT: entry m, float4 j4
        const int idx = tid + s * NT;
        const int m = idx / (T / 4), j4 = idx % (T / 4);
        const unsigned e = idx < n * (T / 4) ? (unsigned)(m * DV + tile * T + 4 * j4) : kSkipElem;
        return DELTA ? buf_raw4<float>(b_r, e) : buf_raw4<TIn>(b_r, e);
    };
    u32x4 bst = u32x4{(unsigned)tid, 0u, 0u, 0u}; // placeholder, stored to the junk slot
    if (MODE != EAGER && wave * 64 < n * (T / 4)) // the wave holds live slots
        bst = shard_load(0);
    // ReplayPrep's coefficients (two-stage path)
    unsigned cst = (unsigned)tid; // placeholder for lanes past 2n+1
    if (STAGED && wave * 64 < 2 * n + 1) {
        const rsrc_t c_r = make_rsrc(a.coef + (long)sh * a.cstride, a.cstride * 4);
        const int ci = tid < n ? tid : tid < 2 * n ? M + tid - n : 2 * M;
        cst = __builtin_amdgcn_raw_buffer_load_b32(c_r, tid < 2 * n + 1 ? (unsigned)ci * 4u : kSkip, 0, 0);
    }
    // key-side factors a_m for this wave's share of the replay coefficients (FUSED)
    unsigned ea[EW][KPL]; // raw words
    const rsrc_t a_r = make_rsrc(static_cast<const TIn *>(a.alog) + (long)sh * M * DK, FUSED ? n * DK * ES : 0);
#pragma unroll
    for (int e = 0; e < EW; ++e) {
        const int m = wave + NW * e;
#pragma unroll
        for (int c = 0; c < KPL; ++c)
            ea[e][c] = (unsigned)tid; // placeholders: entries m >= n are never used
        if (FUSED && m < n) { // wave-uniform
#pragma unroll
            for (int c = 0; c < KPL; ++c) {
                const int i = lane + 64 * c;
                ea[e][c] = buf_raw1<TIn>(a_r, i < DK ? (unsigned)(m * DK + i) : kSkipElem);
            }
        }
    }
    // v and beta for the lanes that finalise (lanes < LPR, all in wave 0)
    const rsrc_t v_r = make_rsrc(static_cast<const TIn *>(a.v) + (long)sh * DV, READS ? DV * ES : 0);
    u32x4 vraw = u32x4{(unsigned)tid, 0u, 0u, 0u}; // placeholder outside wave 0
    if (READS && wave == 0)
        vraw = buf_raw4<TIn>(v_r, tid < LPR ? (unsigned)col : kSkipElem);
    const float bet = (READS && DELTA) ? a.beta[sh] : 0.f;

    // ------------------------------------------------ 1. the tile's base rows --
    const rsrc_t tile_r = make_rsrc(S, DK * DV * 4);
    const unsigned xoff = (unsigned)(r0 * DV + col) * 4u; // this lane's byte offset in a pass
    float4 x[P];
#pragma unroll
    for (int p = 0; p < P; ++p)
        x[p] = buf_ld4_stream(tile_r, xoff, p * RPP * DV * 4);

    // ---------------------------------------- 2. publish the small data in LDS --
    float mq[RW], mk[RW], mell[RW], mu[RW];
#pragma unroll
    for (int j = 0; j < RW; ++j) {
        mq[j] = cvt1<TIn>(rq_[j], tid + j * NT);
        mk[j] = cvt1<TIn>(rk_[j], tid + j * NT);
        // this step's log-decay (a standalone fold adds none)
        mell[j] = (OP != GDN && !FOLDS) ? floor_log_decay(__uint_as_float(rell[j])) : 0.f;
        mu[j] = __uint_as_float(ru[j]);
    }
    // GDN: T = Lam_{n-1} and, in lane m of wave 0, S_m for the coefficient
    // pass and the fold table (ascending order; all terms are <= 0)
    float gT = 0.f;
    if (OP == GDN && MODE != EAGER) {
        const float gl = __uint_as_float(glog);
        float gS = 0.f;
#pragma unroll 1
        for (int j = 0; j < n; ++j) { // uniform
            const float v = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gl), j));
            gT += v;
            gS += j > lane ? v : 0.f;
        }
        if (wave == 0 && lane < n)
            gsum[lane] = gS;
    }
    // GDN: Lam' (a standalone fold: Lam_{n-1}) and e^{Lam'}, which scales the
    // read weights (so the column sums need no scaling afterwards) and the
    // fold's base factor
    const float gnew = gT + gell;
    const float egnew = OP == GDN ? expf(gnew) : 1.f;
    // Per-row tables that depend on T = Lam_{n-1,i}: read weights, fold base
    // factor and offsets.  T is 0 for an empty log; GDN's tables take its
    // scalar e^{Lam'} (egnew) instead of a per-key T.
    auto row_tables = [&](int j, float Tr) {
        const int i = tid + j * NT;
        const float rd = DELTA ? mell[j] : 0.f; // the delta rule reads the decayed state
        float wq, wk = 0.f;
        if (OP == GDN) { // the read's scalar e^{Lam'}, one factor per slot-head
            wq = egnew * mq[j];
            wk = egnew * mk[j];
        } else if (OP == KDA) {
            const float e = expf(Tr + rd);
            wq = e * mq[j];
            wk = e * mk[j];
        } else {
            wq = expf(Tr) * mq[j];
        }
        float *row = dyn + (i < DK ? i : DK); // this lane's entry of every table (or the pad)
        row[0 * TS] = wq;
        if (DELTA)
            row[1 * TS] = wk;
        if (OP != GDN && MAY_WRITE) {
            row[2 * TS] = expf(Tr + mell[j]); // merges fold to Lam'; a standalone fold to Lam_{n-1}
            row[3 * TS] = mell[j];
        }
        if (FUSED)
            row[7 * TS] = rd;
    };
#pragma unroll
    for (int j = 0; j < RW; ++j) {
        const int i = tid + j * NT;
        const bool ok = i < DK;
        float *row = dyn + (ok ? i : DK);
        if (KAPPA_HERE)
            row[4 * TS] = DELTA ? mq[j] * mk[j] : mq[j] * mu[j] * mk[j];
        if (FUSED) {
            row[5 * TS] = mq[j];
            row[6 * TS] = mk[j];
            if (merging)
                (ok ? F + n * DK + i : junk)[0] = mk[j]; // this step's entry folds with k
        }
        if (MODE == EAGER)
            (ok ? F + i : junk)[0] = mk[j]; // the only entry folds with k
        if (!scan)
            row_tables(j, 0.f);
    }
    if (KEYLOG) { // the logged per-key decays into the per-key table
        auto lg_store = [&](int s, u32x4 raw) {
            const int idx = tid + s * NT;
            *reinterpret_cast<float4 *>(idx < nlg4 ? F + 4 * idx : junk) = cvt4<float>(raw);
        };
        lg_store(0, lst);
#pragma unroll 1
        for (int s = 1; s * NT < nlg4; ++s) // long logs (behind the tile's rows)
            lg_store(s, lg_load(s));
    }
    if (MODE != EAGER) {
        auto shard_store = [&](int s, u32x4 raw) {
            const int idx = tid + s * NT;
            const int m = idx / (T / 4), j4 = idx % (T / 4);
            float *dst = idx < n * (T / 4) ? Bt + m * T + 4 * j4 : junk;
            *reinterpret_cast<float4 *>(dst) = DELTA ? cvt4<float>(raw) : cvt4<TIn>(raw);
        };
        shard_store(0, bst);
        // a log longer than one staging pass: the rest now (these loads queue
        // behind the tile's rows, so only such long logs wait for them here)
#pragma unroll 1
        for (int s = 1; s < SB && s * NT < n * (T / 4); ++s)
            shard_store(s, shard_load(s));
    }
    if (STAGED)
        (tid < 2 * n + 1 ? cf + (tid < n ? 2 * tid : tid < 2 * n ? 2 * (tid - n) + 1 : 2 * n) : junk)[0] =
            __uint_as_float(cst);
    __syncthreads();

    // ---- 2b. KDA, RWKV6: suffix sums of the logged decays, key by key in
    //      place (latest entry first, eight entries per LDS round trip); their
    //      total T = Lam_{n-1} completes the per-row tables
    if (scan) { // uniform over the workgroup
#pragma unroll
        for (int j = 0; j < RW; ++j) {
            const int i = tid + j * NT;
            if (i < DK) {
                float acc = 0.f;
#pragma unroll 1
                for (int m0 = n; m0 > 0; m0 -= 8) {
                    float l[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        l[e] = m0 - 1 - e >= 0 ? F[(m0 - 1 - e) * DK + i] : 0.f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        if (m0 - 1 - e >= 0) {
                            F[(m0 - 1 - e) * DK + i] = acc;
                            acc += l[e];
                        }
                    }
                }
                row_tables(j, acc);
            }
        }
        __syncthreads();
    }

    // ------------- 3. FUSED: this wave's replay coefficients (and fold rows)
    if (FUSED) {
        // one log entry m from its raw words: c^q_m, c^k_m and (merging) the
        // entry's fold row
        auto coef_entry = [&](int m, const unsigned *am_raw) {
            // GDN: the entry's scalar factor e^{Lam' - Lam_m} = e^{S_m + ell_t}
            const float g = OP == GDN ? expf(gsum[m] + gell) : 1.f;
            float sq = 0.f, sk = 0.f;
#pragma unroll
            for (int c = 0; c < KPL; ++c) {
                const int i = lane + 64 * c;
                if (i >= DK)
                    continue;
                const float am = cvt1<TIn>(am_raw[c], i);
                // e^{Lam_x,i - Lam_m,i} a_m,i = e^{S_m,i + read offset} a_m,i
                // (GDN: scalar factor applied after the sum)
                const float sm = OP == GDN ? 0.f : F[m * DK + i];
                const float f = OP == GDN ? am : expf(sm + Lx[i]) * am;
                sq = fmaf(f, Qr[i], sq);
                if (DELTA)
                    sk = fmaf(f, Kr[i], sk);
                if (merging) // fold row e^{Lam' - Lam_m} a_m, over suffix-sum row m
                    F[m * DK + i] = OP == GDN ? g * am : OP == KDA ? f : expf(sm + Lf[i]) * am;
            }
            sq = wave_sum_from<1>(sq);
            if (DELTA)
                sk = wave_sum_from<1>(sk);
            if (lane == 0) {
                cf[2 * m] = g * sq;
                cf[2 * m + 1] = g * sk;
            }
        };
        // entries wave, wave + NW, ... below NW*EW: loaded ahead of the tile
#pragma unroll
        for (int e = 0; e < EW; ++e) {
            const int m = wave + NW * e;
            if (m >= n)
                break; // uniform over the wave
            coef_entry(m, ea[e]);
        }
        // a longer log: one entry per wave at a time, loaded here (behind the
        // tile's rows, so only such long logs wait for them)
#pragma unroll 1
        for (int m = NW * EW + wave; m < n; m += NW) {
            unsigned am_raw[KPL];
#pragma unroll
            for (int c = 0; c < KPL; ++c) {
                const int i = lane + 64 * c;
                am_raw[c] = buf_raw1<TIn>(a_r, i < DK ? (unsigned)(m * DK + i) : kSkipElem);
            }
            coef_entry(m, am_raw);
        }
    }

    // -------- 4. column sums over this lane's rows, reduced across lanes/waves
    if (READS) {
        float yq[4] = {0.f, 0.f, 0.f, 0.f}, yk[4] = {0.f, 0.f, 0.f, 0.f}, kap = 0.f;
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const int r = r0 + p * RPP;
            const float wq = Wq[r];
            const float wk = DELTA ? Wk[r] : 0.f;
            if (KAPPA_HERE) // every lane sums its rows; only lane 0's class is used
                kap += Qk[r];
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
            if ((!DELTA && c >= 4 && c < 8) || (!KAPPA_HERE && c == 8))
                continue; // identically zero
            vals[c] = wave_sum_from<LPR>(vals[c]);
        }
        if (lane < LPR) {
#pragma unroll
            for (int c = 0; c < NV; ++c)
                red[wave][lane][c] = vals[c];
        }
    }
    if (READS || FUSED)
        __syncthreads();

    // ------- 5. fold table for MERGE / FOLD (FMERGE, EAGER built theirs above):
    //    F[m][i] = e^{Lam_f,i - Lam_m,i} a_m,i = e^{S_m,i + fold offset} a_m,i,
    //    written over suffix-sum row m; in MERGE the entry n appended by
    //    ReplayPrep (a_n = k, at Lam_f itself) gives exactly k_i.
    if (MODE == MERGE || FOLDS) {
        const rsrc_t af_r = make_rsrc(static_cast<const TIn *>(a.alog) + (long)sh * M * DK, nf * DK * ES);
        const int total = nf * DK;
        for (int base = 0; base < total; base += 4 * NT) {
            float av[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int idx = base + u * NT + tid;
                av[u] = buf_ld_in<TIn>(af_r, idx < total ? (unsigned)idx : kSkipElem);
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int idx = base + u * NT + tid;
                if (idx < total) {
                    const int m = idx / DK;
                    const float ex = m >= n ? 1.f
                                   : expf(OP == GDN ? gsum[m] + gell : F[idx] + Lf[idx % DK]);
                    F[idx] = ex * av[u];
                }
            }
        }
    }

    // ------------------------ 6. finalise this tile's outputs (wave 0)
    // Lane c + LPR g of wave 0 (g < G) takes column group c's partial sums of
    // waves g, g+G, ... and the replay terms of log entries g, g+G, ...; a
    // register reduction over g combines them, then lanes < LPR finish.
    if (READS && wave == 0) {
        constexpr int G = 64 / LPR;
        const int grp = lane / LPR;
        float y[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        float kap = 0.f;
#pragma unroll 1
        for (int w = grp; w < NW; w += G) {
#pragma unroll
            for (int c = 0; c < 8; ++c)
                y[c] += red[w][c4][c];
            kap += red[w][0][8];
        }
        // the log's replay terms sum_m c_m b_m, added onto the base's column
        // sums (q side into y[0..3], k side into y[4..7]); an entry's two
        // coefficients sit side by side, so each entry costs one LDS round
        // trip (its coefficient pair and its value-side factors together)
        if (LOGGED) {
#pragma unroll 1
            for (int m = grp; m < n; m += G) {
                const float4 b = *reinterpret_cast<const float4 *>(Bt + m * T + 4 * c4);
                const float2 cqk = *reinterpret_cast<const float2 *>(cf + 2 * m);
                const float bs[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    y[c] = fmaf(cqk.x, bs[c], y[c]);
                    if (DELTA)
                        y[4 + c] = fmaf(cqk.y, bs[c], y[4 + c]);
                }
            }
        }
#pragma unroll
        for (int c = 0; c < 8; ++c)
            if (DELTA || c < 4)
                y[c] = wave_sum_from<LPR>(y[c]);
        if (KAPPA_HERE)
            kap = wave_sum_from<LPR>(kap);
        if (STAGED)
            kap = cf[2 * n];
        if (lane < LPR) {
            const float4 vv = cvt4<TIn>(vraw);
            const float vs[4] = {vv.x, vv.y, vv.z, vv.w};
            float bt[4], ov[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if (DELTA) {
                    bt[c] = bet * (vs[c] - y[4 + c]);
                    ov[c] = y[c] + kap * bt[c];
                } else {
                    bt[c] = vs[c];
                    ov[c] = y[c] + kap * vs[c];
                }
            }
            *reinterpret_cast<float4 *>(a.o + (long)sh * DV + col) = make_float4(ov[0], ov[1], ov[2], ov[3]);
            if (LOGGED && !merging) { // value-side append of entry n (a merge empties the log)
                const long off = ((long)sh * M + n) * DV + col;
                if (DELTA) {
                    *reinterpret_cast<float4 *>(static_cast<float *>(a.blog) + off) =
                        make_float4(bt[0], bt[1], bt[2], bt[3]);
                } else {
                    TIn *bl = static_cast<TIn *>(a.blog) + off;
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        bl[c] = to_in<TIn>(vs[c]);
                }
            }
            if (writes)
                *reinterpret_cast<float4 *>(Bt + (nb - 1) * T + 4 * c4) = make_float4(bt[0], bt[1], bt[2], bt[3]);
        }
    }

    // Key-side append of entry n (a_n = k and this step's floored log-decay
    // ell_n, whose running sum is the pages' snapshot Lam_n), by tile 0, issued
    // last: stores count against the same wait counter as loads, so a store
    // issued earlier would hold up the wait for the tile's rows.
    if (FUSED && !merging && tile == 0) {
#pragma unroll
        for (int j = 0; j < RW; ++j) {
            const int i = tid + j * NT;
            if (i < DK) {
                // a_n = k as whole 32-bit words: for bf16 the even lane stores
                // the raw word holding k[i] and k[i+1]
                if (sizeof(TIn) == 4 || (i & 1) == 0)
                    *reinterpret_cast<unsigned *>(static_cast<TIn *>(a.alog) + ((long)sh * M + n) * DK + i) = rk_[j];
                if (OP != GDN)
                    L[(long)n * DK + i] = mell[j];
            }
        }
        if (OP == GDN && tid == 0)
            L[n] = gell;
    }

    // --------------------------------------- 7. fold and write the tile once
    if (writes) { // uniform over the workgroup
        __syncthreads();
        const float gs = egnew;
#pragma unroll
        for (int p = 0; p < P; ++p) {
            const float bf = OP == GDN ? gs : Rf[r0 + p * RPP];
            x[p] = make_float4(bf * x[p].x, bf * x[p].y, bf * x[p].z, bf * x[p].w);
        }
        // The rank-nf update in place on the tile, one entry at a time: the
        // entry's value-side factors for this lane's columns are read once and
        // applied to all P rows (a limited unroll keeps the entries' factors
        // from piling up in registers).
#pragma unroll 2
        for (int m = 0; m < nf; ++m) {
            const float4 b = *reinterpret_cast<const float4 *>(Bt + m * T + 4 * c4);
            const float *Fm = F + m * DK + r0;
#pragma unroll
            for (int p = 0; p < P; ++p) {
                const float f = Fm[p * RPP];
                x[p].x = fmaf(f, b.x, x[p].x);
                x[p].y = fmaf(f, b.y, x[p].y);
                x[p].z = fmaf(f, b.z, x[p].z);
                x[p].w = fmaf(f, b.w, x[p].w);
            }
        }
#pragma unroll
        for (int p = 0; p < P; ++p) {
            if (MODE == EAGER)
                buf_st4_stream(tile_r, xoff, p * RPP * DV * 4, x[p]);
            else
                buf_st4(tile_r, xoff, p * RPP * DV * 4, x[p]);
        }
    }
}

// ---------------------------------------------------------------- launchers --

// Largest batch (slot-heads) for which the eager step takes its 512-thread
// tiling (see launch_step_mode).
constexpr int kEagerWideMaxBH = 4096;

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

template <int OP, typename TIn, int DK, int DV, int MODE, int THREADS = 0>
hipError_t launch_step_t(const StepArgs &a, hipStream_t st)
{
    using C = TileCfg<OP, MODE, DK, DV, THREADS>;
    // per-slot launches size LDS for the longest log and may cover one slot
    const int slot_heads = (MODE == SFOLD && a.slot >= 0) ? a.H : a.BH;
    const int n_lds = (MODE == SSTEP || MODE == SFOLD) ? a.M - 1 : a.n;
    const dim3 grid((unsigned)slot_heads * C::NTILE);
    const size_t lds = sizeof(float) * (size_t)dyn_floats(OP, MODE, n_lds, DK, C::T);
    hipLaunchKernelGGL((step_kernel<OP, TIn, DK, DV, MODE, THREADS>), grid, dim3(C::NT), lds, st, a);
    return hipGetLastError();
}

template <int OP, typename TIn, int DK, int DV>
hipError_t launch_step_mode(int mode, const StepArgs &a, hipStream_t st)
{
    switch (mode) {
    case APPEND: return launch_step_t<OP, TIn, DK, DV, APPEND>(a, st);
    case MERGE: return launch_step_t<OP, TIn, DK, DV, MERGE>(a, st);
    case EAGER:
        // The eager step at d_k = 128 on 64-column tiles: 512 threads (4 rows
        // per lane) up to kEagerWideMaxBH slot-heads, 256 threads (8 rows per
        // lane) beyond.  Measured per eager step, 512 against 256 threads:
        // 2.0-2.4% faster at B=64 H=32 (GDN, KDA), 1.5% slower at B=256 H=32.
        if constexpr (DK >= 128 && DV >= 64)
            if (a.BH <= kEagerWideMaxBH)
                return launch_step_t<OP, TIn, DK, DV, EAGER, 512>(a, st);
        return launch_step_t<OP, TIn, DK, DV, EAGER>(a, st);
    case FOLD: return launch_step_t<OP, TIn, DK, DV, FOLD>(a, st);
    case FAPPEND: return launch_step_t<OP, TIn, DK, DV, FAPPEND>(a, st);
    case FMERGE: return launch_step_t<OP, TIn, DK, DV, FMERGE>(a, st);
    case SSTEP: return launch_step_t<OP, TIn, DK, DV, SSTEP>(a, st);
    case SFOLD: return launch_step_t<OP, TIn, DK, DV, SFOLD>(a, st);
    }
    return hipErrorInvalidValue;
}

template <int OP, typename TIn, int DK>
hipError_t launch_step_dv(int dv, int mode, const StepArgs &a, hipStream_t st)
{
    switch (dv) {
    case 16: return launch_step_mode<OP, TIn, DK, 16>(mode, a, st);
    case 32: return launch_step_mode<OP, TIn, DK, 32>(mode, a, st);
    case 64: return launch_step_mode<OP, TIn, DK, 64>(mode, a, st);
    case 128: return launch_step_mode<OP, TIn, DK, 128>(mode, a, st);
    }
    return hipErrorInvalidValue;
}

template <int OP, typename TIn>
hipError_t launch_step_dk(int dk, int dv, int mode, const StepArgs &a, hipStream_t st)
{
    switch (dk) {
    case 16: return launch_step_dv<OP, TIn, 16>(dv, mode, a, st);
    case 32: return launch_step_dv<OP, TIn, 32>(dv, mode, a, st);
    case 64: return launch_step_dv<OP, TIn, 64>(dv, mode, a, st);
    case 128: return launch_step_dv<OP, TIn, 128>(dv, mode, a, st);
    }
    return hipErrorInvalidValue;
}

template <int OP>
hipError_t launch_step(int dtype, int dk, int dv, int mode, const StepArgs &a, hipStream_t st)
{
    return dtype == BF16 ? launch_step_dk<OP, uint16_t>(dk, dv, mode, a, st)
                         : launch_step_dk<OP, float>(dk, dv, mode, a, st);
}

} // namespace dl
