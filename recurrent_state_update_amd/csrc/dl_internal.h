// dl_internal.h -- declarations shared by the host API and the kernel files of
// libdeltalog.  Not installed; the public interface is include/deltalog.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace dl {

enum Op : int { GDN = 0, KDA = 1, RWKV6 = 2 };
enum DType : int { F32 = 0, BF16 = 1 };

// What one launch of the step kernel does with a tile of the state.
enum Mode : int {
    APPEND = 0,  // two-stage append phase: read S-bar, outputs + b_t, no state write
    MERGE = 1,   // two-stage merge phase: as APPEND, then fold all M entries, write S-bar
    EAGER = 2,   // eager baseline: decay, delta rule, rank-1 update, write state
    FOLD = 3,    // standalone merge: fold the n pending entries, write S-bar
    FAPPEND = 4, // one-launch append phase (replay coefficients computed in place)
    FMERGE = 5,  // one-launch merge phase
    SSTEP = 6,   // one-launch step with per-slot logs: each slot appends or merges
    SFOLD = 7    // standalone merge with per-slot logs (one slot or all)
};

// Byte offsets of the log and coefficient arrays inside the workspace.
// Each segment starts on a 256-byte boundary.
struct Layout {
    size_t a_off;   // a-log      [B*H, M, d_k]  input dtype (a_j = k_j)
    size_t b_off;   // b-log      [B*H, M, d_v]  fp32 (delta rule) / input dtype (RWKV6)
    size_t L_off;   // Lambda-log [B*H, M] (GDN) or [B*H, M, d_k] fp32
    size_t c_off;   // coef       [B*H, cstride] fp32: c^q_0..M-1, c^k_0..M-1, kappa
    size_t t_off;   // slot phase [B] int32 (per-slot schedule)
    size_t total;
    int cstride;
};

Layout workspace_layout(long B, long H, int dk, int dv, int M, int op, int dtype);

// Everything a launch needs, passed by value as the kernel argument.
struct StepArgs {
    int BH;          // slot-heads
    int H;           // heads (RWKV6's bonus u is per head)
    int M;           // merge interval
    int n;           // log entries before this step
    const void *q;   // [BH, dk] (r for RWKV6)
    const void *k;   // [BH, dk]
    const void *v;   // [BH, dv]
    const float *beta; // [BH]
    const float *ld;   // [BH] (GDN) or [BH, dk]: this step's log-decay (EAGER and prep)
    const float *u;    // [H, dk] (RWKV6)
    float *base;       // [BH, dk, dv]
    float *o;          // [BH, dv]
    void *alog;
    void *blog;
    float *Llog;
    float *coef;
    int cstride;
    // per-slot schedule: slot b's log length is (tm - t0[b]) mod M
    int tm;          // the handle's step counter mod M
    const int *t0;   // [B] step (mod M) at which each slot's log was last emptied
    int slot;        // SFOLD: the one slot to fold, or -1 for all
};

// Kernel launchers, one set per operator (dl_gdn.hip, dl_kda.hip, dl_rwkv6.hip).
// They return the launch status (hipGetLastError after the launch) or
// hipErrorInvalidValue for an unsupported shape.
hipError_t launch_prep_gdn(int dtype, int dk, const StepArgs &a, hipStream_t st);
hipError_t launch_prep_kda(int dtype, int dk, const StepArgs &a, hipStream_t st);
hipError_t launch_prep_rwkv6(int dtype, int dk, const StepArgs &a, hipStream_t st);
// Set slot phases: one slot (slot >= 0), or all slots (slot < 0; with
// active_only, only those not released).  A kernel, so calls stay capturable.
hipError_t launch_slot_phase(int *t0, int B, int slot, int value, bool active_only, hipStream_t st);
// The static device scratch of dl_decode_step_staged_noalloc (dl_device.hip):
// its size in floats, and its device address on the current device (looked
// up once per device).
constexpr size_t kScratchFloats = size_t(1) << 20; // 4 MiB
hipError_t scratch_on_current_device(float **out);
hipError_t launch_step_gdn(int dtype, int dk, int dv, int mode, const StepArgs &a, hipStream_t st);
hipError_t launch_step_kda(int dtype, int dk, int dv, int mode, const StepArgs &a, hipStream_t st);
hipError_t launch_step_rwkv6(int dtype, int dk, int dv, int mode, const StepArgs &a, hipStream_t st);

} // namespace dl
