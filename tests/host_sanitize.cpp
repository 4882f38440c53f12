// Host-only build of libdeltalog's C ABI (dl_api.hip, plain host code) for
// the sanitizer test: compiled with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer, with every kernel launcher replaced by a stub
// that records what would have been launched.  So the argument checks, the
// overlap arithmetic, the handle life cycle and the append/merge schedule
// (lockstep, two-stage and per-slot) all run on the CPU with no GPU, and
// each recorded launch is checked against the schedule the header documents.
// Exit status 0 when every check holds.
#include "dl_api.hip"

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

namespace dl {

struct Launch {
    int kind; // 0 ReplayPrep, 1 step kernel, 2 slot phase
    int op, mode, n, tm, slot, BH;
    const float *coef;
};
static std::vector<Launch> g_launches;
static float g_fake_scratch[4];

static hipError_t rec_prep(int op, const StepArgs &a)
{
    g_launches.push_back({0, op, -1, a.n, a.tm, a.slot, a.BH, a.coef});
    return hipSuccess;
}
static hipError_t rec_step(int op, int mode, const StepArgs &a)
{
    g_launches.push_back({1, op, mode, a.n, a.tm, a.slot, a.BH, a.coef});
    return hipSuccess;
}
hipError_t launch_prep_gdn(int, int, const StepArgs &a, hipStream_t) { return rec_prep(GDN, a); }
hipError_t launch_prep_kda(int, int, const StepArgs &a, hipStream_t) { return rec_prep(KDA, a); }
hipError_t launch_prep_rwkv6(int, int, const StepArgs &a, hipStream_t) { return rec_prep(RWKV6, a); }
hipError_t launch_step_gdn(int, int, int, int mode, const StepArgs &a, hipStream_t) { return rec_step(GDN, mode, a); }
hipError_t launch_step_kda(int, int, int, int mode, const StepArgs &a, hipStream_t) { return rec_step(KDA, mode, a); }
hipError_t launch_step_rwkv6(int, int, int, int mode, const StepArgs &a, hipStream_t) { return rec_step(RWKV6, mode, a); }
hipError_t launch_slot_phase(int *, int, int slot, int value, bool, hipStream_t)
{
    g_launches.push_back({2, -1, -1, value, -1, slot, 0, nullptr});
    return hipSuccess;
}
hipError_t scratch_on_current_device(float **out)
{
    *out = g_fake_scratch;
    return hipSuccess;
}

} // namespace dl

using dl::g_launches;
static int g_fail = 0;
#define CHECK(c)                                                              \
    do {                                                                      \
        if (!(c)) {                                                           \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++g_fail;                                                         \
        }                                                                     \
    } while (0)

// fake device addresses: aligned and never dereferenced on the host
static void *fake(uintptr_t i) { return reinterpret_cast<void *>(uintptr_t(0x7e0000000000) + (i << 32)); }
static float *BASE = static_cast<float *>(fake(1));
static void *WS = fake(2);
static const void *Q = fake(3), *K = fake(4), *V = fake(5);
static const float *BETA = static_cast<const float *>(fake(6)), *LD = static_cast<const float *>(fake(7));
static const float *U = static_cast<const float *>(fake(8));
static float *O = static_cast<float *>(fake(9));

static dl_state *make(int B, int H, int d, int M, dl_op op, dl_dtype dt = DL_BF16)
{
    dl_state *s = nullptr;
    CHECK(dl_state_create(B, H, d, d, M, op, dt, BASE, WS, op == DL_OP_RWKV6 ? U : nullptr, &s) == DL_OK);
    return s;
}

static void test_status_and_workspace()
{
    for (int st = 0; st <= 6; ++st)
        CHECK(std::strlen(dl_status_string(static_cast<dl_status>(st))) > 0);
    CHECK(std::strcmp(dl_status_string(static_cast<dl_status>(99)), "unknown status") == 0);
    CHECK(dl_workspace_bytes(64, 32, 128, 128, 8, DL_OP_KDA, DL_BF16) >
          dl_workspace_bytes(64, 32, 128, 128, 8, DL_OP_GDN, DL_BF16));
    CHECK(dl_workspace_bytes(0, 1, 16, 16, 4, DL_OP_GDN, DL_F32) == 0);
    CHECK(dl_workspace_bytes(1, 1, 16, 16, 33, DL_OP_GDN, DL_F32) == 0);
    CHECK(dl_workspace_bytes(1, 1, 24, 16, 4, DL_OP_GDN, DL_F32) == 0);
    CHECK(dl_workspace_bytes(1 << 16, 1 << 8, 128, 128, 4, DL_OP_GDN, DL_F32) == 0);
    CHECK(dl_workspace_bytes(1, 1, 16, 16, 4, static_cast<dl_op>(7), DL_F32) == 0);
    CHECK(dl_workspace_bytes(1, 1, 16, 16, 4, DL_OP_GDN, static_cast<dl_dtype>(3)) == 0);
}

static void test_create_validation()
{
    dl_state *s = reinterpret_cast<dl_state *>(1);
    CHECK(dl_state_create(2, 3, 16, 16, 4, DL_OP_GDN, DL_F32, BASE, WS, nullptr, nullptr) == DL_E_INVALID);
    CHECK(dl_state_create(2, 3, 24, 16, 4, DL_OP_GDN, DL_F32, BASE, WS, nullptr, &s) == DL_E_SHAPE && !s);
    CHECK(dl_state_create(2, 3, 16, 16, 0, DL_OP_GDN, DL_F32, BASE, WS, nullptr, &s) == DL_E_INVALID);
    CHECK(dl_state_create(2, 3, 16, 16, 4, DL_OP_RWKV6, DL_F32, BASE, WS, nullptr, &s) == DL_E_INVALID);
    CHECK(dl_state_create(2, 3, 16, 16, 4, DL_OP_GDN, DL_F32, BASE + 1, WS, nullptr, &s) == DL_E_ALIGN);
    CHECK(dl_state_create(2, 3, 16, 16, 4, DL_OP_GDN, DL_F32, BASE, static_cast<char *>(WS) + 16, nullptr, &s) ==
          DL_E_ALIGN);
    // base and workspace overlapping: the workspace starts inside the base
    CHECK(dl_state_create(2, 3, 16, 16, 4, DL_OP_GDN, DL_F32, BASE, BASE + 256, nullptr, &s) == DL_E_INVALID);
    // a large batch (the per-slot host mirror is B ints)
    dl_state *big = nullptr;
    CHECK(dl_state_create(1 << 20, 1, 16, 16, 4, DL_OP_GDN, DL_BF16, BASE, WS, nullptr, &big) == DL_OK);
    CHECK(dl_slot_log_len(big, (1 << 20) - 1) == 0 && dl_slot_log_len(big, 1 << 20) == -1);
    CHECK(dl_state_destroy(big) == DL_OK);
    CHECK(dl_state_destroy(nullptr) == DL_OK);
}

// The lockstep schedule: M-1 appends then a merge, one launch each
static void test_lockstep_schedule(dl_op op)
{
    const int M = 5;
    dl_state *s = make(2, 3, 32, M, op);
    g_launches.clear();
    for (int t = 0; t < 3 * M + 2; ++t) {
        const int n = t % M;
        CHECK(dl_log_len(s) == n);
        CHECK(dl_decode_step(s, Q, K, V, op == DL_OP_RWKV6 ? nullptr : BETA, LD, O, nullptr) == DL_OK);
        CHECK(g_launches.size() == size_t(t + 1));
        const dl::Launch &l = g_launches.back();
        CHECK(l.kind == 1 && l.op == op && l.n == n && l.BH == 6);
        CHECK(l.mode == (n + 1 == M ? dl::FMERGE : dl::FAPPEND));
    }
    CHECK(dl_log_len(s) == 2);
    g_launches.clear();
    CHECK(dl_merge(s, nullptr) == DL_OK && dl_log_len(s) == 0);
    CHECK(g_launches.size() == 1 && g_launches[0].mode == dl::FOLD && g_launches[0].n == 2);
    CHECK(dl_merge(s, nullptr) == DL_OK && g_launches.size() == 1); // empty log: no launch
    CHECK(dl_set_log_len(s, M) == DL_E_INVALID && dl_set_log_len(s, -1) == DL_E_INVALID);
    CHECK(dl_set_log_len(s, 3) == DL_OK && dl_log_len(s) == 3);
    CHECK(dl_state_reset(s) == DL_OK && dl_log_len(s) == 0);
    // missing beta for a delta-rule op, missing log-decay, misaligned output
    if (op != DL_OP_RWKV6)
        CHECK(dl_decode_step(s, Q, K, V, nullptr, LD, O, nullptr) == DL_E_INVALID);
    CHECK(dl_decode_step(s, Q, K, V, BETA, nullptr, O, nullptr) == DL_E_INVALID);
    CHECK(dl_decode_step(s, Q, K, V, BETA, LD, O + 1, nullptr) == DL_E_ALIGN);
    // the output inside the base, the workspace, or an input
    CHECK(dl_decode_step(s, Q, K, V, BETA, LD, BASE + 64, nullptr) == DL_E_INVALID);
    CHECK(dl_decode_step(s, Q, K, V, BETA, LD, static_cast<float *>(WS) + 64, nullptr) == DL_E_INVALID);
    CHECK(dl_decode_step(s, Q, K, V, BETA, LD, static_cast<float *>(const_cast<void *>(V)), nullptr) ==
          DL_E_INVALID);
    // inputs may alias each other
    CHECK(dl_decode_step(s, Q, Q, V, BETA, LD, O, nullptr) == DL_OK && dl_log_len(s) == 1);
    CHECK(dl_state_destroy(s) == DL_OK);
}

// The two-stage split and its call order; the no-alloc variant
static void test_two_stage(dl_op op)
{
    const int M = 3;
    const float *beta = op == DL_OP_RWKV6 ? nullptr : BETA;
    dl_state *s = make(4, 2, 64, M, op);
    g_launches.clear();
    CHECK(dl_append_decode(s, Q, K, V, beta, O, nullptr) == DL_E_STATE);
    for (int t = 0; t < 2 * M; ++t) {
        CHECK(dl_replay_prep(s, Q, K, LD, nullptr) == DL_OK);
        CHECK(dl_replay_prep(s, Q, K, LD, nullptr) == DL_E_STATE);
        CHECK(dl_decode_step(s, Q, K, V, beta, LD, O, nullptr) == DL_E_STATE);
        CHECK(dl_merge(s, nullptr) == DL_E_STATE);
        CHECK(dl_set_log_len(s, 0) == DL_E_STATE);
        CHECK(dl_decode_step_staged_noalloc(s, Q, K, V, beta, LD, O, nullptr) == DL_E_STATE);
        CHECK(dl_append_decode(s, Q, K, V, beta, O, nullptr) == DL_OK);
    }
    CHECK(g_launches.size() == size_t(4 * M));
    for (int t = 0; t < 2 * M; ++t) {
        const dl::Launch &lp = g_launches[2 * t], &la = g_launches[2 * t + 1];
        CHECK(lp.kind == 0 && lp.n == t % M);
        CHECK(la.kind == 1 && la.n == t % M && la.mode == ((t % M) + 1 == M ? dl::MERGE : dl::APPEND));
        CHECK(lp.coef == la.coef && lp.coef != dl::g_fake_scratch); // the workspace's rows
    }
    // no-alloc: the same two launches, coefficients in the static scratch
    g_launches.clear();
    for (int t = 0; t < M; ++t)
        CHECK(dl_decode_step_staged_noalloc(s, Q, K, V, beta, LD, O, nullptr) == DL_OK);
    CHECK(g_launches.size() == size_t(2 * M) && dl_log_len(s) == 0);
    for (int t = 0; t < M; ++t) {
        CHECK(g_launches[2 * t].kind == 0 && g_launches[2 * t].coef == dl::g_fake_scratch);
        CHECK(g_launches[2 * t + 1].mode == (t + 1 == M ? dl::MERGE : dl::APPEND));
        CHECK(g_launches[2 * t + 1].coef == dl::g_fake_scratch);
    }
    CHECK(dl_decode_step_staged_noalloc(s, Q, K, V, beta, nullptr, O, nullptr) == DL_E_INVALID);
    CHECK(dl_state_destroy(s) == DL_OK);
    // coefficient rows beyond the scratch: refused before any launch
    dl_state *big = nullptr;
    CHECK(dl_state_create(128, 128, 16, 16, 32, op, DL_BF16, BASE, WS, op == DL_OP_RWKV6 ? U : nullptr, &big) ==
          DL_OK);
    g_launches.clear();
    CHECK(dl_decode_step_staged_noalloc(big, Q, K, V, beta, LD, O, nullptr) == DL_E_SCRATCH);
    CHECK(g_launches.empty() && dl_log_len(big) == 0);
    CHECK(dl_state_destroy(big) == DL_OK);
}

// Per-slot logs: phases, admission, release, per-slot merge
static void test_per_slot(dl_op op)
{
    const int B = 5, M = 4;
    const float *beta = op == DL_OP_RWKV6 ? nullptr : BETA;
    dl_state *s = make(B, 2, 16, M, op);
    CHECK(dl_decode_step(s, Q, K, V, beta, LD, O, nullptr) == DL_OK); // n = 1
    CHECK(dl_state_enable_slots(s, nullptr) == DL_E_STATE);         // needs an empty log
    CHECK(dl_merge(s, nullptr) == DL_OK);
    CHECK(dl_slot_admit(s, 0, nullptr) == DL_E_STATE);              // not per-slot yet
    CHECK(dl_state_enable_slots(s, nullptr) == DL_OK);
    CHECK(dl_state_enable_slots(s, nullptr) == DL_E_STATE);
    CHECK(dl_log_len(s) == -1);
    CHECK(dl_replay_prep(s, Q, K, LD, nullptr) == DL_E_STATE);
    CHECK(dl_decode_step_staged_noalloc(s, Q, K, V, beta, LD, O, nullptr) == DL_E_STATE);
    CHECK(dl_set_log_len(s, 0) == DL_E_STATE && dl_state_reset(s) == DL_E_STATE);
    CHECK(dl_slot_admit(s, -1, nullptr) == DL_E_INVALID && dl_slot_admit(s, B, nullptr) == DL_E_INVALID);
    CHECK(dl_slot_log_len(s, B) == -1 && dl_slot_log_len(nullptr, 0) == -1);
    // slot b admitted at step b: its log length is (t - b) mod M
    g_launches.clear();
    int t = 0;
    for (; t < 2 * M + 1; ++t) {
        if (t < B)
            CHECK(dl_slot_admit(s, t, nullptr) == DL_OK);
        CHECK(dl_decode_step(s, Q, K, V, beta, LD, O, nullptr) == DL_OK);
        CHECK(g_launches.back().kind == 1 && g_launches.back().mode == dl::SSTEP);
        CHECK(g_launches.back().tm == t % M);
        for (int b = 0; b < B; ++b) {
            const int want = b <= t ? (t + 1 - b) % M : (t + 1) % M;
            CHECK(dl_slot_log_len(s, b) == want);
        }
    }
    CHECK(dl_slot_release(s, 2, nullptr) == DL_OK && dl_slot_log_len(s, 2) == 0);
    g_launches.clear();
    CHECK(dl_slot_merge(s, 2, nullptr) == DL_OK && g_launches.empty()); // released: nothing to fold
    const int n1 = dl_slot_log_len(s, 1);
    CHECK(dl_slot_merge(s, 1, nullptr) == DL_OK);
    CHECK(dl_slot_log_len(s, 1) == 0);
    if (n1 > 0)
        CHECK(g_launches.size() == 2 && g_launches[0].mode == dl::SFOLD && g_launches[0].slot == 1);
    CHECK(dl_merge(s, nullptr) == DL_OK);
    for (int b = 0; b < B; ++b)
        CHECK(dl_slot_log_len(s, b) == 0);
    CHECK(dl_slot_admit(s, 2, nullptr) == DL_OK && dl_slot_log_len(s, 2) == 0);
    CHECK(dl_decode_step(s, Q, K, V, beta, LD, O, nullptr) == DL_OK && dl_slot_log_len(s, 2) == 1);
    CHECK(dl_state_destroy(s) == DL_OK);
}

static void test_eager_and_suggest()
{
    g_launches.clear();
    CHECK(dl_eager_step(DL_OP_GDN, 2, 3, 32, 32, DL_BF16, BASE, Q, K, V, BETA, LD, nullptr, O, nullptr) == DL_OK);
    CHECK(g_launches.size() == 1 && g_launches[0].mode == dl::EAGER);
    CHECK(dl_eager_step(DL_OP_RWKV6, 2, 3, 32, 32, DL_BF16, BASE, Q, K, V, nullptr, LD, nullptr, O, nullptr) ==
          DL_E_INVALID); // u missing
    CHECK(dl_eager_step(DL_OP_GDN, 2, 3, 32, 32, DL_BF16, BASE, Q, K, V, BETA, LD, nullptr, BASE + 8, nullptr) ==
          DL_E_INVALID); // o inside S
    CHECK(dl_eager_step(DL_OP_GDN, 2, 3, 24, 32, DL_BF16, BASE, Q, K, V, BETA, LD, nullptr, O, nullptr) ==
          DL_E_SHAPE);
    for (int op = 0; op < 3; ++op) {
        const int m = dl_suggest_merge_interval(64, 32, 128, 128, static_cast<dl_op>(op), DL_BF16);
        CHECK(m >= 1 && m <= 32);
    }
    CHECK(dl_suggest_merge_interval(64, 32, 24, 128, DL_OP_GDN, DL_BF16) == 0);
    double app[32], mer[32];
    for (int n = 0; n < 32; ++n) {
        app[n] = 25.0 + 0.3 * n;
        mer[n] = 48.0 + 0.3 * n;
    }
    const int m = dl_choose_merge_interval(app, mer, 32);
    CHECK(m > 1 && m < 32);
    CHECK(dl_choose_merge_interval(app, mer, 1) == 1);
    CHECK(dl_choose_merge_interval(nullptr, mer, 32) == 0 && dl_choose_merge_interval(app, nullptr, 32) == 0);
    CHECK(dl_choose_merge_interval(app, mer, 0) == 0 && dl_choose_merge_interval(app, mer, 33) == 0);
    app[3] = -1.0;
    CHECK(dl_choose_merge_interval(app, mer, 32) == 0);
    app[3] = 25.9;
    mer[5] = std::nan("");
    CHECK(dl_choose_merge_interval(app, mer, 32) == 0);
}

int main()
{
    test_status_and_workspace();
    test_create_validation();
    for (int op = 0; op < 3; ++op) {
        test_lockstep_schedule(static_cast<dl_op>(op));
        test_two_stage(static_cast<dl_op>(op));
        test_per_slot(static_cast<dl_op>(op));
    }
    test_eager_and_suggest();
    // many handles created and destroyed (the leak checker sees every one)
    for (int i = 0; i < 1000; ++i)
        CHECK(dl_state_destroy(make(1 + i % 7, 1 + i % 3, 16, 1 + i % 32, static_cast<dl_op>(i % 3))) == DL_OK);
    if (g_fail) {
        std::fprintf(stderr, "%d checks failed\n", g_fail);
        return 1;
    }
    std::printf("host API checks passed\n");
    return 0;
}
