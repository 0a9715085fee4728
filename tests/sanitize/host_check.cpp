// host_check.cpp -- the host side of libdeltalog (include/deltalog.h), built
// with the address and undefined-behaviour sanitizers against launchers that
// only record (stub_launch.cpp).  Device addresses are fake, aligned and never
// dereferenced.  Checks the argument validation, the aliasing rules, the
// lockstep and per-slot log-length bookkeeping and which kernel mode each
// call asks for (the signal-papers summary, Fig. 4: append while L < C, fold
// when L reaches C).  Test infrastructure; prints the number of checks and
// exits 0, or names the first failed check and exits 1.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "../../include/deltalog.h"
#include "stub_launch.h"

using dlk::g_launches;

static int g_checks = 0;

#define CHECK(cond)                                                                     \
    do {                                                                                \
        ++g_checks;                                                                     \
        if (!(cond)) {                                                                  \
            fprintf(stderr, "host_check: %s:%d: check failed: %s (last error: %s)\n",   \
                    __FILE__, __LINE__, #cond, dl_last_error());                        \
            exit(1);                                                                    \
        }                                                                               \
    } while (0)

static void *addr(uintptr_t a) { return reinterpret_cast<void *>(a); }

// Fake device layout: base, workspace, inputs and outputs 16 MB apart.
static const uintptr_t BASE = 0x7f0000000000ull, WS = BASE + (1ull << 30), IN = BASE + (2ull << 30),
                       DST = BASE + (3ull << 30), PREP = BASE + (4ull << 30);
static const uintptr_t MB16 = 1ull << 24;

static dl_step_args token(int op, int t) {
    const uintptr_t b = IN + (uintptr_t)t * 8 * MB16;
    dl_step_args a;
    a.q = addr(b);
    a.k = addr(b + MB16);
    a.v = addr(b + 2 * MB16);
    a.beta = op == DL_RWKV6 ? nullptr : static_cast<const float *>(addr(b + 3 * MB16));
    a.decay = static_cast<const float *>(addr(b + 4 * MB16));
    a.bonus = op == DL_RWKV6 ? static_cast<const float *>(addr(IN - MB16)) : nullptr;
    a.out = static_cast<float *>(addr(b + 5 * MB16));
    return a;
}

static void check_configs() {
    const int widths[3] = {32, 64, 128};
    for (int op = 0; op < 3; ++op)
        for (int dt = 0; dt < 2; ++dt)
            for (int dk : widths)
                for (int dv : widths)
                    for (int C : {1, 7, 8, 16, 32}) {
                        dl_config c = {op, dt, 3, 5, dk, dv, C};
                        const size_t ws = dl_workspace_bytes(&c);
                        size_t off[3];
                        CHECK(ws > 0);
                        CHECK(dl_workspace_layout(&c, off) == DL_OK);
                        CHECK(off[0] == 0 && off[1] > off[0] && off[2] > off[1] && off[2] < ws);
                        const size_t xs = op == DL_RWKV6 ? (dt ? 2 : 4) : 4;
                        CHECK(off[1] >= (size_t)15 * C * dv * xs);
                        CHECK(dl_prep_bytes(&c) == (size_t)15 * (2 * dk + 2 * (C <= 8 ? 8 : C <= 16 ? 16 : 32) + 4) * 4);
                        const double us = dl_predict_token_us(&c, 0, 0);
                        CHECK(us > 0 && us < 1e6);
                        const int best = dl_choose_capacity(&c, 32, 0, 0);
                        CHECK(best >= 1 && best <= 32);
                    }
    dl_config bad[] = {{3, 0, 1, 1, 64, 64, 4}, {0, 2, 1, 1, 64, 64, 4}, {0, 0, 0, 1, 64, 64, 4},
                       {0, 0, 1, 1, 64, 64, 0}, {0, 0, 1, 1, 64, 64, 33}, {0, 0, 1, 1, 48, 64, 4},
                       {0, 0, 1, 1, 64, 16, 4}, {0, 0, 1 << 30, 1 << 30, 32, 32, 4}};
    const int want[] = {DL_ERR_ARG, DL_ERR_ARG, DL_ERR_SHAPE, DL_ERR_SHAPE, DL_ERR_SHAPE,
                        DL_ERR_UNSUPPORTED, DL_ERR_UNSUPPORTED, DL_ERR_SHAPE};
    for (size_t i = 0; i < sizeof(bad) / sizeof(bad[0]); ++i) {
        dl_state *h = nullptr;
        CHECK(dl_workspace_bytes(&bad[i]) == 0);
        CHECK(dl_state_init(&h, &bad[i], static_cast<float *>(addr(BASE)), addr(WS), 1ull << 40) == want[i]);
        CHECK(h == nullptr);
    }
}

static void check_lockstep(int op, int dk, int dv) {
    const int C = 5;
    dl_config c = {op, DL_BF16, 2, 3, dk, dv, C};
    dl_state *h = nullptr;
    const size_t ws = dl_workspace_bytes(&c);
    CHECK(dl_state_init(&h, &c, static_cast<float *>(addr(BASE)), addr(WS), ws) == DL_OK);
    CHECK(dl_log_length(h) == 0);
    g_launches.clear();
    // three cycles of single steps: appends at L = 0..C-2, the fused fold at C-1
    for (int t = 0; t < 3 * C; ++t) {
        dl_step_args a = token(op, t % 4);
        const int L = t % C;
        CHECK(dl_decode_step(h, &a, nullptr) == DL_OK);
        CHECK(g_launches.size() == (size_t)t + 1);
        const dlk::Launch &l = g_launches.back();
        CHECK(l.kind == dlk::KIND_STEP && l.L == L && l.C == C && l.N == 6 && l.dk == dk && l.dv == dv);
        CHECK(l.op == op && l.cmax == 8 && !l.slots && !l.prep);
        CHECK(l.mode == (L + 1 == C ? dlk::MODE_MERGE : dlk::MODE_APPEND));
        CHECK(dl_log_length(h) == (t + 1) % C);
    }
    // an early merge folds L entries and empties the log; at L = 0 it is a no-op
    dl_step_args a0 = token(op, 0);
    CHECK(dl_decode_step(h, &a0, nullptr) == DL_OK && dl_decode_step(h, &a0, nullptr) == DL_OK);
    g_launches.clear();
    CHECK(dl_materialize(h, static_cast<float *>(addr(DST)), nullptr) == DL_OK);
    CHECK(g_launches.size() == 1 && g_launches[0].mode == dlk::MODE_FOLD && g_launches[0].L == 2);
    CHECK(dl_log_length(h) == 2);
    CHECK(dl_merge(h, nullptr) == DL_OK);
    CHECK(g_launches.size() == 2 && g_launches[1].mode == dlk::MODE_FOLD && dl_log_length(h) == 0);
    CHECK(dl_merge(h, nullptr) == DL_OK && g_launches.size() == 2);
    // split replay: each append is the key-side stage then the tiles; the fold stays fused
    CHECK(dl_set_split_replay(h, addr(PREP), dl_prep_bytes(&c)) == DL_OK);
    g_launches.clear();
    for (int t = 0; t < C; ++t) CHECK(dl_decode_step(h, &a0, nullptr) == DL_OK);
    CHECK(g_launches.size() == (size_t)2 * (C - 1) + 1);
    for (int t = 0; t < C - 1; ++t) {
        CHECK(g_launches[2 * t].mode == dlk::MODE_PREP && g_launches[2 * t].prep && g_launches[2 * t].L == t);
        CHECK(g_launches[2 * t + 1].mode == dlk::MODE_PREPPED && g_launches[2 * t + 1].L == t);
    }
    CHECK(g_launches.back().mode == dlk::MODE_MERGE);
    CHECK(dl_set_split_replay(h, nullptr, 0) == DL_OK);
    // the allocation-free step: the same two stages on the static scratch, the fold fused
    g_launches.clear();
    for (int t = 0; t < C; ++t) CHECK(dl_decode_step_noalloc(h, &a0, nullptr) == DL_OK);
    CHECK(g_launches.size() == (size_t)2 * (C - 1) + 1);
    for (int t = 0; t < C - 1; ++t) {
        CHECK(g_launches[2 * t].mode == dlk::MODE_PREP && g_launches[2 * t].prep && g_launches[2 * t].L == t);
        CHECK(g_launches[2 * t + 1].mode == dlk::MODE_PREPPED && g_launches[2 * t + 1].prep);
    }
    CHECK(g_launches.back().mode == dlk::MODE_MERGE && !g_launches.back().prep && dl_log_length(h) == 0);
    // several tokens per call: within the log, filling it, passing its end, and one token
    std::vector<dl_step_args> toks;
    for (int t = 0; t < 8; ++t) toks.push_back(token(op, t));
    g_launches.clear();
    CHECK(dl_decode_tokens(h, toks.data(), 3, nullptr) == DL_OK);  // L 0 -> 3
    CHECK(g_launches.back().kind == dlk::KIND_CHUNK && g_launches.back().L == 0 && g_launches.back().K == 3);
    CHECK(!g_launches.back().segmented && dl_log_length(h) == 3);
    CHECK(dl_decode_tokens(h, toks.data(), 2, nullptr) == DL_OK);  // L 3 -> fills at 5, folds
    CHECK(g_launches.back().L == 3 && !g_launches.back().segmented && dl_log_length(h) == 0);
    CHECK(dl_decode_tokens(h, toks.data(), 4, nullptr) == DL_OK);  // L 0 -> 4
    CHECK(dl_decode_tokens(h, toks.data(), 8, nullptr) == DL_OK);  // L 4 -> passes the end twice -> 2
    CHECK(g_launches.back().segmented && g_launches.back().L == 4 && g_launches.back().K == 8);
    CHECK(dl_log_length(h) == (4 + 8) % C);
    CHECK(dl_decode_tokens(h, toks.data(), 5, nullptr) == DL_OK);  // L 2 -> passes the end once -> 2
    CHECK(!g_launches.back().segmented && g_launches.back().L == 2 && g_launches.back().K == 5);
    CHECK(dl_log_length(h) == (2 + 5) % C);
    const size_t before = g_launches.size();
    CHECK(dl_decode_tokens(h, toks.data(), 1, nullptr) == DL_OK);  // one token: the single-token kernel
    CHECK(g_launches.size() == before + 1 && g_launches.back().kind == dlk::KIND_STEP);
    CHECK(dl_decode_tokens(h, toks.data(), 0, nullptr) == DL_ERR_SHAPE);
    CHECK(dl_decode_tokens(h, toks.data(), 9, nullptr) == DL_ERR_SHAPE);
    // aliasing: an output over an input, over the base, over the workspace; a dst over the log
    dl_step_args bad = token(op, 0);
    bad.out = static_cast<float *>(const_cast<void *>(bad.v));
    const int L0 = dl_log_length(h);
    CHECK(dl_decode_step(h, &bad, nullptr) == DL_ERR_ARG);
    bad = token(op, 0);
    bad.out = static_cast<float *>(addr(BASE + 4096));
    CHECK(dl_decode_step(h, &bad, nullptr) == DL_ERR_ARG);
    bad = token(op, 0);
    bad.k = addr(WS + 64);
    CHECK(dl_decode_step(h, &bad, nullptr) == DL_ERR_ARG);
    CHECK(dl_materialize(h, static_cast<float *>(addr(WS + ws - 256)), nullptr) == DL_ERR_ARG);
    CHECK(dl_log_length(h) == L0);
    // graph capture: refused away from an empty log; at L = 0 it either records (a GPU is
    // present) or reports the runtime's refusal (none is), and never changes L
    dl_graph *g = nullptr;
    const int rc = dl_graph_capture_cycle(&g, h, toks.data());
    if (L0 != 0)
        CHECK(rc == DL_ERR_ARG && g == nullptr);
    else
        CHECK((rc == DL_OK && g != nullptr) || (rc == DL_ERR_HIP && g == nullptr));
    if (g) dl_graph_destroy(g);
    CHECK(dl_log_length(h) == L0);
    dl_state_destroy(h);
    // the eager step
    g_launches.clear();
    dl_step_args e = token(op, 1);
    CHECK(dl_eager_step(&c, static_cast<float *>(addr(BASE)), &e, nullptr) == DL_OK);
    CHECK(g_launches.size() == 1 && g_launches[0].mode == dlk::MODE_EAGER);
    e.q = addr(BASE + 256);
    CHECK(dl_eager_step(&c, static_cast<float *>(addr(BASE)), &e, nullptr) == DL_ERR_ARG);
}

static void check_slots(int op) {
    const int C = 4, B = 5, H = 2;
    dl_config c = {op, DL_F32, B, H, 64, 32, C};
    dl_state *h = nullptr;
    g_launches.clear();
    CHECK(dl_state_init_slots(&h, &c, static_cast<float *>(addr(BASE)), addr(WS), dl_workspace_bytes(&c), nullptr) ==
          DL_OK);
    CHECK(g_launches.size() == 1 && g_launches[0].kind == dlk::KIND_SLOT_SET && g_launches[0].slot == -1);
    CHECK(g_launches[0].set_active && g_launches[0].active_value == 0);
    for (int b = 0; b < B; ++b) CHECK(dl_slot_log_length(h, b) == -1);
    dl_step_args a = token(op, 0);
    // no slot active: a step launches nothing, but time moves on
    g_launches.clear();
    CHECK(dl_decode_step(h, &a, nullptr) == DL_OK && g_launches.empty());
    int steps = 1, origin[B];
    for (int b = 0; b < B; ++b) origin[b] = -1;
    for (int b = 0; b < B; ++b) {
        CHECK(dl_slot_activate(h, b, nullptr) == DL_OK);
        CHECK(g_launches.back().kind == dlk::KIND_SLOT_SET && g_launches.back().slot == b);
        CHECK(g_launches.back().base_value == steps && g_launches.back().active_value == 1);
        origin[b] = steps;
        CHECK(dl_slot_log_length(h, b) == 0);
        CHECK(dl_decode_step(h, &a, nullptr) == DL_OK);
        CHECK(g_launches.back().kind == dlk::KIND_STEP && g_launches.back().mode == dlk::MODE_AUTO);
        CHECK(g_launches.back().slots && g_launches.back().step == (unsigned)steps);
        ++steps;
        for (int s = 0; s <= b; ++s) CHECK(dl_slot_log_length(h, s) == (steps - origin[s]) % C);
    }
    std::vector<dl_step_args> toks;
    for (int t = 0; t < 8; ++t) toks.push_back(token(op, t));
    CHECK(dl_decode_tokens(h, toks.data(), 7, nullptr) == DL_OK);
    CHECK(g_launches.back().kind == dlk::KIND_CHUNK && g_launches.back().segmented && g_launches.back().slots);
    CHECK(g_launches.back().step == (unsigned)steps);
    steps += 7;
    for (int b = 0; b < B; ++b) CHECK(dl_slot_log_length(h, b) == (steps - origin[b]) % C);
    CHECK(dl_decode_tokens(h, toks.data(), 3, nullptr) == DL_OK);  // K <= C: at most one fold per slot
    CHECK(g_launches.back().kind == dlk::KIND_CHUNK && !g_launches.back().segmented && g_launches.back().slots);
    CHECK(g_launches.back().step == (unsigned)steps);
    steps += 3;
    for (int b = 0; b < B; ++b) CHECK(dl_slot_log_length(h, b) == (steps - origin[b]) % C);
    // one slot folded early: only its log empties
    int target = -1;
    for (int b = 0; b < B && target < 0; ++b)
        if (dl_slot_log_length(h, b) > 0) target = b;
    CHECK(target >= 0);
    g_launches.clear();
    CHECK(dl_slot_merge(h, target, nullptr) == DL_OK);
    CHECK(g_launches.size() == 2 && g_launches[0].mode == dlk::MODE_FOLD && g_launches[0].N == H);
    CHECK(g_launches[1].kind == dlk::KIND_SLOT_SET && g_launches[1].slot == target);
    origin[target] = steps;
    for (int b = 0; b < B; ++b) CHECK(dl_slot_log_length(h, b) == (steps - origin[b]) % C);
    CHECK(dl_materialize_slot(h, 2, static_cast<float *>(addr(DST)), nullptr) == DL_OK);
    CHECK(g_launches.back().mode == dlk::MODE_FOLD && g_launches.back().N == H);
    CHECK(dl_materialize_slot(h, 2, static_cast<float *>(addr(BASE)), nullptr) == DL_ERR_ARG);
    CHECK(dl_slot_deactivate(h, 3, nullptr) == DL_OK && dl_slot_log_length(h, 3) == -1);
    CHECK(dl_slot_merge(h, 3, nullptr) == DL_ERR_ARG);
    CHECK(dl_slot_activate(h, B, nullptr) == DL_ERR_ARG && dl_slot_activate(h, -1, nullptr) == DL_ERR_ARG);
    // a whole-handle merge resets every active slot's origin
    g_launches.clear();
    CHECK(dl_merge(h, nullptr) == DL_OK);
    for (int b = 0; b < B; ++b)
        if (b != 3) CHECK(dl_slot_log_length(h, b) == 0);
    CHECK(dl_set_split_replay(h, addr(PREP), dl_prep_bytes(&c)) == DL_ERR_UNSUPPORTED);
    CHECK(dl_decode_step_noalloc(h, &a, nullptr) == DL_ERR_UNSUPPORTED);
    CHECK(dl_log_length(h) == -1);
    dl_state_destroy(h);
}

// The allocation-free step refuses a configuration whose records exceed its scratch.
static void check_noalloc_limit() {
    for (int heads : {7598, 7599}) {
        dl_config c = {DL_GDN, DL_BF16, heads, 1, 128, 128, 8};
        CHECK(dl_prep_bytes(&c) == (size_t)heads * 1104);
        dl_state *h = nullptr;
        CHECK(dl_state_init(&h, &c, static_cast<float *>(addr(BASE)), addr(BASE + (1ull << 36)),
                            dl_workspace_bytes(&c)) == DL_OK);
        dl_step_args a = token(DL_GDN, 0);
        a.q = addr(BASE + (2ull << 36));  // inputs clear of this large base
        a.k = addr(BASE + (2ull << 36) + (1ull << 30));
        a.v = addr(BASE + (2ull << 36) + (2ull << 30));
        a.beta = static_cast<const float *>(addr(BASE + (2ull << 36) + (3ull << 30)));
        a.decay = static_cast<const float *>(addr(BASE + (2ull << 36) + (4ull << 30)));
        a.out = static_cast<float *>(addr(BASE + (2ull << 36) + (5ull << 30)));
        const int rc = dl_decode_step_noalloc(h, &a, nullptr);
        CHECK(rc == (heads == 7598 ? DL_OK : DL_ERR_WORKSPACE));
        CHECK(dl_log_length(h) == (heads == 7598 ? 1 : 0));
        dl_state_destroy(h);
    }
}

int main() {
    check_configs();
    check_noalloc_limit();
    for (int op = 0; op < 3; ++op) {
        check_lockstep(op, 128, 128);
        check_lockstep(op, 64, 128);
        check_lockstep(op, 128, 32);
        check_slots(op);
    }
    CHECK(dl_status_string(DL_OK)[0] != '\0' && dl_status_string(-99)[0] != '\0');
    dl_state_destroy(nullptr);
    dl_graph_destroy(nullptr);
    printf("host_check: %d checks passed\n", g_checks);
    return 0;
}
