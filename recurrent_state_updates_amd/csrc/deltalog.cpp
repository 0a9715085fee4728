// deltalog.cpp -- the C ABI declared in include/deltalog.h: argument
// validation, the host-side log-length bookkeeping and kernel dispatch.
//
// The handle lives in host memory only.  On a lockstep handle the log length
// L is the same for every slot and head, so it is tracked here and passed to
// each launch; the launch mode follows from (L, C): append while L + 1 < C,
// and decode + fold when the token fills the log (the signal-papers summary,
// caption of Fig. 4: append while L < C, materialise when L = C).  On a
// per-slot handle each slot's length is (steps issued - the slot's origin)
// mod C; the origins live in the workspace, written in stream order by a
// small kernel, and the workgroups of one launch read them to choose between
// appending and folding.  A host mirror of the origins serves validation and
// dl_slot_log_length.
#include "../../include/deltalog.h"

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include <algorithm>
#include <new>
#include <string>
#include <vector>

#include "launch.h"

struct dl_state {
    dl_config cfg;
    float *base;
    void *logX;
    void *logK;
    float *logG;
    int L;  // lockstep log length
    // per-slot logs (continuous batching): device arrays in the workspace and
    // their host mirror; slot b's log length is (step - base[b]) mod C
    bool slots;
    int *slot_base;
    unsigned char *slot_active;
    std::vector<unsigned> h_base;
    std::vector<unsigned char> h_active;
    unsigned step;
    // split replay: per-head prep records (NULL: the fused per-tile preparation)
    float *prep;
    // byte ranges the handle's launches write: the base, the part of the
    // workspace the kernels use, the prep records (empty when unset)
    uintptr_t base_lo, base_hi, ws_lo, ws_hi, prep_lo, prep_hi;
};

// A merge cycle captured for replay (dl_graph_capture_cycle).
struct dl_graph {
    dl_state *h;
    hipGraphExec_t exec;
};

namespace {

thread_local std::string g_last_error;

dl_status fail(dl_status st, const std::string &msg) {
    g_last_error = msg;
    return st;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A byte range [lo, hi) of device memory; a NULL pointer is an empty range.
struct Span {
    uintptr_t lo, hi;
};

Span span(const void *p, size_t bytes) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return p ? Span{a, a + bytes} : Span{0, 0};
}

bool overlap(Span a, Span b) { return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi; }

// A buffer a call writes, by name, for the messages.
struct Written {
    Span s;
    const char *name;
};

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

size_t in_size(int dtype) { return dtype == DL_BF16 ? 2 : 4; }

// Compile-time bound on log entries of the kernels that serve capacity C.
int cmax_of(const dl_config *cfg) { return cfg->C <= 8 ? 8 : (cfg->C <= 16 ? 16 : 32); }

// Validate a config; on success *heads receives B*H.
dl_status check_config(const dl_config *cfg, size_t *heads) {
    if (!cfg) return fail(DL_ERR_ARG, "cfg is NULL");
    if (cfg->op < DL_GDN || cfg->op > DL_RWKV6) return fail(DL_ERR_ARG, "cfg->op is not a dl_op");
    if (cfg->in_dtype != DL_F32 && cfg->in_dtype != DL_BF16)
        return fail(DL_ERR_ARG, "cfg->in_dtype is not a dl_dtype");
    if (cfg->B <= 0 || cfg->H <= 0 || cfg->dk <= 0 || cfg->dv <= 0)
        return fail(DL_ERR_SHAPE, "B, H, dk and dv must be positive");
    if (cfg->C < 1 || cfg->C > DL_MAX_CAPACITY) return fail(DL_ERR_SHAPE, "C must lie in [1, 32]");
    auto built = [](int w) { return w == 32 || w == 64 || w == 128; };
    if (!built(cfg->dk) || !built(cfg->dv)) return fail(DL_ERR_UNSUPPORTED, "dk and dv must each be 32, 64 or 128");
    const size_t n = (size_t)cfg->B * (size_t)cfg->H;
    // a launch holds at most 2^32 work-items and the widest kernel runs 512 per head
    if (n > (size_t)DL_MAX_HEADS) return fail(DL_ERR_SHAPE, "B * H exceeds DL_MAX_HEADS");
    *heads = n;
    return DL_OK;
}

struct Layout {
    size_t x, k, g, sb, sa, total;
};

Layout layout_of(const dl_config *cfg, size_t heads) {
    const size_t entries = heads * (size_t)cfg->C;
    const size_t xs = cfg->op == DL_RWKV6 ? in_size(cfg->in_dtype) : 4;
    const size_t gw = cfg->op == DL_GDN ? 1 : (size_t)cfg->dk;
    Layout l;
    l.x = 0;
    l.k = round_up(entries * cfg->dv * xs, 256);
    l.g = l.k + round_up(entries * cfg->dk * in_size(cfg->in_dtype), 256);
    l.sb = l.g + round_up(entries * gw * 4, 256);            // per-slot log origin [B] int32
    l.sa = l.sb + round_up((size_t)cfg->B * 4, 256);         // per-slot active flag [B] uint8
    l.total = l.sa + round_up((size_t)cfg->B, 256);
    return l;
}

// The byte ranges of one token's inputs ([0] q, [1] k, [2] v, [3] beta,
// [4] decay, [5] bonus) and of its output.
struct TokenSpans {
    Span in[6];
    Span out;
};

TokenSpans token_spans(const dl_config *cfg, const dl_step_args *a) {
    const size_t n = (size_t)cfg->B * (size_t)cfg->H, es = in_size(cfg->in_dtype);
    TokenSpans t;
    t.in[0] = span(a->q, n * cfg->dk * es);
    t.in[1] = span(a->k, n * cfg->dk * es);
    t.in[2] = span(a->v, n * cfg->dv * es);
    t.in[3] = span(a->beta, n * 4);
    t.in[4] = span(a->decay, (cfg->op == DL_GDN ? n : n * cfg->dk) * 4);
    t.in[5] = span(a->bonus, (size_t)cfg->H * cfg->dk * 4);
    t.out = span(a->out, n * cfg->dv * 4);
    return t;
}

// No aliasing a launch could race on: the token's output overlaps none of its
// inputs, and neither overlaps a buffer the call writes.
dl_status check_token_aliasing(const dl_config *cfg, const dl_step_args *a, const Written *w, int nw) {
    static const char *in_names[6] = {"q", "k", "v", "beta", "decay", "bonus"};
    const TokenSpans t = token_spans(cfg, a);
    for (int i = 0; i < 6; ++i)
        if (overlap(t.out, t.in[i]))
            return fail(DL_ERR_ARG, std::string("out overlaps the token's input ") + in_names[i]);
    for (int j = 0; j < nw; ++j) {
        if (overlap(t.out, w[j].s)) return fail(DL_ERR_ARG, std::string("out overlaps the ") + w[j].name);
        for (int i = 0; i < 6; ++i)
            if (overlap(t.in[i], w[j].s))
                return fail(DL_ERR_ARG, std::string("input ") + in_names[i] + " overlaps the " + w[j].name +
                                            ", which the call writes");
    }
    return DL_OK;
}

// The buffers a handle's decode, merge and materialise launches write.
int handle_written(const dl_state *h, Written w[3]) {
    w[0] = {Span{h->base_lo, h->base_hi}, "base"};
    w[1] = {Span{h->ws_lo, h->ws_hi}, "workspace"};
    w[2] = {Span{h->prep_lo, h->prep_hi}, "prep buffer"};
    return 3;
}

dl_status check_args(const dl_config *cfg, const dl_step_args *a) {
    if (!a) return fail(DL_ERR_ARG, "args is NULL");
    if (!a->q || !a->k || !a->v || !a->decay || !a->out)
        return fail(DL_ERR_ARG, "args->q, k, v, decay and out must be non-NULL");
    if (cfg->op == DL_RWKV6) {
        if (a->beta) return fail(DL_ERR_ARG, "args->beta must be NULL for RWKV6");
        if (!a->bonus) return fail(DL_ERR_ARG, "args->bonus is required for RWKV6");
    } else {
        if (!a->beta) return fail(DL_ERR_ARG, "args->beta is required for GDN and KDA");
        if (a->bonus) return fail(DL_ERR_ARG, "args->bonus must be NULL for GDN and KDA");
    }
    const size_t es = in_size(cfg->in_dtype);
    auto addr = [](const void *p) { return reinterpret_cast<uintptr_t>(p); };
    // the kernels read q and k four channels at a time (one 8- or 16-byte
    // load), and the per-channel decays and the bonus as float4
    if (addr(a->q) % (4 * es) != 0 || addr(a->k) % (4 * es) != 0)
        return fail(DL_ERR_ARG, "q and k must be aligned to four elements (8 bytes in bf16, 16 in f32)");
    if (addr(a->v) % es != 0) return fail(DL_ERR_ARG, "v must be aligned to its element size");
    if ((cfg->op != DL_GDN && addr(a->decay) % 16 != 0) || addr(a->bonus) % 16 != 0)
        return fail(DL_ERR_ARG, "the per-channel decay and the bonus must be 16-byte aligned");
    const void *f32_ptrs[] = {a->beta, a->decay, a->out};
    for (const void *p : f32_ptrs)
        if (addr(p) % 4 != 0) return fail(DL_ERR_ARG, "beta, decay and out must be 4-byte aligned");
    return DL_OK;
}

// check_args plus the aliasing rules against a handle's buffers.
dl_status check_step(const dl_state *h, const dl_step_args *a) {
    dl_status st = check_args(&h->cfg, a);
    if (st != DL_OK) return st;
    Written w[3];
    const int nw = handle_written(h, w);
    return check_token_aliasing(&h->cfg, a, w, nw);
}

// The single-token and multi-token kernels of one operator, by key width.
template <int OP>
hipError_t step_of_op(const dl_config *cfg, int mode, const dlk::StepParams &p, hipStream_t s) {
    const int bf16 = cfg->in_dtype == DL_BF16, cmax = cmax_of(cfg);
    switch (cfg->dk) {
        case 32: return dlk::launch_step<OP, 32>(bf16, cfg->dv, mode, cmax, p, s);
        case 64: return dlk::launch_step<OP, 64>(bf16, cfg->dv, mode, cmax, p, s);
        case 128: return dlk::launch_step<OP, 128>(bf16, cfg->dv, mode, cmax, p, s);
        default: return hipErrorInvalidValue;
    }
}

template <int OP>
hipError_t chunk_of_op(const dl_config *cfg, const dlk::ChunkParams &p, hipStream_t s) {
    const int bf16 = cfg->in_dtype == DL_BF16, cmax = cmax_of(cfg);
    switch (cfg->dk) {
        case 32: return dlk::launch_chunk<OP, 32>(bf16, cfg->dv, cmax, p, s);
        case 64: return dlk::launch_chunk<OP, 64>(bf16, cfg->dv, cmax, p, s);
        case 128: return dlk::launch_chunk<OP, 128>(bf16, cfg->dv, cmax, p, s);
        default: return hipErrorInvalidValue;
    }
}

dl_status launch(const dl_config *cfg, int mode, const dlk::StepParams &p, void *stream) {
    const hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    switch (cfg->op) {
        case DL_GDN: e = step_of_op<dlk::OP_GDN>(cfg, mode, p, s); break;
        case DL_KDA: e = step_of_op<dlk::OP_KDA>(cfg, mode, p, s); break;
        default: e = step_of_op<dlk::OP_RWKV6>(cfg, mode, p, s); break;
    }
    if (e != hipSuccess)
        return fail(DL_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
    return DL_OK;
}

dlk::StepParams params_of(const dl_config *cfg, size_t heads) {
    dlk::StepParams p = {};
    p.C = cfg->C;
    p.H = cfg->H;
    p.N = (int)heads;
    return p;
}

void set_token(dlk::StepParams &p, const dl_step_args *a) {
    p.q = a->q;
    p.k = a->k;
    p.v = a->v;
    p.beta = a->beta;
    p.decay = a->decay;
    p.bonus = a->bonus;
    p.out = a->out;
}

void set_log(dlk::StepParams &p, const dl_state *h) {
    p.base = h->base;
    p.logX = h->logX;
    p.logK = h->logK;
    p.logG = h->logG;
    p.L = h->L;
    p.prep = h->prep;
    if (h->slots) {
        p.slot_base = h->slot_base;
        p.slot_active = h->slot_active;
        p.step = h->step;
    }
}

int slot_length(const dl_state *h, int b) { return (int)((h->step - h->h_base[b]) % (unsigned)h->cfg.C); }

dl_status slot_set(dl_state *h, int slot, int set_base, int base_value, int set_active, int active_value,
                   int only_active, void *stream) {
    const hipError_t e = dlk::launch_slot_set(h->slot_base, h->slot_active, h->cfg.B, slot, set_base, base_value,
                                              set_active, active_value, only_active,
                                              static_cast<hipStream_t>(stream));
    if (e != hipSuccess)
        return fail(DL_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
    return DL_OK;
}

dl_status init_handle(dl_state **out, const dl_config *cfg, float *base, void *workspace,
                      size_t workspace_bytes, bool slots) {
    if (!out) return fail(DL_ERR_ARG, "out is NULL");
    *out = nullptr;
    size_t heads = 0;
    dl_status st = check_config(cfg, &heads);
    if (st != DL_OK) return st;
    if (!base || !workspace) return fail(DL_ERR_ARG, "base and workspace must be non-NULL");
    if (!aligned16(base) || !aligned16(workspace))
        return fail(DL_ERR_ARG, "base and workspace must be 16-byte aligned");
    const Layout l = layout_of(cfg, heads);
    if (workspace_bytes < l.total)
        return fail(DL_ERR_WORKSPACE, "workspace is smaller than dl_workspace_bytes(cfg) = " +
                                          std::to_string(l.total));
    const Span sb = span(base, heads * (size_t)cfg->dk * (size_t)cfg->dv * 4);
    const Span sw = span(workspace, l.total);
    if (overlap(sb, sw)) return fail(DL_ERR_ARG, "base and workspace overlap");
    dl_state *h = new (std::nothrow) dl_state;
    if (!h) return fail(DL_ERR_ARG, "out of host memory");
    char *ws = static_cast<char *>(workspace);
    h->cfg = *cfg;
    h->base = base;
    h->logX = ws + l.x;
    h->logK = ws + l.k;
    h->logG = reinterpret_cast<float *>(ws + l.g);
    h->L = 0;
    h->slots = slots;
    h->slot_base = reinterpret_cast<int *>(ws + l.sb);
    h->slot_active = reinterpret_cast<unsigned char *>(ws + l.sa);
    h->step = 0;
    h->prep = nullptr;
    h->base_lo = sb.lo;
    h->base_hi = sb.hi;
    h->ws_lo = sw.lo;
    h->ws_hi = sw.hi;
    h->prep_lo = h->prep_hi = 0;
    if (slots) {
        h->h_base.assign(cfg->B, 0u);
        h->h_active.assign(cfg->B, 0);
    }
    *out = h;
    g_last_error.clear();
    return DL_OK;
}

// Per-head bytes of the traffic model (mirrored by traffic.py for the bench).
struct HeadBytes {
    double base, token, out, entry, shared;
};

HeadBytes head_bytes(const dl_config *cfg) {
    const double d = cfg->dk, s = (double)in_size(cfg->in_dtype);
    HeadBytes b;
    b.base = 4.0 * d * cfg->dv;
    b.token = 2.0 * d * s + cfg->dv * s + (cfg->op != DL_RWKV6 ? 4.0 : 0.0) +
              (cfg->op == DL_GDN ? 4.0 : 4.0 * d);
    b.out = 4.0 * cfg->dv;
    b.entry = (cfg->op == DL_RWKV6 ? cfg->dv * s : 4.0 * cfg->dv) + d * s +
              (cfg->op == DL_GDN ? 4.0 : 4.0 * d);
    b.shared = cfg->op == DL_RWKV6 ? 4.0 * d * cfg->H : 0.0;
    return b;
}

}  // namespace

extern "C" {

size_t dl_workspace_bytes(const dl_config *cfg) {
    size_t heads = 0;
    if (check_config(cfg, &heads) != DL_OK) return 0;
    return layout_of(cfg, heads).total;
}

dl_status dl_workspace_layout(const dl_config *cfg, size_t offsets[3]) {
    size_t heads = 0;
    dl_status st = check_config(cfg, &heads);
    if (st != DL_OK) return st;
    if (!offsets) return fail(DL_ERR_ARG, "offsets is NULL");
    const Layout l = layout_of(cfg, heads);
    offsets[0] = l.x;
    offsets[1] = l.k;
    offsets[2] = l.g;
    return DL_OK;
}

dl_status dl_state_init(dl_state **out, const dl_config *cfg, float *base, void *workspace,
                        size_t workspace_bytes) {
    return init_handle(out, cfg, base, workspace, workspace_bytes, false);
}

dl_status dl_state_init_slots(dl_state **out, const dl_config *cfg, float *base, void *workspace,
                              size_t workspace_bytes, void *stream) {
    dl_status st = init_handle(out, cfg, base, workspace, workspace_bytes, true);
    if (st != DL_OK) return st;
    st = slot_set(*out, -1, 1, 0, 1, 0, 0, stream);  // every slot inactive, origin 0
    if (st != DL_OK) {
        delete *out;
        *out = nullptr;
    }
    return st;
}

dl_status dl_slot_activate(dl_state *h, int slot, void *stream) {
    if (!h || !h->slots) return fail(DL_ERR_ARG, "handle is NULL or not a per-slot handle");
    if (slot < 0 || slot >= h->cfg.B) return fail(DL_ERR_ARG, "slot out of range");
    dl_status st = slot_set(h, slot, 1, (int)h->step, 1, 1, 0, stream);
    if (st != DL_OK) return st;
    h->h_base[slot] = h->step;
    h->h_active[slot] = 1;
    return DL_OK;
}

dl_status dl_slot_deactivate(dl_state *h, int slot, void *stream) {
    if (!h || !h->slots) return fail(DL_ERR_ARG, "handle is NULL or not a per-slot handle");
    if (slot < 0 || slot >= h->cfg.B) return fail(DL_ERR_ARG, "slot out of range");
    dl_status st = slot_set(h, slot, 0, 0, 1, 0, 0, stream);
    if (st != DL_OK) return st;
    h->h_active[slot] = 0;
    return DL_OK;
}

int dl_slot_log_length(const dl_state *h, int slot) {
    if (!h || !h->slots || slot < 0 || slot >= h->cfg.B || !h->h_active[slot]) return -1;
    return slot_length(h, slot);
}

dl_status dl_decode_step(dl_state *h, const dl_step_args *a, void *stream) {
    if (!h) return fail(DL_ERR_ARG, "handle is NULL");
    size_t heads = 0;
    dl_status st = check_config(&h->cfg, &heads);
    if (st != DL_OK) return st;
    st = check_step(h, a);
    if (st != DL_OK) return st;
    dlk::StepParams p = params_of(&h->cfg, heads);
    set_log(p, h);
    set_token(p, a);
    p.dst = h->base;
    if (h->slots) {
        // one launch: each active slot appends, or decodes and folds when its
        // token fills its log (its workgroups choose at run time)
        bool any = false;
        for (int b = 0; b < h->cfg.B; ++b) any = any || h->h_active[b];
        if (any && (st = launch(&h->cfg, dlk::MODE_AUTO, p, stream)) != DL_OK) return st;
        ++h->step;
        return DL_OK;
    }
    const bool fold = h->L + 1 == h->cfg.C;
    if (fold || !h->prep) {
        st = launch(&h->cfg, fold ? dlk::MODE_MERGE : dlk::MODE_APPEND, p, stream);
    } else {
        // split replay: the key-side stage once per head, then the tiles
        st = launch(&h->cfg, dlk::MODE_PREP, p, stream);
        if (st == DL_OK) st = launch(&h->cfg, dlk::MODE_PREPPED, p, stream);
    }
    if (st != DL_OK) return st;
    h->L = fold ? 0 : h->L + 1;
    return DL_OK;
}

dl_status dl_decode_step_noalloc(dl_state *h, const dl_step_args *a, void *stream) {
    if (!h) return fail(DL_ERR_ARG, "handle is NULL");
    if (h->slots) return fail(DL_ERR_UNSUPPORTED, "the allocation-free decode step needs a lockstep handle");
    size_t heads = 0;
    dl_status st = check_config(&h->cfg, &heads);
    if (st != DL_OK) return st;
    const size_t need = dl_prep_bytes(&h->cfg);
    if (need > DL_NOALLOC_PREP_BYTES)
        return fail(DL_ERR_WORKSPACE, "this configuration's prep records take " + std::to_string(need) +
                                          " bytes, more than the static scratch of DL_NOALLOC_PREP_BYTES = " +
                                          std::to_string((size_t)DL_NOALLOC_PREP_BYTES));
    st = check_step(h, a);
    if (st != DL_OK) return st;
    dlk::StepParams p = params_of(&h->cfg, heads);
    set_log(p, h);
    set_token(p, a);
    p.dst = h->base;
    const bool fold = h->L + 1 == h->cfg.C;
    if (fold) {
        // the fold step keeps its fused form (as with a prep buffer): no scratch
        p.prep = nullptr;
        st = launch(&h->cfg, dlk::MODE_MERGE, p, stream);
    } else {
        void *scr = nullptr;
        const hipError_t e = dlk::static_prep_scratch(&scr);
        if (e != hipSuccess)
            return fail(DL_ERR_HIP, std::string("static scratch lookup failed: ") + hipGetErrorString(e));
        p.prep = static_cast<float *>(scr);
        st = launch(&h->cfg, dlk::MODE_PREP, p, stream);
        if (st == DL_OK) st = launch(&h->cfg, dlk::MODE_PREPPED, p, stream);
    }
    if (st != DL_OK) return st;
    h->L = fold ? 0 : h->L + 1;
    return DL_OK;
}

dl_status dl_decode_tokens(dl_state *h, const dl_step_args *args, int K, void *stream) {
    if (!h) return fail(DL_ERR_ARG, "handle is NULL");
    size_t heads = 0;
    dl_status st = check_config(&h->cfg, &heads);
    if (st != DL_OK) return st;
    if (!args) return fail(DL_ERR_ARG, "args is NULL");
    if (K < 1 || K > DL_MAX_TOKENS) return fail(DL_ERR_SHAPE, "K must lie in [1, 8]");
    for (int t = 0; t < K; ++t)
        if ((st = check_step(h, &args[t])) != DL_OK) return st;
    // one launch reads every token's inputs and writes every token's output:
    // no output may overlap another token's inputs or output
    for (int t = 0; t < K; ++t) {
        const TokenSpans ts = token_spans(&h->cfg, &args[t]);
        for (int u = 0; u < K; ++u) {
            if (u == t) continue;
            const TokenSpans us = token_spans(&h->cfg, &args[u]);
            if (overlap(ts.out, us.out))
                return fail(DL_ERR_ARG, "two tokens of the call write overlapping outputs");
            for (const Span &in : us.in)
                if (overlap(ts.out, in))
                    return fail(DL_ERR_ARG, "a token's out overlaps another token's input");
        }
    }
    // the bonus is a per-head parameter: one launch takes it from the first token
    for (int t = 1; t < K; ++t)
        if (args[t].bonus != args[0].bonus)
            return fail(DL_ERR_ARG, "every token of a call must carry the same bonus");
    const hipStream_t s = static_cast<hipStream_t>(stream);
    // tokens t0 .. t0 + k - 1 of the call as one chunk
    auto chunk_of = [&](int t0, int k) {
        dlk::ChunkParams p = {};
        p.base = h->base;
        for (int t = 0; t < k; ++t) {
            const dl_step_args &a = args[t0 + t];
            p.q[t] = a.q;
            p.k[t] = a.k;
            p.v[t] = a.v;
            p.beta[t] = a.beta;
            p.decay[t] = a.decay;
            p.out[t] = a.out;
        }
        p.bonus = args[t0].bonus;
        p.logX = h->logX;
        p.logK = h->logK;
        p.logG = h->logG;
        p.C = h->cfg.C;
        p.H = h->cfg.H;
        p.N = (int)heads;
        p.K = k;
        return p;
    };
    auto launch_chunk = [&](const dlk::ChunkParams &p) -> dl_status {
        hipError_t e;
        switch (h->cfg.op) {
            case DL_GDN: e = chunk_of_op<dlk::OP_GDN>(&h->cfg, p, s); break;
            case DL_KDA: e = chunk_of_op<dlk::OP_KDA>(&h->cfg, p, s); break;
            default: e = chunk_of_op<dlk::OP_RWKV6>(&h->cfg, p, s); break;
        }
        if (e != hipSuccess)
            return fail(DL_ERR_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
        return DL_OK;
    };
    // one token: the single-token kernel is faster than a chunk of one
    if (K == 1) return dl_decode_step(h, &args[0], stream);
    if (h->slots) {
        // Every slot's log fills at its own token: one launch, in which each
        // slot folds when its log fills and goes on from there.
        dlk::ChunkParams p = chunk_of(0, K);
        p.segmented = K > h->cfg.C;
        p.slot_base = h->slot_base;
        p.slot_active = h->slot_active;
        p.step = h->step;
        if ((st = launch_chunk(p)) != DL_OK) return st;
        h->step += (unsigned)K;
        return DL_OK;
    }
    // a call that passes the log's end folds there and goes on in the same
    // launch; one of more tokens than C folds more than once (segmented)
    dlk::ChunkParams p = chunk_of(0, K);
    p.L = h->L;
    p.segmented = K > h->cfg.C;
    if ((st = launch_chunk(p)) != DL_OK) return st;
    h->L = (h->L + K) % h->cfg.C;
    return DL_OK;
}

dl_status dl_merge(dl_state *h, void *stream) {
    if (!h) return fail(DL_ERR_ARG, "handle is NULL");
    size_t heads = 0;
    dl_status st = check_config(&h->cfg, &heads);
    if (st != DL_OK) return st;
    if (h->slots) {
        bool any = false;
        for (int b = 0; b < h->cfg.B; ++b) any = any || (h->h_active[b] && slot_length(h, b) > 0);
        if (!any) return DL_OK;
        dlk::StepParams p = params_of(&h->cfg, heads);
        set_log(p, h);
        p.dst = h->base;
        if ((st = launch(&h->cfg, dlk::MODE_FOLD, p, stream)) != DL_OK) return st;
        // every active slot's log is now empty: its origin moves to this step
        if ((st = slot_set(h, -1, 1, (int)h->step, 0, 0, 1, stream)) != DL_OK) return st;
        for (int b = 0; b < h->cfg.B; ++b)
            if (h->h_active[b]) h->h_base[b] = h->step;
        return DL_OK;
    }
    if (h->L == 0) return DL_OK;
    dlk::StepParams p = params_of(&h->cfg, heads);
    set_log(p, h);
    p.dst = h->base;
    st = launch(&h->cfg, dlk::MODE_FOLD, p, stream);
    if (st != DL_OK) return st;
    h->L = 0;
    return DL_OK;
}

dl_status dl_materialize(const dl_state *h, float *dst, void *stream) {
    if (!h) return fail(DL_ERR_ARG, "handle is NULL");
    if (!dst) return fail(DL_ERR_ARG, "dst is NULL");
    if (!aligned16(dst)) return fail(DL_ERR_ARG, "dst must be 16-byte aligned");
    size_t heads = 0;
    dl_status st = check_config(&h->cfg, &heads);
    if (st != DL_OK) return st;
    // the launch reads the base, the log and (never) the prep records while
    // its workgroups write dst: dst must overlap none of them
    const Span sd = span(dst, heads * (size_t)h->cfg.dk * (size_t)h->cfg.dv * 4);
    Written w[3];
    const int nw = handle_written(h, w);
    for (int j = 0; j < nw; ++j)
        if (overlap(sd, w[j].s))
            return fail(DL_ERR_ARG, std::string("dst overlaps the ") + w[j].name + " (use dl_merge to fold in place)");
    dlk::StepParams p = params_of(&h->cfg, heads);
    set_log(p, h);
    p.dst = dst;
    return launch(&h->cfg, dlk::MODE_FOLD, p, stream);
}

// A FOLD launch over the H heads of one slot: every pointer moves to that
// slot's heads, so the kernel sees a batch of one (its slot index is 0).
dlk::StepParams slot_fold_params(const dl_state *h, int slot, float *dst) {
    const dl_config &c = h->cfg;
    const size_t head0 = (size_t)slot * (size_t)c.H;
    const size_t xs = c.op == DL_RWKV6 ? in_size(c.in_dtype) : 4;
    const size_t gw = c.op == DL_GDN ? 1 : (size_t)c.dk;
    dlk::StepParams p = params_of(&c, (size_t)c.H);
    p.base = h->base + head0 * (size_t)c.dk * (size_t)c.dv;
    p.dst = dst;
    p.logX = static_cast<char *>(h->logX) + head0 * (size_t)c.C * (size_t)c.dv * xs;
    p.logK = static_cast<char *>(h->logK) + head0 * (size_t)c.C * (size_t)c.dk * in_size(c.in_dtype);
    p.logG = h->logG + head0 * (size_t)c.C * gw;
    p.L = h->L;
    p.prep = nullptr;
    if (h->slots) {
        p.slot_base = h->slot_base + slot;
        p.slot_active = h->slot_active + slot;
        p.step = h->step;
    }
    return p;
}

int dl_log_length(const dl_state *h) { return (h && !h->slots) ? h->L : -1; }

dl_status dl_materialize_slot(const dl_state *h, int slot, float *dst, void *stream) {
    if (!h) return fail(DL_ERR_ARG, "handle is NULL");
    if (slot < 0 || slot >= h->cfg.B) return fail(DL_ERR_ARG, "slot out of range");
    if (!dst) return fail(DL_ERR_ARG, "dst is NULL");
    if (!aligned16(dst)) return fail(DL_ERR_ARG, "dst must be 16-byte aligned");
    const size_t blk = (size_t)h->cfg.H * (size_t)h->cfg.dk * (size_t)h->cfg.dv;
    const Span sd = span(dst, blk * 4);
    Written w[3];
    const int nw = handle_written(h, w);
    for (int j = 0; j < nw; ++j)
        if (overlap(sd, w[j].s)) return fail(DL_ERR_ARG, std::string("dst overlaps the ") + w[j].name);
    if (h->slots && !h->h_active[slot]) return fail(DL_ERR_ARG, "slot is not active");
    return launch(&h->cfg, dlk::MODE_FOLD, slot_fold_params(h, slot, dst), stream);
}

dl_status dl_slot_merge(dl_state *h, int slot, void *stream) {
    if (!h || !h->slots) return fail(DL_ERR_ARG, "handle is NULL or not a per-slot handle");
    if (slot < 0 || slot >= h->cfg.B) return fail(DL_ERR_ARG, "slot out of range");
    if (!h->h_active[slot]) return fail(DL_ERR_ARG, "slot is not active");
    if (slot_length(h, slot) == 0) return DL_OK;
    const size_t head0 = (size_t)slot * (size_t)h->cfg.H;
    dl_status st = launch(&h->cfg, dlk::MODE_FOLD,
                          slot_fold_params(h, slot, h->base + head0 * (size_t)h->cfg.dk * (size_t)h->cfg.dv), stream);
    if (st != DL_OK) return st;
    // the slot's log is now empty: its origin moves to this step
    if ((st = slot_set(h, slot, 1, (int)h->step, 0, 0, 0, stream)) != DL_OK) return st;
    h->h_base[slot] = h->step;
    return DL_OK;
}

size_t dl_prep_bytes(const dl_config *cfg) {
    size_t heads = 0;
    if (check_config(cfg, &heads) != DL_OK) return 0;
    return heads * (size_t)dlk::prep_stride(cfg->dk, cmax_of(cfg)) * 4;
}

dl_status dl_set_split_replay(dl_state *h, void *prep, size_t prep_bytes) {
    if (!h) return fail(DL_ERR_ARG, "handle is NULL");
    if (h->slots) return fail(DL_ERR_UNSUPPORTED, "split replay needs a lockstep handle");
    if (!prep) {
        h->prep = nullptr;
        h->prep_lo = h->prep_hi = 0;
        return DL_OK;
    }
    if (!aligned16(prep)) return fail(DL_ERR_ARG, "prep must be 16-byte aligned");
    const size_t need = dl_prep_bytes(&h->cfg);
    if (prep_bytes < need)
        return fail(DL_ERR_WORKSPACE, "prep is smaller than dl_prep_bytes(cfg) = " + std::to_string(need));
    const Span sp = span(prep, need);
    if (overlap(sp, Span{h->base_lo, h->base_hi}) || overlap(sp, Span{h->ws_lo, h->ws_hi}))
        return fail(DL_ERR_ARG, "prep overlaps the base or the workspace");
    h->prep = static_cast<float *>(prep);
    h->prep_lo = sp.lo;
    h->prep_hi = sp.hi;
    return DL_OK;
}

dl_status dl_graph_capture_cycle(dl_graph **out, dl_state *h, const dl_step_args *args) {
    if (!out) return fail(DL_ERR_ARG, "out is NULL");
    *out = nullptr;
    if (!h) return fail(DL_ERR_ARG, "handle is NULL");
    if (h->slots) return fail(DL_ERR_UNSUPPORTED, "graph capture needs a lockstep handle");
    if (h->L != 0) return fail(DL_ERR_ARG, "a cycle is captured at an empty log (dl_log_length() == 0)");
    if (!args) return fail(DL_ERR_ARG, "args is NULL");
    dl_status st;
    for (int t = 0; t < h->cfg.C; ++t)
        if ((st = check_step(h, &args[t])) != DL_OK) return st;
    hipStream_t cs = nullptr;
    hipError_t e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
    if (e != hipSuccess) return fail(DL_ERR_HIP, std::string("hipStreamCreate: ") + hipGetErrorString(e));
    e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess) {
        (void)hipStreamDestroy(cs);
        return fail(DL_ERR_HIP, std::string("hipStreamBeginCapture: ") + hipGetErrorString(e));
    }
    // recording runs nothing; a whole cycle brings L back to 0 either way
    st = DL_OK;
    for (int t = 0; t < h->cfg.C && st == DL_OK; ++t) st = dl_decode_step(h, &args[t], cs);
    hipGraph_t g = nullptr;
    const hipError_t ee = hipStreamEndCapture(cs, &g);
    h->L = 0;
    (void)hipStreamDestroy(cs);
    if (st != DL_OK || ee != hipSuccess) {
        if (g) (void)hipGraphDestroy(g);
        return st != DL_OK ? st : fail(DL_ERR_HIP, std::string("hipStreamEndCapture: ") + hipGetErrorString(ee));
    }
    hipGraphExec_t exec = nullptr;
    e = hipGraphInstantiate(&exec, g, nullptr, nullptr, 0);
    (void)hipGraphDestroy(g);
    if (e != hipSuccess) return fail(DL_ERR_HIP, std::string("hipGraphInstantiate: ") + hipGetErrorString(e));
    dl_graph *gr = new (std::nothrow) dl_graph;
    if (!gr) {
        (void)hipGraphExecDestroy(exec);
        return fail(DL_ERR_ARG, "out of host memory");
    }
    gr->h = h;
    gr->exec = exec;
    *out = gr;
    return DL_OK;
}

dl_status dl_graph_launch(dl_graph *g, void *stream) {
    if (!g) return fail(DL_ERR_ARG, "graph is NULL");
    if (g->h->L != 0) return fail(DL_ERR_ARG, "the handle's log is not empty: a cycle replays at L == 0");
    const hipError_t e = hipGraphLaunch(g->exec, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(DL_ERR_HIP, std::string("hipGraphLaunch: ") + hipGetErrorString(e));
    return DL_OK;
}

void dl_graph_destroy(dl_graph *g) {
    if (!g) return;
    (void)hipGraphExecDestroy(g->exec);
    delete g;
}

dl_status dl_eager_step(const dl_config *cfg, float *state, const dl_step_args *a, void *stream) {
    size_t heads = 0;
    dl_status st = check_config(cfg, &heads);
    if (st != DL_OK) return st;
    if (!state) return fail(DL_ERR_ARG, "state is NULL");
    if (!aligned16(state)) return fail(DL_ERR_ARG, "state must be 16-byte aligned");
    st = check_args(cfg, a);
    if (st != DL_OK) return st;
    const Written w = {span(state, heads * (size_t)cfg->dk * (size_t)cfg->dv * 4), "state"};
    if ((st = check_token_aliasing(cfg, a, &w, 1)) != DL_OK) return st;
    dlk::StepParams p = params_of(cfg, heads);
    set_token(p, a);
    p.base = state;
    p.dst = state;
    return launch(cfg, dlk::MODE_EAGER, p, stream);
}

double dl_predict_token_us(const dl_config *cfg, double read_gbps, double copy_gbps) {
    const double read[3] = {read_gbps, read_gbps, read_gbps};
    const double copy[3] = {copy_gbps, copy_gbps, copy_gbps};
    return dl_predict_token_us_bounds(cfg, read, copy);
}

double dl_predict_token_us_bounds(const dl_config *cfg, const double read_gbps[3], const double copy_gbps[3]) {
    size_t heads = 0;
    if (!read_gbps || !copy_gbps) return -1.0;
    if (check_config(cfg, &heads) != DL_OK) return -1.0;
    // the rates of the kernels this capacity runs (built for 8, 16 or 32 entries)
    const int fam = cfg->C <= 8 ? 0 : (cfg->C <= 16 ? 1 : 2);
    double read = read_gbps[fam], copy = copy_gbps[fam];
    // defaults: the stream ceilings of the kernels' own access pattern on
    // MI355X, measured in sequence with a cold Infinity Cache (bench.py's
    // `ceilings`, GDN B=128 H=32 d=128): a read of every head, an in-place copy
    if (read <= 0) read = 6760.0;
    if (copy <= 0) copy = 5580.0;
    const HeadBytes b = head_bytes(cfg);
    const double n = (double)heads;
    const int C = cfg->C;
    double us = 0.0;
    for (int L = 0; L + 1 < C; ++L)  // appends
        us += (n * (b.base + b.token + b.out + (L + 1) * b.entry) + b.shared) / (read * 1e3);
    us += (n * (2.0 * b.base + b.token + b.out + (C - 1) * b.entry) + b.shared) / (copy * 1e3);
    return us / C;
}

int dl_choose_capacity(const dl_config *cfg, int max_c, double read_gbps, double copy_gbps) {
    const double read[3] = {read_gbps, read_gbps, read_gbps};
    const double copy[3] = {copy_gbps, copy_gbps, copy_gbps};
    return dl_choose_capacity_bounds(cfg, max_c, read, copy);
}

int dl_choose_capacity_bounds(const dl_config *cfg, int max_c, const double read_gbps[3], const double copy_gbps[3]) {
    size_t heads = 0;
    dl_status st = check_config(cfg, &heads);
    if (st != DL_OK) return st;
    if (max_c < 1 || max_c > DL_MAX_CAPACITY) return fail(DL_ERR_SHAPE, "max_c must lie in [1, 32]");
    if (!read_gbps || !copy_gbps) return fail(DL_ERR_ARG, "read_gbps and copy_gbps must point to three rates each");
    dl_config c = *cfg;
    int best = 1;
    double best_us = 0.0;
    for (int C = 1; C <= max_c; ++C) {
        c.C = C;
        const double us = dl_predict_token_us_bounds(&c, read_gbps, copy_gbps);
        if (C == 1 || us < best_us) {
            best = C;
            best_us = us;
        }
    }
    return best;
}

void dl_state_destroy(dl_state *h) { delete h; }

const char *dl_status_string(int status) {
    switch (status) {
        case DL_OK: return "ok";
        case DL_ERR_ARG: return "invalid argument";
        case DL_ERR_SHAPE: return "invalid shape";
        case DL_ERR_UNSUPPORTED: return "unsupported configuration";
        case DL_ERR_HIP: return "HIP runtime error";
        case DL_ERR_WORKSPACE: return "workspace too small";
        default: return "unknown status";
    }
}

const char *dl_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
