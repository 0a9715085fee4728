/*
 * deltalog.h -- C ABI of the DeltaLog recurrent-state decode library for
 * AMD Instinct MI355X (gfx950).
 *
 * Method.  "DeltaLog: Deferred Materialization of Recurrent States for Linear
 * Attention Decoding" (Lin, Sun, Sun).  Each attention head of a linear-
 * attention layer keeps a dense recurrent state of shape [dk, dv]; eager
 * decoding rewrites the whole [B, H, dk, dv] tensor after every token
 * although a token only contributes O(dk + dv) numbers (gist.science summary,
 * section "Problema").  DeltaLog keeps instead a dense base state plus a
 * bounded log of compact update factors and their log-decay metadata
 * (section "Meccanismo Core: Base + Log"); it appends to the log while its
 * length L is below the capacity C and folds the log into the base when L
 * reaches C (signal-papers summary, caption of Fig. 4), so the logical state
 * always equals the eager one (DeltaLog abstract).  Operators: GDN, KDA and
 * RWKV6 (gist.science summary, section "Operatori").
 *
 * Logical state after L logged tokens (exact algebra, per head):
 *     S = diag(e^{g_L}) Sbar + sum_{i<L} diag(e^{g_L - g_i}) k_i x_i^T
 * with g_i the cumulative log-decay since the last fold, k_i the token's key
 * and x_i its value-side factor: u_i = beta_i (v_i - (decayed state)^T k_i)
 * for the delta rules (GDN, KDA), v_i for RWKV6.
 *
 * Conventions for every entry point:
 *  - Device pointers are HIP device (or managed) memory owned by the caller.
 *    The library never allocates, frees or synchronises device memory; it
 *    enqueues kernels on the caller's stream and returns.  Inputs may be
 *    reused or freed once the stream has passed the call.
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *  - State buffers (base, dst, state) and the workspace must be 16-byte
 *    aligned.  The kernels read q and k four channels at a time, so those
 *    must be aligned to four elements (8 bytes in bf16, 16 in f32), and the
 *    per-channel decay (KDA, RWKV6) and the bonus as float4, so those must
 *    be 16-byte aligned; every other device pointer must be aligned to its
 *    element size.
 *  - Aliasing (checked on byte ranges, DL_ERR_ARG): the base and the
 *    workspace are disjoint; a token's out overlaps none of its inputs; no
 *    input or output of a token overlaps the base, the workspace or the
 *    prep buffer of the handle (every launch may write them); the tokens of
 *    one dl_decode_tokens call write disjoint outputs that overlap no
 *    token's inputs; a materialise dst overlaps none of the base, the
 *    workspace and the prep buffer; the prep buffer overlaps neither the
 *    base nor the workspace; for dl_eager_step no input or output overlaps
 *    the state.
 *  - Return values are dl_status codes: DL_OK (0) or a negative error.  Every
 *    argument is checked before anything is enqueued, so on any error but
 *    DL_ERR_HIP nothing was enqueued and the handle is unchanged;
 *    dl_last_error() then returns a message naming the argument at fault.
 *    DL_ERR_HIP means the runtime refused a launch; a call that issues
 *    several launches may have enqueued the earlier ones, so the handle and
 *    the device state are then undefined (re-create the handle from a saved
 *    state).
 *    Faults inside a kernel (e.g. a freed buffer) surface asynchronously at
 *    the caller's next synchronisation, not through these codes.
 *  - A handle is not thread-safe; distinct handles are independent.
 *
 * Tensor layouts (row-major, last index contiguous; N = B*H heads, head
 * n = b*H + h):
 *    state / base  [B, H, dk, dv] fp32
 *    q (r), k      [B, H, dk]     input dtype (fp32 or bf16)
 *    v             [B, H, dv]     input dtype
 *    beta          [B, H]         fp32   (GDN, KDA)
 *    decay         GDN: alpha [B, H]; KDA: a [B, H, dk]; RWKV6: w [B, H, dk];
 *                  fp32, every value in (0, 1] (0 is undefined behaviour)
 *    bonus         [H, dk]        fp32   (RWKV6 per-head bonus u)
 *    out           [B, H, dv]     fp32
 * Supported shapes: dk == dv in {32, 64, 128}; 1 <= C <= DL_MAX_CAPACITY;
 * B*H <= DL_MAX_HEADS (a launch holds at most 2^32 work-items and the widest
 * kernel runs 512 per head; at dk = 128 that bound is a 550 GB state).
 */
#ifndef DELTALOG_H
#define DELTALOG_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DL_MAX_CAPACITY 32
#define DL_MAX_TOKENS 8
#define DL_MAX_HEADS (1 << 23)

typedef enum { DL_GDN = 0, DL_KDA = 1, DL_RWKV6 = 2 } dl_op;
typedef enum { DL_F32 = 0, DL_BF16 = 1 } dl_dtype;

typedef enum {
    DL_OK = 0,
    DL_ERR_ARG = -1,          /* null or misaligned pointer, bad enum value, aliasing */
    DL_ERR_SHAPE = -2,        /* non-positive or overflowing sizes, C out of [1, 32] */
    DL_ERR_UNSUPPORTED = -3,  /* valid but not built: dk != dv or dk not in {32,64,128} */
    DL_ERR_HIP = -4,          /* the HIP runtime refused a launch */
    DL_ERR_WORKSPACE = -5     /* workspace smaller than dl_workspace_bytes() */
} dl_status;

/* Shape of one layer's recurrent state.  op: dl_op; in_dtype: dl_dtype of
 * q (or r), k and v; B slots of H heads; key width dk, value width dv; log
 * capacity C (the merge interval: tokens per fold). */
typedef struct {
    int op;
    int in_dtype;
    int B, H, dk, dv;
    int C;
} dl_config;

/* Inputs and output of one decode token for all B*H heads.  beta must be
 * NULL for RWKV6 and non-NULL otherwise; bonus must be non-NULL for RWKV6
 * and NULL otherwise. */
typedef struct {
    const void *q;      /* q_t (GDN, KDA) or r_t (RWKV6)  [B,H,dk] in_dtype */
    const void *k;      /* k_t                            [B,H,dk] in_dtype */
    const void *v;      /* v_t                            [B,H,dv] in_dtype */
    const float *beta;  /* beta_t [B,H] */
    const float *decay; /* alpha_t [B,H] (GDN) or a_t / w_t [B,H,dk] */
    const float *bonus; /* RWKV6 bonus u [H,dk] */
    float *out;         /* o_t [B,H,dv] fp32, written */
} dl_step_args;

typedef struct dl_state dl_state; /* opaque, host memory only */

/* Bytes of device workspace holding the bounded update log of capacity C
 * for cfg: per head, up to C compact update factors and their log-decay
 * metadata (gist.science summary, "Meccanismo Core: Base + Log": the
 * bounded update log beside the dense base), i.e. O(C (dk + dv)) numbers
 * against the dk * dv of the state ("Problema": a token contributes
 * O(dk + dv)).  Value factors, key copies and cumulative log-decays; see
 * dl_workspace_layout.  Returns 0 for an invalid or unsupported cfg. */
size_t dl_workspace_bytes(const dl_config *cfg);

/* Byte offsets inside the workspace of its three arrays, for inspection:
 *   offsets[0]: value factors X [N][C][dv]  fp32 (GDN, KDA: u_i) or in_dtype (RWKV6: v_i)
 *   offsets[1]: key copies    K [N][C][dk]  in_dtype (exact copies of k_i)
 *   offsets[2]: log-decays    G [N][C] (GDN) or [N][C][dk] fp32, cumulative
 *               base-2 log of the decay since the last fold, through token i
 * Entry i of head n is valid for i < dl_log_length().  Returns DL_OK or an
 * error for an invalid cfg or a NULL offsets. */
dl_status dl_workspace_layout(const dl_config *cfg, size_t offsets[3]);

/* Create a handle over a caller-owned base state and workspace: the dense
 * base, the history up to the last merge, and the bounded log of recent
 * compact factors beside it (gist.science summary, "Meccanismo Core: Base +
 * Log"); the state of each head is a dk x dv matrix and the layer's a
 * [B,H,dk,dv] tensor ("Problema").
 *   base       [B,H,dk,dv] fp32 device memory holding the current dense state
 *              (the initial state, or a state saved after a fold: resume)
 *   workspace  device memory of at least dl_workspace_bytes(cfg) bytes,
 *              disjoint from the base
 * The log starts empty (L = 0); no device work is done.  *out receives the
 * handle (NULL on error).  The buffers must outlive the handle. */
dl_status dl_state_init(dl_state **out, const dl_config *cfg, float *base,
                        void *workspace, size_t workspace_bytes);

/* Decode one token for every head (the append step; the signal-papers
 * summary, Fig. 4, and gist.science "Fase di Append" / "Fase di Merge").
 * Writes out = o_t.  If L + 1 < C it appends the token's compact factors
 * and leaves the base untouched (L becomes L + 1).  If L + 1 == C the same
 * launch also folds all C factors into the base with one read and one write
 * of the base (L becomes 0).  With C == 1 every step is the eager update. */
dl_status dl_decode_step(dl_state *h, const dl_step_args *args, void *stream);

/* Decode K consecutive tokens of every head (1 <= K <= DL_MAX_TOKENS):
 * args[0..K-1] are the tokens in order, each as for dl_decode_step, and
 * args[t].out receives o_t.  The tokens share one read of the base in one
 * launch: the log grows by the call's tokens, and when it fills (at any
 * token of the call) the kernel folds it into the base and the call's later
 * tokens start the new log (as many folds as the call fills the log, more
 * than one only when K > C).  K == 1 is one dl_decode_step.  The result
 * equals K calls of dl_decode_step up to rounding.  The RWKV6 bonus is a
 * per-head parameter, so every token must carry the same bonus pointer
 * (DL_ERR_ARG otherwise).  On a per-slot handle each slot folds at its own
 * token, in the same single launch; inactive slots are untouched.  This is
 * the multi-token neighbour of single-token decode (drafted tokens to
 * verify, short continuations); it follows from the same base-plus-log
 * representation (gist.science summary, "Meccanismo Core: Base + Log"). */
dl_status dl_decode_tokens(dl_state *h, const dl_step_args *args, int K, void *stream);

/* Fold the current log into the base now, L becomes 0: the merge phase
 * (gist.science summary, "Fase di Merge": the accumulated logical state,
 * base plus replayed log entries, is written back into the dense base and
 * the log is reset), taken before the log is full.  dl_decode_step runs the
 * same fold by itself when a token fills the log.  Output-neutral: later
 * outputs are unchanged.  A no-op when L == 0. */
dl_status dl_merge(dl_state *h, void *stream);

/* Write the logical dense state [B,H,dk,dv] fp32 into dst without changing
 * the handle, the base or the log: the state eager decoding would hold
 * after the same tokens (the signal-papers summary, Fig. 4: the logical
 * state that a merge materialises into the base; Fig. 12 (b): the
 * materialised recurrent state whose relative error the pages report).
 * dst must overlap none of the base, the workspace and the prep buffer
 * (DL_ERR_ARG). */
dl_status dl_materialize(const dl_state *h, float *dst, void *stream);

/* Current log length L in [0, C) of a lockstep handle -- the L of the
 * signal-papers summary, Fig. 4 (append while L < C, materialise when
 * L = C) -- or -1 for a NULL or a per-slot handle (see dl_slot_log_length). */
int dl_log_length(const dl_state *h);

/* Split replay (the pages' staged kernel: gist.science summary, "Implementazione
 * del Kernel" -- a shared ReplayPrep stage computes the replay coefficients
 * once per slot-head, then parallel AppendDecode stages run the value tiles;
 * ablated against graph replay in the signal-papers summary, Fig. 9).
 *
 * By default every value-tile workgroup of an append recomputes the key-side
 * preparation itself while its base tile is in flight (fused).  With a prep
 * buffer set, each append instead runs two launches: one workgroup per head
 * computes the scaled key and query (receptance), the replay coefficients
 * and the token's scalar term into a per-head record and appends the key
 * side of the entry; then the tile workgroups read that record.  The fold
 * step (L + 1 == C) and dl_decode_tokens keep their fused form.  Results
 * equal the fused path up to fp32 rounding.
 *
 * dl_prep_bytes: bytes of that buffer for cfg (N records of 2*dk + 2*M + 4
 * fp32, M the smallest of 8, 16 and 32 not below C); 0 for an invalid cfg.
 * dl_set_split_replay: prep = device memory of at least dl_prep_bytes bytes,
 * 16-byte aligned, owned by the caller and outliving its use (it holds no
 * state between steps), or NULL to return to the fused form.  Lockstep
 * handles only (DL_ERR_UNSUPPORTED on a per-slot handle); DL_ERR_WORKSPACE
 * for a short buffer.  Host-only: enqueues nothing. */
size_t dl_prep_bytes(const dl_config *cfg);
dl_status dl_set_split_replay(dl_state *h, void *prep, size_t prep_bytes);

/* The decode step for callers that cannot allocate device memory (code
 * under graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Does what dl_decode_step does in the split-replay form (see
 * dl_set_split_replay), with the per-head prep records held in a static
 * device array of the library -- DL_NOALLOC_PREP_BYTES (8 MiB) on each GPU
 * it runs on, for the life of the process -- instead of a caller buffer.
 * It allocates nothing and calls no allocating routine; the caller still
 * passes the inputs and the output.  The first call on a device looks up
 * that device's copy of the array (hipGetSymbolAddress).  Every call writes
 * the records it reads and nothing carries from one call to the next; all
 * calls on one GPU share the array, so calls that may run at the same time
 * on one GPU (different streams, different threads) race.  Lockstep handles
 * only (DL_ERR_UNSUPPORTED on a per-slot handle); DL_ERR_WORKSPACE when
 * dl_prep_bytes(cfg) exceeds DL_NOALLOC_PREP_BYTES (at dk = 128 and C <= 8,
 * for instance, up to 7598 heads); DL_ERR_HIP if the array's address cannot
 * be found.  Otherwise as dl_decode_step. */
#define DL_NOALLOC_PREP_BYTES (8u << 20)
dl_status dl_decode_step_noalloc(dl_state *h, const dl_step_args *args, void *stream);

/* Graph replay of one merge cycle (the pages time their kernels under graph
 * replay: signal-papers summary, Fig. 9).
 *
 * dl_graph_capture_cycle records the C decode steps of one whole cycle --
 * args[0..C-1], each as for dl_decode_step, in the handle's current mode
 * (fused or split replay) -- into a HIP graph, without running them.  The
 * log must be empty (dl_log_length() == 0, else DL_ERR_ARG); a whole cycle
 * leaves it empty again, so the graph can be replayed any number of times.
 * The graph keeps every pointer it was recorded with (inputs, outputs, base,
 * workspace, prep): the caller refills the same input buffers before each
 * replay.  Lockstep handles only (DL_ERR_UNSUPPORTED otherwise).  It creates
 * and destroys a private capture stream and instantiates the graph, so
 * unlike the other calls it asks the HIP runtime for resources.  *out
 * receives the graph (NULL on error).
 *
 * dl_graph_launch enqueues one replay (C tokens) on `stream`; DL_ERR_ARG if
 * the handle's log is not empty (a dl_decode_step since the last replay
 * that did not complete a cycle).  dl_graph_destroy releases the graph (NULL
 * is allowed); destroy it before its handle. */
typedef struct dl_graph dl_graph; /* opaque, host memory only */
dl_status dl_graph_capture_cycle(dl_graph **out, dl_state *h, const dl_step_args *args);
dl_status dl_graph_launch(dl_graph *g, void *stream);
void dl_graph_destroy(dl_graph *g);

/* Per-slot logs (continuous batching).  The pages prepare replay
 * coefficients per slot-head (gist.science summary, "Implementazione del
 * Kernel") and serve many concurrent requests; here each of the B slots has
 * its own log length, so requests may join and leave at any token.
 *
 * dl_state_init_slots is dl_state_init for such a handle, with every slot
 * inactive; it enqueues one small kernel on `stream` (the workspace holds the
 * per-slot bookkeeping).  On a per-slot handle:
 *  - dl_decode_step decodes only active slots: a slot whose token fills its
 *    log also folds it into its base in the same step; inactive slots' inputs
 *    are ignored and their outputs left untouched;
 *  - dl_merge folds every active slot's log (an early merge);
 *  - dl_materialize writes the logical state of active slots only.
 * Returns as for the lockstep calls. */
dl_status dl_state_init_slots(dl_state **out, const dl_config *cfg, float *base, void *workspace,
                              size_t workspace_bytes, void *stream);

/* Start a request in `slot` with an empty log: from the next decode step the
 * slot's base block [H,dk,dv] is its dense state (the caller writes it before
 * that step, in stream order).  DL_ERR_ARG for a bad slot or a lockstep
 * handle. */
dl_status dl_slot_activate(dl_state *h, int slot, void *stream);

/* Stop decoding `slot` (its base and log stay as they are until the slot is
 * activated again).  DL_ERR_ARG for a bad slot or a lockstep handle. */
dl_status dl_slot_deactivate(dl_state *h, int slot, void *stream);

/* Log length of an active slot in [0, C), or -1 for an inactive or invalid
 * slot or a lockstep handle. */
int dl_slot_log_length(const dl_state *h, int slot);

/* Write the logical state of one slot, [H,dk,dv] fp32, into dst (for
 * example to save a request that leaves); nothing else changes.  Lockstep
 * and per-slot handles; one launch over the slot's H heads only.
 * DL_ERR_ARG for a bad slot, an inactive
 * slot of a per-slot handle, or a dst that overlaps the base, the workspace
 * or the prep buffer. */
dl_status dl_materialize_slot(const dl_state *h, int slot, float *dst, void *stream);

/* Fold one active slot's log into its base block now (an early merge of that
 * slot alone, output-neutral); the slot's log becomes empty.  Per-slot
 * handles only (DL_ERR_ARG otherwise, or for a bad or inactive slot); a
 * no-op when the slot's log is empty. */
dl_status dl_slot_merge(dl_state *h, int slot, void *stream);

/* The eager dense update for comparison (gist.science "Problema"): reads
 * the [B,H,dk,dv] fp32 state, writes out = o_t and the updated state in
 * place.  Uses only cfg's op, in_dtype, B, H, dk, dv (C is ignored). */
dl_status dl_eager_step(const dl_config *cfg, float *state, const dl_step_args *args,
                        void *stream);

/* Modelled time per decode token (microseconds, amortised over one merge
 * cycle of cfg->C tokens) from the per-launch traffic: each append moves the
 * base, the token and the L entries it replays plus the entry it writes, at
 * read_gbps; the token that fills the log moves the base twice, at copy_gbps
 * (gist.science summary, "Modello di Traffico": appends of compact factors,
 * one amortised dense write per interval, replay of the log).  Bandwidths
 * <= 0 select the stream ceilings measured on MI355X at the kernels' own
 * access pattern (include/deltalog_probe.h), in sequence with a cold
 * Infinity Cache: 6760 GB/s for a read of every head, 5580 GB/s for an
 * in-place copy.  The kernels run at 85-96 % of those ceilings, so the
 * prediction is a lower bound, 5-15 % under the measured time.  Host-only.
 * Returns a negative value for an invalid cfg. */
double dl_predict_token_us(const dl_config *cfg, double read_gbps, double copy_gbps);

/* The capacity C in [1, max_c] (max_c <= DL_MAX_CAPACITY) with the smallest
 * dl_predict_token_us for cfg's other fields -- the interval that balances
 * replay traffic against dense-write savings (gist.science, "Modello di
 * Traffico").  Host-only.  Returns the C, or a negative dl_status for an
 * invalid cfg or max_c. */
int dl_choose_capacity(const dl_config *cfg, int max_c, double read_gbps, double copy_gbps);

/* The same model with a rate per kernel family.  A capacity runs the
 * kernels built for a log of 8 (C <= 8), 16 (C <= 16) or 32 entries; the
 * larger bounds hold more key-side registers per lane, which costs some
 * shapes (the 64 x 64 heads) more than the bytes show.  read_gbps[f] and
 * copy_gbps[f] are the rates the family f = 0, 1, 2 (8, 16, 32 entries)
 * reaches for its appends and its fold -- for instance the stream ceilings
 * scaled by the measured over modelled time of one capacity of that family
 * (bench.py --capacity-study).  A rate <= 0 selects the default ceiling as
 * above.  Both arrays hold three values and must not be NULL
 * (dl_predict_token_us_bounds returns a negative value,
 * dl_choose_capacity_bounds DL_ERR_ARG).  dl_predict_token_us and
 * dl_choose_capacity are these with one rate for all three families.
 * Host-only. */
double dl_predict_token_us_bounds(const dl_config *cfg, const double read_gbps[3], const double copy_gbps[3]);
int dl_choose_capacity_bounds(const dl_config *cfg, int max_c, const double read_gbps[3], const double copy_gbps[3]);

/* Release a handle (NULL is allowed).  Device buffers are not touched. */
void dl_state_destroy(dl_state *h);

/* Static description of a status code; never NULL. */
const char *dl_status_string(int status);

/* Message describing the last error returned on the calling thread
 * ("" if none).  Valid until the thread's next call into the library. */
const char *dl_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DELTALOG_H */
