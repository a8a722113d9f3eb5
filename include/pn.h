/*
 * pn.h - C ABI of the MI355X one-token decode library.
 *
 * The library computes the architecture forward step of a Llama-family
 * transformer, forward(model, token, state) -> logits, one token per sequence
 * ("Core Engine API", section "pn_model struct": the forward function pointer
 * takes a model, one token and a state and returns the logits), for one
 * sequence or for a batch of independent sequences that each advance one token
 * at their own position ("Engine Architecture", section "Continuous-Batch VLM
 * Decoder": one M=B decode over all slots, each slot finishing on its own).
 *
 * Conventions shared by every entry point:
 *  - Plain C types only.  Pointers named *_dev are device pointers; every
 *    other pointer is host memory.  `stream` is a hipStream_t passed as void*
 *    (NULL = the default stream).
 *  - The caller owns all device memory.  The library owns only the host
 *    handles (pn_model, pn_state) and allocates no device memory, neither at
 *    create time nor per token: a model and each state live in buffers the
 *    caller passes in, sized by pn_model_bytes / pn_state_bytes.  This mirrors
 *    the pages' pre-sized scratch arena with no allocation per token ("Core
 *    Engine API", section "Scratch (arena) estimation"; "Engine
 *    Architecture", section "Memory Model").
 *  - Calls that take a stream only enqueue work on it and return; completion
 *    is observed through the stream.  This is the device form of the pages'
 *    non-blocking begin/poll step ("Core Engine API", section "Async
 *    forward-step seam").  Calls that use one model must be ordered on one
 *    stream (the pages keep one step in flight per model).  A state must not
 *    be used by two calls at once.
 *  - Return value: 0 on success, else a negative PN_E* code; every failure
 *    sets a message readable through pn_last_error() (thread-local).  All
 *    argument checks happen on the host before anything is enqueued, so a
 *    failed call leaves the device untouched.  One exception: a multi-chunk
 *    pn_prefill into a pooled state whose pool runs out in a later chunk
 *    returns PN_ERANGE after the earlier chunks were enqueued (their tokens
 *    are in the cache and pos counts them; see pn_prefill).
 */
#ifndef PN_H
#define PN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    PN_OK = 0,
    PN_EINVAL = -1,       /* bad config, NULL pointer, duplicate state, bad token/layer index */
    PN_ERANGE = -2,       /* buffer too small, position past the state's capacity */
    PN_EUNSUPPORTED = -3, /* valid but unsupported shape or dtype combination */
    PN_EHIP = -4          /* HIP runtime failure */
};

typedef enum { PN_F32 = 0, PN_BF16 = 1, PN_I8 = 2, PN_Q8_0 = 3, PN_Q4_0 = 4 } pn_dtype;

/* Model dimensions and storage types.  Field names and defaults follow the
 * pages' config keys ("Engine Architecture", section "Config Parsing"):
 * n_kv_head defaults to n_head, n_ctx to 2048, rope_theta to 10000,
 * rms_norm_eps to 1e-5, sliding_window to 0 (off); here n_kv_head 0 stands
 * for n_head.  n_expert > 0 selects the
 * top-k MoE FFN ("Engine Architecture", section "Architecture Detection":
 * Mixtral is llama with an expert count > 0).
 *
 *  w_dtype   matrices: PN_F32, PN_BF16, PN_I8 (symmetric int8 with one fp32
 *            scale per output row), or a GGUF-style block quantisation,
 *            dequantised inside the mat-vec ("Engine Architecture", section
 *            "Weight Loading Modes"): each row is K/32 blocks, PN_Q8_0 blocks
 *            of 34 bytes (an fp16 scale d, then 32 int8 codes q; weight d*q),
 *            PN_Q4_0 blocks of 18 bytes (an fp16 scale d, then 16 bytes whose
 *            byte i holds code i in its low nibble and code i+16 in its high
 *            one; weight d*(code-8)).  Block formats need act_dtype PN_BF16
 *            and n_embd, n_ff multiples of 32.  The token embedding
 *            and the MoE router are fp32 when w_dtype is PN_F32 and bf16
 *            otherwise; norm gains are fp32.
 *  kv_dtype  cached K and V: PN_F32, PN_BF16, or PN_Q4_0 (k is cached after
 *            RoPE).  A Q4 cache (the pages' serve layer counts a Q4-quantised
 *            KV cache: "Serve Layer Architecture", section "Environment
 *            Variables") keeps each head vector of k and v as 32-dim blocks of
 *            an fp16 scale d and 4-bit codes, value d*(code-8), set when the
 *            token is appended: m = the element of largest magnitude (the first
 *            on ties), d = fp16(m/-8), code = clamp(rint(x/d)+8, 0, 15), in
 *            fp32; 9*head_dim/16 bytes per cached vector.  Not with rope_neox.
 *  act_dtype type that every mat-vec input (normed x, attention output, FFN
 *            hidden, final normed x) is rounded to: PN_F32 or PN_BF16.  The
 *            residual stream, q, softmax and all accumulators stay fp32.
 *            PN_I8 weights need act_dtype PN_BF16.  With int8 and block
 *            (Q8_0, Q4_0) weights the bf16 activations enter the f16 matrix
 *            cores as f16, exactly for magnitudes 2^-17 .. 65504: larger ones
 *            become inf (the step's logits then show it) and smaller ones keep
 *            fewer bits (below 2^-25 they are 0).  Normed inputs stay far inside
 *            (|x| <= sqrt(n_embd) * max|gain|); the FFN hidden values do for any
 *            weights that keep |silu(gate) * up| under 65504.
 *  max_batch largest n accepted by pn_forward_batch (1..16; with act_dtype
 *            PN_F32 and bf16/int8 weights, 1..5).
 *  rope_neox, qkv_bias  the variants that share the Llama forward through
 *            config flags ("Engine Architecture", section "Architecture
 *            Detection"): attention biases (Qwen2), added to q, k and v before
 *            RoPE; the NeoX RoPE of Phi-3, which rotates (i, i + d/2) instead
 *            of (2i, 2i+1) with the same angles.  0 (default) or 1.  A fused
 *            QKV or gate+up checkpoint needs no flag: pass pointers into it
 *            (wk = wq + H*d rows, w_up = w_gate + F rows).
 *  prefill_chunk  rows per pn_prefill chunk on the wide path, 1..256, or 0
 *            (chunks of max_batch through the decode kernels).  The wide path
 *            takes each chunk through every projection as one matrix product
 *            on the matrix cores, so a weight is read once per chunk (with
 *            experts: each expert's once, over the rows routed to it); it needs
 *            w_dtype PN_BF16, PN_I8, PN_Q8_0 or PN_Q4_0 and kv_dtype PN_F32 or
 *            PN_BF16 (PN_EUNSUPPORTED otherwise), and adds its row buffers to
 *            pn_model_bytes. */
typedef struct pn_config {
    int32_t n_layer, n_embd, n_head, n_kv_head, head_dim, n_ff, n_vocab;
    int32_t n_ctx;          /* default state capacity when pn_state_* is given max_ctx 0 */
    int32_t n_expert;       /* 0 = dense SwiGLU FFN */
    int32_t n_expert_used;  /* top-k (1..8) when n_expert > 0 */
    int32_t sliding_window; /* 0 = off; else the step at pos attends to pos-W+1..pos */
    int32_t max_batch;
    float rope_theta, rms_norm_eps;
    int32_t w_dtype, kv_dtype, act_dtype; /* pn_dtype values */
    int32_t rope_neox; /* 1: RoPE rotates the half-split pairs (i, i + head_dim/2) */
    int32_t qkv_bias;  /* 1: the q, k, v projections add fp32 biases (b_q, b_k, b_v) */
    int32_t prefill_chunk; /* 0: pn_prefill goes in chunks of max_batch; 1..256: in chunks
                              of this many rows through the wide prefill path (below) */
} pn_config;

/* Device pointers of one layer's weights, logical row-major [out][in] (PN_Q8_0:
 * each row its K/32 blocks).  The expert matrices are stacked: X = max(1,
 * n_expert) blocks of gate/up [F][E] and down [E][F].  Scales (s_*) are required iff w_dtype == PN_I8 (one fp32
 * per output row, stacked like the matrices), else ignored. */
typedef struct pn_layer_weights {
    const float *attn_norm, *ffn_norm;   /* [E] */
    const void *wq, *wk, *wv, *wo;       /* [H*d][E], [Hk*d][E], [Hk*d][E], [E][H*d] */
    const void *w_gate, *w_up, *w_down;  /* [X][F][E], [X][F][E], [X][E][F] */
    const void *w_router;                /* [n_expert][E]; NULL for dense */
    const float *s_q, *s_k, *s_v, *s_o, *s_gate, *s_up, *s_down;
    const float *b_q, *b_k, *b_v;        /* [H*d], [Hk*d], [Hk*d]; required iff qkv_bias */
} pn_layer_weights;

typedef struct pn_weights {
    const void *tok_embd;  /* [V][E] */
    const float *out_norm; /* [E] */
    const void *w_out;     /* [V][E] LM head (untied) */
    const float *s_out;    /* [V] iff PN_I8 */
    const pn_layer_weights *layers; /* host array of n_layer entries */
} pn_weights;

typedef struct pn_model pn_model;
typedef struct pn_state pn_state;
typedef struct pn_pool pn_pool;

/* Fill *cfg with the pages' defaults; dimensions are left 0. */
void pn_config_default(pn_config *cfg);

/* Validate a config without touching the device.  0 or PN_EINVAL / PN_EUNSUPPORTED. */
int pn_config_check(const pn_config *cfg);

/* Bytes of device memory a model of this config needs (packed weights plus
 * per-model scratch for max_batch sequences); 0 if the config is invalid. */
size_t pn_model_bytes(const pn_config *cfg);

/* Build a model in the caller's device buffer `dev_buf` (>= pn_model_bytes,
 * 256-byte aligned): the weights are re-laid into the library's tiled format
 * by kernels enqueued on `stream`.  The source weights may be freed once that
 * stream work has completed.  On success *out holds a host handle. */
int pn_model_create(const pn_config *cfg, const pn_weights *w, void *dev_buf, size_t bytes,
                    void *stream, pn_model **out);

/* The same in steps, for models whose source weights do not fit on the device
 * next to the packed copy: pn_model_init lays the model out in dev_buf without
 * touching the device; pn_model_load_globals packs the embedding, final norm
 * and LM head; pn_model_load_layer packs one layer.  The model may be used
 * once the globals and every layer have been loaded and that stream work has
 * completed; each source buffer may be freed once its call's work has. */
int pn_model_init(const pn_config *cfg, void *dev_buf, size_t bytes, pn_model **out);
int pn_model_load_globals(pn_model *m, const void *tok_embd, const float *out_norm, const void *w_out,
                          const float *s_out, void *stream);
int pn_model_load_layer(pn_model *m, int32_t layer, const pn_layer_weights *w, void *stream);

/* Release the host handle (the device buffer stays the caller's). */
void pn_model_free(pn_model *m);

/* Bytes of device memory one state of capacity max_ctx positions needs (paged
 * K/V cache for every layer, page table, attention split scratch); 0 if invalid
 * (max_ctx < 1, or one layer's K pool would reach 2 GiB: about a million
 * positions of 8 bf16 KV heads of 128 dims). */
size_t pn_state_bytes(const pn_model *m, int32_t max_ctx);

/* Create a state (pos = 0, K/V zeroed, identity page table) in `dev_buf`
 * (>= pn_state_bytes, 256-byte aligned).  Zeroing is enqueued on `stream`. */
int pn_state_new(pn_model *m, int32_t max_ctx, void *dev_buf, size_t bytes, void *stream,
                 pn_state **out);

/* Zero every cached K and V and set pos = 0 ("Core Engine API", section
 * "State lifecycle": reset zeros the kv tensors and resets pos).  A pooled
 * state gives its pages back instead (a page is zeroed when next taken). */
int pn_state_reset(pn_state *s, void *stream);

/* Write cached K and V of positions pos0..pos0+n-1 of one layer from device
 * arrays k_dev, v_dev laid out [n][n_kv_head][head_dim] in kv_dtype (k after
 * RoPE; fp32 for a PN_Q4_0 cache, quantised as an append quantises).  Used to resume or to prefill a cache.  Does not change pos.  A
 * pooled state takes pages for those positions (PN_ERANGE if the pool runs
 * out or if pos0 lies below pages that went back to the pool). */
int pn_state_set_kv(pn_state *s, int32_t layer, int32_t pos0, int32_t n, const void *k_dev,
                    const void *v_dev, void *stream);

/* Map logical page i (positions i*page_size .. i*page_size+page_size-1) to
 * physical page pages[i] of the state's own pool.  `pages` is a host array
 * holding a permutation of 0..n-1, n = pn_state_pages(s).  Cached contents are
 * not moved: set the table before writing K/V. */
int pn_state_set_page_table(pn_state *s, const int32_t *pages, int32_t n, void *stream);
int32_t pn_state_pages(const pn_state *s);
int32_t pn_page_size(void);

/* Number of positions already cached (the position the next step writes).
 * Moving pos leaves the cache as it is.  On a pooled state, the positions the
 * next step reads get pages (zeroed, enqueued on `stream`) where they have
 * none; PN_ERANGE if the pool runs out, or if that window reaches positions
 * whose pages went back to the pool (see pn_state_new_pooled). */
int pn_state_set_pos(pn_state *s, int32_t pos, void *stream);
int32_t pn_state_pos(const pn_state *s);
int32_t pn_state_max_ctx(const pn_state *s);

/* Read (and clear) the state's sticky device error flags; synchronizes
 * `stream`.  Bit 0: a token id outside [0, n_vocab) was fed (row 0 was used
 * instead).  Bit 1: a NaN logit was seen by the argmax. */
int pn_state_check(pn_state *s, void *stream, int32_t *flags_out);

void pn_state_free(pn_state *s);

/* ---- shared page pool ------------------------------------------------------
 *
 * States of a continuously batched decode (sequences join and leave the batch
 * between steps: "Serve Layer Architecture", section "Batched Decode", "D2 -
 * continuous batching"; "Engine Architecture", section "Continuous-Batch VLM
 * Decoder": a finished sequence's state is recycled for the next) can draw
 * their K/V pages from one pool instead of each reserving max_ctx positions.
 * A pooled state takes a page (page_size positions of every layer's K and V)
 * when a step, a prefill, pn_state_set_kv or pn_state_set_pos first needs one,
 * zeroes it, and gives every page back on pn_state_reset and pn_state_free
 * (the pages' reset: "Core Engine API", section "State lifecycle").  With a
 * sliding window, the pages wholly before the window of the state's next step
 * go back to the pool after each step, so a windowed sequence holds at most
 * about window / page_size + 2 pages however long it runs.  Results are those
 * of private states, bit for bit.  The pool's page bookkeeping is host-side:
 * all states of a pool must be driven from one thread and on one stream (a
 * page returned by one state may be zeroed for another by the next call).
 * When the pool runs out, the step, prefill chunk, set_kv or set_pos fails
 * with PN_ERANGE before anything is enqueued for it and every state is as
 * before that call (a prefill keeps the chunks it has already done: pos
 * tells how far it got). */

/* Bytes of device memory a pool of n_pages pages needs; 0 if n_pages < 1 or
 * one layer's K pages would reach 2 GiB. */
size_t pn_pool_bytes(const pn_model *m, int32_t n_pages);

/* Create a pool of n_pages pages in `dev_buf` (>= pn_pool_bytes, 256-byte
 * aligned).  Nothing is enqueued: pages are zeroed when a state takes them. */
int pn_pool_new(pn_model *m, int32_t n_pages, void *dev_buf, size_t bytes, pn_pool **out);

/* Pages not held by any state; -1 for NULL. */
int32_t pn_pool_free_pages(const pn_pool *p);

/* Release the pool's host handle; if states of the pool are alive, the handle
 * goes with the last of them (the device buffer stays the caller's and must
 * outlive every state of the pool). */
void pn_pool_free(pn_pool *p);

/* Bytes of device memory a pooled state of capacity max_ctx positions needs
 * (page table and attention split scratch; its K/V live in the pool). */
size_t pn_state_bytes_pooled(const pn_model *m, int32_t max_ctx);

/* Create a state (pos = 0, no pages) whose K/V pages come from `pool` in
 * `dev_buf` (>= pn_state_bytes_pooled, 256-byte aligned).  max_ctx bounds pos
 * as for pn_state_new; pn_state_set_page_table is not available (the pool
 * assigns pages).  Errors: PN_EINVAL (NULL, pool of another model or already
 * freed), PN_ERANGE (buffer too small). */
int pn_state_new_pooled(pn_model *m, pn_pool *pool, int32_t max_ctx, void *dev_buf, size_t bytes,
                        void *stream, pn_state **out);

/* One decode step of one sequence: embed token_dev[0], append its k and v at
 * pos, attend over the window ending at pos, run the FFN, and write the
 * logits (logits_dev [n_vocab] fp32, may be NULL) and the greedy id (argmax_dev
 * [1] int32, lowest index among equal maxima; may be NULL).  pos is advanced
 * on the host at enqueue.  token_dev may alias argmax_dev of the previous step
 * (greedy feedback with no host round trip). */
int pn_forward_step(pn_model *m, pn_state *s, const int32_t *token_dev, float *logits_dev,
                    int32_t *argmax_dev, void *stream);

/* One decode step of n distinct states (1 <= n <= max_batch), each at its own
 * pos: row i of tokens_dev [n], logits_dev [n][n_vocab] and argmax_dev [n]
 * belongs to states[i].  Same semantics as n independent pn_forward_step calls. */
int pn_forward_batch(pn_model *m, pn_state *const *states, int32_t n, const int32_t *tokens_dev,
                     float *logits_dev, int32_t *argmax_dev, void *stream);

/* Prefill: feed the n prompt tokens tokens_dev [n] (device) to state s at
 * positions pos..pos+n-1 and advance pos by n.  The result is that of n
 * pn_forward_step calls, one per token ("Engine Architecture", section
 * "Generation Loop": prefill runs the forward for each prompt token), up to
 * fp32 summation order: row t of logits_dev [n][n_vocab] and argmax_dev [n]
 * (either may be NULL) are the logits and greedy id after token t, and the
 * cache holds every token's K/V.  The tokens go in chunks (the pages' chunked
 * prefill: "Serve Layer Architecture", section "Batched Decode", "L2 - chunked
 * prefill"), so every weight is read once per chunk instead of once per token:
 * with prefill_chunk 0, chunks of max_batch, each one batched step whose rows
 * are consecutive positions of the state; otherwise chunks of prefill_chunk
 * rows on the wide path, whose fp32 sums run in another order (split K).  With
 * both outputs NULL the wide path skips the LM head.  Errors: PN_EINVAL (NULL pointer, n < 1, state
 * of another model), PN_ERANGE (pos + n > max_ctx, checked before anything is
 * enqueued; a pooled state's pool ran out: checked per chunk, so the chunks
 * before the one that found the pool empty stay done and pos counts them). */
int pn_prefill(pn_model *m, pn_state *s, const int32_t *tokens_dev, int32_t n, float *logits_dev,
               int32_t *argmax_dev, void *stream);

/* ---- sampling ------------------------------------------------------------- */

/* Sampling parameters of one row ("Engine Architecture", section "Sampling";
 * the pages' sampler seam takes them per request: "Core Engine API", section
 * "Sampler seam"). */
typedef struct pn_sampling_params {
    float temperature;     /* <= 0: greedy, the argmax of the raw logits (the rest unused) */
    float repeat_penalty;  /* applied to the distinct tokens of the row's recent window; 1 = none */
    int32_t top_k;         /* keep the top_k highest (1..4096) */
    float top_p;           /* keep the shortest top-ranked prefix whose probability exceeds
                              top_p; >= 1 = no cut */
} pn_sampling_params;

/* Sample one token per row of logits_dev [n][n_vocab] (fp32, device, not
 * modified) into ids_dev [n] (int32, device), on `stream`, in the pages'
 * order: divide by the temperature (fp32); penalise the row's recent tokens
 * (z / r if z > 0, else z * r); rank tokens by value, equal values by lower
 * index; keep the top_k; softmax over them (exp(z - z_max), fp64 sums); keep
 * the shortest prefix whose cumulative probability exceeds top_p of the total;
 * return the first token of the prefix whose cumulative probability exceeds
 * u times the prefix total.  u_dev [n] holds the caller's uniform draws in
 * [0, 1) (the random numbers are an input, so a seeded caller reproduces its
 * tokens).  recent_dev [n][n_recent] (0 <= n_recent <= 1024) lists each row's
 * recent tokens; entries < 0 or >= n_vocab are empty; it may be NULL when
 * n_recent is 0.  params is a host array [n]; 1 <= n <= max_batch.  Uses the
 * model's scratch (calls on one model must be stream-ordered).  Errors:
 * PN_EINVAL (NULL pointer, bad n, n_recent, NaN or non-positive penalty),
 * PN_EUNSUPPORTED (top_k outside 1..4096 with a positive temperature). */
int pn_sample(pn_model *m, const float *logits_dev, int32_t n, const pn_sampling_params *params,
              const int32_t *recent_dev, int32_t n_recent, const float *u_dev, int32_t *ids_dev, void *stream);

/* Sampling for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same sampler as pn_sample, with no model.  Its scratch is a file-scope
 * device array of fixed size (about 17 MB, held on each GPU the library runs
 * on until the process ends), so it needs no buffer from the caller; rows and
 * vocabulary are bounded by that array: 1 <= n <= 16, 1 <= n_vocab <= 262144
 * (PN_EINVAL beyond).  The call allocates nothing.  All calls on one GPU share
 * its array: calls that overlap on one GPU (other streams, other threads)
 * race, so order them.  Arguments, outputs and other errors as pn_sample,
 * with n_vocab giving the row length of logits_dev. */
int pn_sample_noalloc(const float *logits_dev, int32_t n, int32_t n_vocab, const pn_sampling_params *params,
                      const int32_t *recent_dev, int32_t n_recent, const float *u_dev, int32_t *ids_dev,
                      void *stream);

/* ---- tuning and measurement ------------------------------------------------ */

/* Kernel classes, for timing. */
enum {
    PN_K_EMBED = 0, PN_K_QKV, PN_K_ATTN, PN_K_O, PN_K_GATEUP, PN_K_DOWN, PN_K_LMHEAD,
    PN_K_ARGMAX, PN_K_ROUTER, PN_K_MOE_GATEUP, PN_K_MOE_DOWN, PN_K_MOE_COMBINE, PN_K_COUNT
};

/* Options (tuning only; results change at most by fp32 rounding):
 *  PN_OPT_ATTN_KEYS_PER_SPLIT  0 = automatic (about 256 attention
 *                              work-groups, or 512 when each split still
 *                              gets 8 pages, shared among the slots in
 *                              proportion to their windows), else a multiple
 *                              of 64: a slot's window of P pages of 64 keys is
 *                              cut into ceil(P / (value / 64)) splits that
 *                              share its pages evenly (at most the state's
 *                              split scratch, 256 splits);
 *  PN_OPT_ATTN_KERNEL          attention over a bf16 cache: 0 = automatic,
 *                              1 = vector units, 2 = matrix cores (an fp32
 *                              cache always uses the vector units);
 *  PN_OPT_ATTN_COMBINE         0 = automatic: a batch-1 decode step over a
 *                              bf16 cache on the matrix cores with at most 4
 *                              query heads per KV head and a window of at most
 *                              48 pages of 64 keys takes at most 8 attention
 *                              splits per head and combines them in the O
 *                              projection's prologue; 1 = always the separate
 *                              split-merge launch;
 *  PN_OPT_ATTN_WAVES           decode attention over a bf16 cache on the
 *                              matrix cores (at most 4 query heads per KV
 *                              head): waves per work-group, 0 = automatic (8
 *                              where the splits are combined in the O
 *                              prologue, else 4), 4 or 8 (ignored where the
 *                              combine runs in the O prologue);
 *  PN_OPT_GEMM_PROLOGUE        the O projection's input conversion in a
 *                              batched step: 0 = automatic (each wave of a
 *                              16-wave work-group converts its own k range of
 *                              every slot, up to 8 slots), 1 = the work-group
 *                              converts it together (the same values either
 *                              way);
 *  PN_OPT_WAVES_*              waves per work-group (4, 8 or 16) of the QKV,
 *                              O, gate/up, down and LM-head projections. */
enum {
    PN_OPT_ATTN_KEYS_PER_SPLIT = 1,
    PN_OPT_ATTN_KERNEL = 2,
    PN_OPT_ATTN_COMBINE = 3,
    PN_OPT_ATTN_WAVES = 4,
    PN_OPT_GEMM_PROLOGUE = 5,
    PN_OPT_WAVES_QKV = 10, PN_OPT_WAVES_O, PN_OPT_WAVES_GATEUP, PN_OPT_WAVES_DOWN, PN_OPT_WAVES_LMHEAD
};
int pn_model_set_option(pn_model *m, int32_t option, int64_t value);

/* Time every launch of kernel class `kernel` with HIP events recorded on the
 * launch stream, from pn_profile_begin until pn_profile_end (which
 * synchronizes the stream and reports the summed milliseconds and the
 * number of launches). */
int pn_profile_begin(pn_model *m, int32_t kernel);
int pn_profile_end(pn_model *m, void *stream, double *total_ms, int64_t *launches);

/* Enqueue `reps` launches of kernel class `kernel` (QKV, ATTN, O, GATEUP,
 * DOWN or LMHEAD; ATTN includes the split merge) back to back, cycling
 * through that class's launches of the most recent step (one per layer)
 * with their arguments, so that a caller can time the class with events
 * around the whole batch under the weight streams of a real step.  A QKV replay appends its
 * k, v rows to a model-owned scratch page rather than to any state; the
 * other classes rewrite only model scratch (activations, which the next
 * step rebuilds) and, for LMHEAD, the logits buffer of the recorded step.
 * PN_EINVAL when the class has no recorded launch (none since the model was
 * created, or a state of the recorded step was freed since). */
int pn_profile_replay(pn_model *m, int32_t kernel, int32_t reps, void *stream);

/* Routing record of an MoE model, for measurement (the bytes of a step's
 * expert FFN are those of the experts its rows chose).  With log_dev non-NULL,
 * decode call i (pn_forward_step or pn_forward_batch, counted from this call)
 * writes the experts each layer chose for each row into
 * log_dev[i % n_steps][n_layer][max_batch][n_expert_used] (int32, device,
 * caller-owned; rows past the call's n are not written), in the router kernel
 * itself (no extra launch).  NULL turns it off.  Errors: PN_EINVAL (NULL
 * model, a dense model, n_steps < 1). */
int pn_model_route_log(pn_model *m, int32_t *log_dev, int32_t n_steps);

/* Residual trace, for checking a deep model one layer at a time (each layer is
 * a function of its input residual, the cache and the position, so a
 * reference can recompute any layer from the device's own input).  With
 * trace_dev non-NULL, each later decode call (pn_forward_step,
 * pn_forward_batch) copies the fp32 residual stream x of its rows as it enters
 * each layer, and as it leaves the last one, into
 * trace_dev[n_layer + 1][max_batch][n_embd] (device, caller-owned; rows past
 * the call's n are not written): one device-to-device copy per layer on the
 * call's stream.  NULL turns it off.  Errors: PN_EINVAL (NULL model). */
int pn_model_trace(pn_model *m, float *trace_dev);

/* Streaming read ceiling, for measurement: read `bytes` (a positive multiple
 * of 16) of device memory at src_dev (16-byte aligned) with 16-byte loads
 * spread over every compute unit (their xor reaches *sink_dev, one device
 * word, caller-owned, only in the rare case that it equals a fixed constant:
 * the sink keeps the loads live and is not a checksum).  Its achieved bandwidth is the measured read ceiling
 * that the decode kernels' HBM rates are set against.  Errors: PN_EINVAL. */
int pn_stream_read(const void *src_dev, size_t bytes, uint32_t *sink_dev, void *stream);

/* Message of the last failure on this thread ("" if none). */
const char *pn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PN_H */
