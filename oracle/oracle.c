/*
 * oracle.c - plain, slow CPU reference of one decode step of a Llama-family
 * transformer, computed in fp64.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code with the HIP library.
 *
 * What it computes follows the Pantheon engine pages ("Core Engine API" and
 * "Engine Architecture"):
 *   - the forward signature forward(model, token, state) -> logits and the
 *     state {kv_cache, pos} (Core Engine API, sections "pn_model struct" and
 *     "pn_state struct");
 *   - the per-token intermediates listed by the scratch-arena sizing: per
 *     layer 5*n_embd + 3*n_ff + 2*n_kv_head*head_dim values (x, normed x,
 *     attention output, projections, FFN gate/up/hidden and the new k, v),
 *     MoE adding router logits and the chosen ids and weights, and once per
 *     token the normed output, the scores and the logits (Core Engine API,
 *     section "Scratch (arena) estimation");
 *   - the config keys and defaults: rope_theta 10000, rms_norm_eps 1e-5,
 *     sliding_window 0 = off, n_kv_head defaulting to n_head (Engine
 *     Architecture, section "Config Parsing");
 *   - Llama, Mistral and Mixtral sharing one forward, MoE switched on by an
 *     expert count > 0 and the window by a config flag (Engine Architecture,
 *     section "Architecture Detection");
 *   - greedy decoding = argmax of the logits (Engine Architecture, section
 *     "Sampling", temperature 0);
 *   - quantised weights dequantised inside the mat-vec, norms kept in F32
 *     (Engine Architecture, section "Weight Loading Modes");
 *   - a Q4 KV cache (Serve Layer Architecture, section "Environment
 *     Variables": the admission math counts a Q4-quantised KV cache): k and v
 *     kept as 32-dim Q4_0-style blocks (orc_q4_kv_round gives the reading);
 *   - the variants that share the Llama forward through config flags:
 *     attention biases (Qwen2) and, from Phi-3, the NeoX half-split RoPE
 *     (Engine Architecture, section "Architecture Detection").
 * Where the pages are silent the plain Llama reading is taken: RMSNorm with
 * eps inside the root; RoPE on adjacent pairs (2i, 2i+1) with
 * w_i = theta^(-2i/d) (NeoX: on the pairs (i, i + d/2), same w_i), applied to
 * q and k only, after the biases, k cached after rotation;
 * query head h reads kv head floor(h / (n_head / n_kv_head)); scores scaled by
 * 1/sqrt(d); the window holds the keys t with pos - W < t <= pos; SwiGLU FFN
 * down(silu(gate x) * up x); MoE softmax router, top-k with ties to the lower
 * index, weights renormalised over the chosen experts; untied LM head behind
 * a final RMSNorm.
 *
 * Precision.  Every stored value (fp32, bf16, int8 times an fp32 row scale,
 * or a Q8_0 / Q4_0 code times its block's fp16 scale) is widened to double on read
 * and all arithmetic is double.  The
 * values that the decode step stores in a narrower type are rounded at the
 * same points: the inputs of every mat-vec (normed x, attention output,
 * FFN hidden, final normed x) to the activation type, and the appended k, v
 * to the KV type.  Decisions that floating point takes, and that pick a
 * discrete result, are taken in fp32, the precision the GPU decides in: the
 * argmax of the logits and the router's top-k compare values rounded to fp32,
 * and a value stored as bf16 is first rounded to fp32, then to its bf16 code.
 * (With bf16 activations a 32-layer model is chaotic enough that a difference
 * of one fp32 ulp before a bf16 rounding moves its logits by about 1%.)
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_I8 = 2, ORC_Q8_0 = 3, ORC_Q4_0 = 4 };

/* Q8_0 block-quantised rows (GGUF-style): each row is cols/32 blocks of
 * 34 bytes, an fp16 scale d followed by 32 int8 codes q; weight = d * q. */
enum { Q8_BLOCK = 32, Q8_BLOCK_BYTES = 34 };

/* Q4_0 block-quantised rows (GGUF-style): each row is cols/32 blocks of
 * 18 bytes, an fp16 scale d followed by 16 bytes of 4-bit codes: byte i holds
 * code i in its low nibble and code i + 16 in its high nibble; weight =
 * d * (code - 8). */
enum { Q4_BLOCK_BYTES = 18 };

typedef struct {
    int32_t n_layer, n_embd, n_head, n_kv_head, head_dim, n_ff, n_vocab;
    int32_t n_expert, n_expert_used, sliding_window;
    double rope_theta, rms_norm_eps;
    int32_t w_dtype, kv_dtype, act_dtype;
    int32_t rope_neox; /* 1: rotate the half-split pairs (i, i + d/2) */
} orc_config;

/* Weight table (array of pointers, all host memory, matrices row-major [out][in]):
 *   [0] tok_embd [V][E]   (fp32 when w_dtype is fp32, else bf16)
 *   [1] out_norm [E] fp32     [2] w_out [V][E]     [3] s_out [V] (int8 only)
 *   per layer l, at 4 + l * orc_layer_stride(cfg):
 *   +0 attn_norm  +1 ffn_norm  +2 wq [H*d][E]  +3 wk [Hk*d][E]  +4 wv [Hk*d][E]
 *   +5 wo [E][H*d]  +6..+9 row scales of q, k, v, o (int8 only)
 *   +10 router [n_expert][E] (fp32 when w_dtype is fp32, else bf16)
 *   +11..+13 q, k, v biases [H*d], [Hk*d], [Hk*d] fp32, or NULL (no bias)
 *   +16 + 6e: gate [F][E], up [F][E], down [E][F], then their row scales.  */
int orc_layer_stride(const orc_config *c) { return 16 + 6 * (c->n_expert > 0 ? c->n_expert : 1); }

enum { T_EMBD = 0, T_OUT_NORM = 1, T_OUT = 2, T_S_OUT = 3, T_LAYER0 = 4 };
enum { L_ATTN_NORM = 0, L_FFN_NORM, L_WQ, L_WK, L_WV, L_WO, L_SQ, L_SK, L_SV, L_SO, L_ROUTER, L_BQ, L_BK, L_BV };

/* ------------------------------------------------------------------ rounding */

/* nearest bf16 value of v, ties to even (bf16 keeps 8 significant bits) */
double orc_round_bf16(double v) {
    if (v == 0.0 || !isfinite(v)) return v;
    int e;
    double m = frexp(v, &e);
    return ldexp(nearbyint(ldexp(m, 8)), e - 8);
}

/* Sensitivity probe, for the tests only (off unless a test sets it): with
 * eps > 0 every value about to be stored as bf16 is first multiplied by
 * (1 + eps * u), u uniform in [-1, 1) from a SplitMix64 counter (Steele, Lea
 * and Flood, "Fast splittable pseudorandom number generators", 2014).  It
 * measures how far the logits move when every bf16 rounding sees an input off
 * by a relative eps, as a GPU's fp32 arithmetic may be. */
static double g_pert_eps = 0.0;
static uint64_t g_pert_ctr = 0;

void orc_set_perturbation(double eps, uint64_t seed) {
    g_pert_eps = eps;
    g_pert_ctr = seed;
}

static double perturb(double v) {
    uint64_t z = (g_pert_ctr += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    double u = (double)(z >> 11) * 0x1.0p-52 - 1.0;
    return v * (1.0 + g_pert_eps * u);
}

/* v stored in type dt: fp32, or the bf16 code of its fp32 value (the decision
 * is taken in fp32, the precision the GPU decides in: fp64 -> fp32 -> bf16) */
static double round_to(double v, int dt) {
    if (dt == ORC_BF16) {
        if (g_pert_eps != 0.0) v = perturb(v);
        return orc_round_bf16((double)(float)v);
    }
    return (double)(float)v;
}

/* the storage rounding above, exported for the tests */
double orc_round_store(double v, int dt) { return round_to(v, dt); }

static uint16_t bf16_bits(double v) {
    float f = (float)orc_round_bf16((double)(float)v);
    uint32_t b;
    memcpy(&b, &f, 4);
    return (uint16_t)(b >> 16);
}

static double bf16_value(uint16_t h) {
    uint32_t b = (uint32_t)h << 16;
    float f;
    memcpy(&f, &b, 4);
    return (double)f;
}

/* IEEE binary16 bits -> double (normal, subnormal, zero, inf, NaN) */
double orc_half_to_double(uint16_t h) {
    int sign = h >> 15, e = (h >> 10) & 31, m = h & 1023;
    double v;
    if (e == 0) v = ldexp((double)m, -24);                    /* subnormal or zero */
    else if (e == 31) v = m ? NAN : INFINITY;
    else v = ldexp((double)(1024 + m), e - 25);               /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* weight (r, c) of a Q8_0 matrix with `cols` columns, dequantised: d * q */
static double q8_weight(const void *W, int cols, int r, int c) {
    const uint8_t *blk = (const uint8_t *)W + ((size_t)r * (size_t)(cols / Q8_BLOCK) + (size_t)(c / Q8_BLOCK)) * Q8_BLOCK_BYTES;
    uint16_t dbits = (uint16_t)(blk[0] | (blk[1] << 8));
    return orc_half_to_double(dbits) * (double)(int8_t)blk[2 + c % Q8_BLOCK];
}

/* weight (r, c) of a Q4_0 matrix with `cols` columns, dequantised: d * (code - 8) */
static double q4_weight(const void *W, int cols, int r, int c) {
    const uint8_t *blk = (const uint8_t *)W + ((size_t)r * (size_t)(cols / Q8_BLOCK) + (size_t)(c / Q8_BLOCK)) * Q4_BLOCK_BYTES;
    uint16_t dbits = (uint16_t)(blk[0] | (blk[1] << 8));
    int i = c % Q8_BLOCK;
    int code = i < 16 ? (blk[2 + i] & 15) : (blk[2 + i - 16] >> 4);
    return orc_half_to_double(dbits) * (double)(code - 8);
}

/* element i of a stored tensor, widened to double (int8: the raw code) */
static double rd(const void *p, int dt, size_t i) {
    switch (dt) {
        case ORC_F32: return (double)((const float *)p)[i];
        case ORC_BF16: return bf16_value(((const uint16_t *)p)[i]);
        default: return (double)((const int8_t *)p)[i];
    }
}

/* ------------------------------------------------------------------ building blocks */

static int g_threads = 1;

/* y[r] = sum_c W[r][c] * x[c]; int8 rows are scaled by s[r] after the sum;
 * Q8_0 and Q4_0 weights are dequantised (d * q, d * (code - 8)) before the product ("Weight Loading
 * Modes": dequantisation per block inside the mat-vec) */
static void matvec(const void *W, int dt, const float *s, int rows, int cols, const double *x,
                   double *y) {
#pragma omp parallel for num_threads(g_threads) schedule(static) if (g_threads > 1)
    for (int r = 0; r < rows; ++r) {
        double acc = 0.0;
        size_t base = (size_t)r * (size_t)cols;
        if (dt == ORC_Q8_0)
            for (int c = 0; c < cols; ++c) acc += q8_weight(W, cols, r, c) * x[c];
        else if (dt == ORC_Q4_0)
            for (int c = 0; c < cols; ++c) acc += q4_weight(W, cols, r, c) * x[c];
        else
            for (int c = 0; c < cols; ++c) acc += rd(W, dt, base + (size_t)c) * x[c];
        y[r] = (dt == ORC_I8) ? (double)s[r] * acc : acc;
    }
}

/* the mat-vec above, exported for the tests (one thread) */
void orc_matvec(const void *W, int dt, const float *s, int rows, int cols, const double *x, double *y) {
    int t = g_threads;
    g_threads = 1;
    matvec(W, dt, s, rows, cols, x, y);
    g_threads = t;
}

/* y = x * (mean(x^2) + eps)^(-1/2) * g */
void orc_rmsnorm(const double *x, const float *g, int n, double eps, double *y) {
    double ss = 0.0;
    for (int i = 0; i < n; ++i) ss += x[i] * x[i];
    double inv = 1.0 / sqrt(ss / (double)n + eps);
    for (int i = 0; i < n; ++i) y[i] = x[i] * inv * (double)g[i];
}

/* rotate pairs (u[2i], u[2i+1]) of one head vector by pos * theta^(-2i/d) */
void orc_rope(double *u, int d, int pos, double theta) {
    for (int i = 0; i < d / 2; ++i) {
        double w = pow(theta, -2.0 * (double)i / (double)d);
        double phi = (double)pos * w;
        double c = cos(phi), s = sin(phi);
        double a = u[2 * i], b = u[2 * i + 1];
        u[2 * i] = a * c - b * s;
        u[2 * i + 1] = a * s + b * c;
    }
}

/* NeoX form: rotate pairs (u[i], u[i + d/2]) of one head vector by
 * pos * theta^(-2i/d) (the half-split RoPE that "Engine Architecture",
 * section "Architecture Detection", names for Phi-3) */
void orc_rope_neox(double *u, int d, int pos, double theta) {
    int h = d / 2;
    for (int i = 0; i < h; ++i) {
        double w = pow(theta, -2.0 * (double)i / (double)d);
        double phi = (double)pos * w;
        double c = cos(phi), s = sin(phi);
        double a = u[i], b = u[i + h];
        u[i] = a * c - b * s;
        u[i + h] = a * s + b * c;
    }
}

/* one query against T keys/values [T][d]: o = sum_t softmax(q.K_t / sqrt(d)) V_t */
void orc_attend(const double *q, const double *K, const double *V, int T, int d, double *o) {
    double *sc = (double *)malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
    double mx = -INFINITY;
    double scale = 1.0 / sqrt((double)d);
    for (int t = 0; t < T; ++t) {
        double dot = 0.0;
        for (int i = 0; i < d; ++i) dot += q[i] * K[(size_t)t * d + i];
        sc[t] = dot * scale;
        if (sc[t] > mx) mx = sc[t];
    }
    double den = 0.0;
    for (int t = 0; t < T; ++t) {
        sc[t] = exp(sc[t] - mx);
        den += sc[t];
    }
    for (int i = 0; i < d; ++i) o[i] = 0.0;
    for (int t = 0; t < T; ++t) {
        double a = sc[t] / den;
        for (int i = 0; i < d; ++i) o[i] += a * V[(size_t)t * d + i];
    }
    free(sc);
}

/* Grouped-query attention of all heads at position pos.
 * q [H][d]; K, V [Hk][T][d] hold positions 0..T-1 (T > pos); W = window (0 = off).
 * Query head h reads kv head h / (H / Hk); keys t with max(0, pos-W+1) <= t <= pos. */
void orc_attention(const double *q, const double *K, const double *V, int H, int Hk, int d,
                   int T, int pos, int W, double *o) {
    int G = H / Hk;
    int t0 = (W > 0 && pos - W + 1 > 0) ? pos - W + 1 : 0;
    int n = pos - t0 + 1;
#pragma omp parallel for num_threads(g_threads) schedule(static) if (g_threads > 1)
    for (int h = 0; h < H; ++h) {
        int j = h / G;
        const double *Kj = K + ((size_t)j * T + t0) * d;
        const double *Vj = V + ((size_t)j * T + t0) * d;
        orc_attend(q + (size_t)h * d, Kj, Vj, n, d, o + (size_t)h * d);
    }
}

double orc_silu(double z) { return z / (1.0 + exp(-z)); }

/* Top-k routing of one token: ids by descending router logit compared in fp32
 * (ties -> lower index); weights = softmax over all experts, renormalised over
 * the chosen ones (equal to a softmax over the chosen logits). Returns the
 * fp32 gap between the k-th and (k+1)-th logits (inf if k == n).  With `swap`
 * (and k < n) the (k+1)-th expert takes the k-th one's place: the other valid
 * choice when those two logits are a near tie that fp32 cannot order. */
static double route(const double *r, int n, int k, int swap, int32_t *ids, double *w) {
    char *used = (char *)calloc((size_t)n, 1);
    for (int a = 0; a < k; ++a) {
        int best = -1;
        float bv = 0.0f;
        for (int e = 0; e < n; ++e) {
            if (used[e]) continue;
            float v = (float)r[e];
            if (best < 0 || v > bv) { best = e; bv = v; }
        }
        used[best] = 1;
        ids[a] = best;
    }
    double gap = INFINITY;
    if (k < n) {
        float kth = (float)r[ids[k - 1]], next = -INFINITY;
        int inext = -1;
        for (int e = 0; e < n; ++e)
            if (!used[e] && (inext < 0 || (float)r[e] > next)) { next = (float)r[e]; inext = e; }
        gap = (double)kth - (double)next;
        if (swap) ids[k - 1] = inext;
    }
    free(used);
    double mx = -INFINITY;
    for (int e = 0; e < n; ++e) if (r[e] > mx) mx = r[e];
    double den = 0.0;
    for (int e = 0; e < n; ++e) den += exp(r[e] - mx);
    double sel = 0.0;
    for (int a = 0; a < k; ++a) {
        w[a] = exp(r[ids[a]] - mx) / den;
        sel += w[a];
    }
    for (int a = 0; a < k; ++a) w[a] /= sel;
    return gap;
}

double orc_moe_route(const double *r, int n, int k, int32_t *ids, double *w) {
    return route(r, n, k, 0, ids, w);
}

double orc_moe_route_swapped(const double *r, int n, int k, int32_t *ids, double *w) {
    return route(r, n, k, 1, ids, w);
}

/* index of the largest logit compared in fp32, lowest index among equal maxima;
 * -1 if any logit is NaN */
int orc_argmax(const double *logits, int n) {
    int best = 0;
    float bv = (float)logits[0];
    for (int i = 0; i < n; ++i) {
        float v = (float)logits[i];
        if (v != v) return -1;
        if (v > bv) { bv = v; best = i; }
    }
    return best;
}

/* ------------------------------------------------------------------ state */

typedef struct {
    orc_config cfg;
    int max_ctx, pos;
    void **k, **v; /* per layer [Hk][max_ctx][d] in kv dtype */
} orc_state;

/* bytes per cached element: a Q4_0 cache is kept here as its exact dequantised fp32 values */
static size_t kv_elem(const orc_config *c) { return c->kv_dtype == ORC_BF16 ? 2 : 4; }
static int kv_store_dt(const orc_config *c) { return c->kv_dtype == ORC_Q4_0 ? ORC_F32 : c->kv_dtype; }

/* fp16 bits of a finite float, round to nearest even (magnitudes past 65504 give inf) */
static uint16_t half_rne(float f) {
    uint16_t sign = (uint16_t)(signbit(f) ? 0x8000 : 0);
    double a = fabs((double)f);
    if (a == 0.0) return sign;
    int e;
    double m = frexp(a, &e); /* a = m 2^e, m in [0.5, 1) */
    int E = e - 1 + 15;
    if (E >= 1) {
        double r = nearbyint(ldexp(m, 11));
        if (r == 2048.0) { r = 1024.0; E += 1; }
        if (E >= 31) return (uint16_t)(sign | 0x7C00);
        return (uint16_t)(sign | (E << 10) | ((int)r - 1024));
    }
    return (uint16_t)(sign | (uint16_t)nearbyint(ldexp(a, 24)));
}

/* A Q4 KV cache stores each head vector in blocks of 32 dims, Q4_0-style: an
 * fp16 scale d and 4-bit codes, value d * (code - 8).  The pages only name the
 * Q4 KV cache; the rule taken here: m = the element of largest magnitude (the
 * first on ties), d = fp16(m / -8), code = clamp(rint(x / d) + 8, 0, 15) (all
 * codes 8 when d is 0).  Every decision is taken on fp32 values with fp32
 * division, as the GPU takes it.  out[i] receives the stored value. */
void orc_q4_kv_round(const double *u, int d, double *out) {
    for (int b = 0; b + 32 <= d; b += 32) {
        float f[32];
        int im = 0;
        for (int i = 0; i < 32; ++i) {
            f[i] = (float)u[b + i];
            if (fabsf(f[i]) > fabsf(f[im])) im = i;
        }
        float dv = f[im] / -8.0f;
        float dd = (float)orc_half_to_double(half_rne(dv));
        for (int i = 0; i < 32; ++i) {
            int code = 8;
            if (dd != 0.0f) {
                volatile float q = f[i] / dd; /* fp32 quotient, correctly rounded */
                float r = nearbyintf(q) + 8.0f;
                code = r < 0.0f ? 0 : (r > 15.0f ? 15 : (int)r);
            }
            out[b + i] = (double)dd * (double)(code - 8);
        }
    }
}

/* a head vector [d] as the cache stores it */
static void kv_round_head(const orc_config *c, const double *u, int d, double *out) {
    if (c->kv_dtype == ORC_Q4_0) {
        orc_q4_kv_round(u, d, out);
        return;
    }
    for (int i = 0; i < d; ++i) out[i] = round_to(u[i], c->kv_dtype);
}

orc_state *orc_state_new(const orc_config *c, int max_ctx) {
    orc_state *s = (orc_state *)calloc(1, sizeof(orc_state));
    s->cfg = *c;
    s->max_ctx = max_ctx;
    s->k = (void **)calloc((size_t)c->n_layer, sizeof(void *));
    s->v = (void **)calloc((size_t)c->n_layer, sizeof(void *));
    size_t bytes = (size_t)c->n_kv_head * (size_t)max_ctx * (size_t)c->head_dim * kv_elem(c);
    for (int l = 0; l < c->n_layer; ++l) {
        s->k[l] = calloc(1, bytes);
        s->v[l] = calloc(1, bytes);
        if (!s->k[l] || !s->v[l]) return NULL;
    }
    return s;
}

void orc_state_free(orc_state *s) {
    if (!s) return;
    for (int l = 0; l < s->cfg.n_layer; ++l) {
        free(s->k[l]);
        free(s->v[l]);
    }
    free(s->k);
    free(s->v);
    free(s);
}

void orc_state_set_pos(orc_state *s, int pos) { s->pos = pos; }
int orc_state_pos(const orc_state *s) { return s->pos; }

/* copy stored K/V of positions pos0..pos0+n-1, given as [n][Hk][d] in kv dtype
 * (a Q4 cache takes fp32 vectors and stores them as an append would) */
int orc_state_set_kv(orc_state *s, int layer, int pos0, int n, const void *k, const void *v) {
    const orc_config *c = &s->cfg;
    if (layer < 0 || layer >= c->n_layer || pos0 < 0 || pos0 + n > s->max_ctx) return -2;
    size_t es = kv_elem(c), d = (size_t)c->head_dim;
    double *u = (double *)malloc(sizeof(double) * d), *r = (double *)malloc(sizeof(double) * d);
    for (int t = 0; t < n; ++t)
        for (int j = 0; j < c->n_kv_head; ++j) {
            size_t src = ((size_t)t * c->n_kv_head + j) * d * es;
            size_t dst = ((size_t)j * s->max_ctx + (size_t)(pos0 + t)) * d * es;
            if (c->kv_dtype == ORC_Q4_0) {
                for (int w = 0; w < 2; ++w) {
                    const float *in = (const float *)((const char *)(w ? v : k) + src);
                    float *o = (float *)((char *)(w ? s->v[layer] : s->k[layer]) + dst);
                    for (size_t i = 0; i < d; ++i) u[i] = (double)in[i];
                    orc_q4_kv_round(u, (int)d, r);
                    for (size_t i = 0; i < d; ++i) o[i] = (float)r[i];
                }
                continue;
            }
            memcpy((char *)s->k[layer] + dst, (const char *)k + src, d * es);
            memcpy((char *)s->v[layer] + dst, (const char *)v + src, d * es);
        }
    free(u);
    free(r);
    return 0;
}

static void store_kv(void *base, int dt, size_t i, double v) {
    if (dt == ORC_BF16)
        ((uint16_t *)base)[i] = bf16_bits(v);
    else
        ((float *)base)[i] = (float)v;
}

/* ------------------------------------------------------------------ one layer */

typedef struct {
    double *xn, *q, *k, *v, *o, *tmp, *g, *u, *h, *y, *acc, *r;
} scratch;

static void scratch_new(const orc_config *c, scratch *s) {
    size_t E = c->n_embd, Hd = (size_t)c->n_head * c->head_dim, F = c->n_ff;
    size_t Kd = (size_t)c->n_kv_head * c->head_dim;
    s->xn = malloc(sizeof(double) * E);
    s->q = malloc(sizeof(double) * Hd);
    s->k = malloc(sizeof(double) * Kd);
    s->v = malloc(sizeof(double) * Kd);
    s->o = malloc(sizeof(double) * Hd);
    s->tmp = malloc(sizeof(double) * E);
    s->g = malloc(sizeof(double) * F);
    s->u = malloc(sizeof(double) * F);
    s->h = malloc(sizeof(double) * F);
    s->y = malloc(sizeof(double) * E);
    s->acc = malloc(sizeof(double) * E);
    s->r = malloc(sizeof(double) * (size_t)(c->n_expert > 0 ? c->n_expert : 1));
}

static void scratch_free(scratch *s) {
    free(s->xn); free(s->q); free(s->k); free(s->v); free(s->o); free(s->tmp);
    free(s->g); free(s->u); free(s->h); free(s->y); free(s->acc); free(s->r);
}

static const void *T(const void *const *tab, int i) { return tab[i]; }

static int wdt(const orc_config *c) { return c->w_dtype; }
static int aux_dt(const orc_config *c) { return c->w_dtype == ORC_F32 ? ORC_F32 : ORC_BF16; }

/* the FFN of one token: x += FFN(round_act(RMSNorm(x) * g_ffn)); returns the
 * router's fp32 k-th/(k+1)-th gap for MoE layers, +inf otherwise; `swap`
 * routes to the (k+1)-th expert in place of the k-th (see route) */
static double ffn(const orc_config *c, const void *const *tab, int lb, double *x, scratch *s,
                  int32_t *ids_out, int swap) {
    int E = c->n_embd, F = c->n_ff;
    orc_rmsnorm(x, (const float *)T(tab, lb + L_FFN_NORM), E, c->rms_norm_eps, s->xn);
    for (int i = 0; i < E; ++i) s->xn[i] = round_to(s->xn[i], c->act_dtype);
    int n_used = c->n_expert > 0 ? c->n_expert_used : 1;
    int32_t *ids = (int32_t *)malloc(sizeof(int32_t) * (size_t)n_used);
    double *w = (double *)malloc(sizeof(double) * (size_t)n_used);
    double gap = INFINITY;
    if (c->n_expert > 0) {
        matvec(T(tab, lb + L_ROUTER), aux_dt(c), NULL, c->n_expert, E, s->xn, s->r);
        gap = route(s->r, c->n_expert, n_used, swap, ids, w);
    } else {
        ids[0] = 0;
        w[0] = 1.0;
    }
    for (int i = 0; i < E; ++i) s->acc[i] = 0.0;
    for (int a = 0; a < n_used; ++a) {
        int eb = lb + 16 + 6 * ids[a];
        matvec(T(tab, eb + 0), wdt(c), (const float *)T(tab, eb + 3), F, E, s->xn, s->g);
        matvec(T(tab, eb + 1), wdt(c), (const float *)T(tab, eb + 4), F, E, s->xn, s->u);
        for (int i = 0; i < F; ++i) s->h[i] = round_to(orc_silu(s->g[i]) * s->u[i], c->act_dtype);
        matvec(T(tab, eb + 2), wdt(c), (const float *)T(tab, eb + 5), E, F, s->h, s->y);
        for (int i = 0; i < E; ++i) s->acc[i] += w[a] * s->y[i];
        if (ids_out) ids_out[a] = ids[a];
    }
    for (int i = 0; i < E; ++i) x[i] += s->acc[i];
    free(ids);
    free(w);
    return gap;
}

/* y[r] += b[r] when the bias exists */
static void add_bias(double *y, const void *b, int n) {
    if (!b) return;
    for (int r = 0; r < n; ++r) y[r] += (double)((const float *)b)[r];
}

/* q, k, v of one token at position pos: round_act(RMSNorm(x)*g), projections,
 * biases (Qwen2's attention biases: "Engine Architecture", section
 * "Architecture Detection"), RoPE */
static void qkv(const orc_config *c, const void *const *tab, int lb, const double *x, int pos,
                scratch *s) {
    int E = c->n_embd, d = c->head_dim, H = c->n_head, Hk = c->n_kv_head;
    orc_rmsnorm(x, (const float *)T(tab, lb + L_ATTN_NORM), E, c->rms_norm_eps, s->xn);
    for (int i = 0; i < E; ++i) s->xn[i] = round_to(s->xn[i], c->act_dtype);
    matvec(T(tab, lb + L_WQ), wdt(c), (const float *)T(tab, lb + L_SQ), H * d, E, s->xn, s->q);
    matvec(T(tab, lb + L_WK), wdt(c), (const float *)T(tab, lb + L_SK), Hk * d, E, s->xn, s->k);
    matvec(T(tab, lb + L_WV), wdt(c), (const float *)T(tab, lb + L_SV), Hk * d, E, s->xn, s->v);
    add_bias(s->q, T(tab, lb + L_BQ), H * d);
    add_bias(s->k, T(tab, lb + L_BK), Hk * d);
    add_bias(s->v, T(tab, lb + L_BV), Hk * d);
    void (*rot)(double *, int, int, double) = c->rope_neox ? orc_rope_neox : orc_rope;
    for (int h = 0; h < H; ++h) rot(s->q + (size_t)h * d, d, pos, c->rope_theta);
    for (int j = 0; j < Hk; ++j) rot(s->k + (size_t)j * d, d, pos, c->rope_theta);
}

/* x += W_o * round_act(o) */
static void attn_out(const orc_config *c, const void *const *tab, int lb, double *x, scratch *s) {
    int E = c->n_embd, Hd = c->n_head * c->head_dim;
    for (int i = 0; i < Hd; ++i) s->o[i] = round_to(s->o[i], c->act_dtype);
    matvec(T(tab, lb + L_WO), wdt(c), (const float *)T(tab, lb + L_SO), E, Hd, s->o, s->tmp);
    for (int i = 0; i < E; ++i) x[i] += s->tmp[i];
}

/* logits = W_out * round_act(RMSNorm(x) * g_out) */
static void head(const orc_config *c, const void *const *tab, const double *x, double *logits,
                 scratch *s) {
    int E = c->n_embd;
    orc_rmsnorm(x, (const float *)T(tab, T_OUT_NORM), E, c->rms_norm_eps, s->xn);
    for (int i = 0; i < E; ++i) s->xn[i] = round_to(s->xn[i], c->act_dtype);
    matvec(T(tab, T_OUT), wdt(c), (const float *)T(tab, T_S_OUT), c->n_vocab, E, s->xn, logits);
}

static void embed(const orc_config *c, const void *const *tab, int token, double *x) {
    for (int i = 0; i < c->n_embd; ++i)
        x[i] = rd(T(tab, T_EMBD), aux_dt(c), (size_t)token * c->n_embd + (size_t)i);
}

/* ------------------------------------------------------------------ decode step */

/* Layer l of one token at position p: x += attention(...) + FFN(...), with
 * the token's k, v appended to the state's cache at p (state->pos is not
 * moved).  Returns the router's fp32 k-th/(k+1)-th gap (+inf for dense);
 * `ids` (optional, [n_expert_used]) receives the chosen experts and `swap`
 * routes to the (k+1)-th expert in place of the k-th. */
static double layer_step(const orc_config *c, const void *const *tab, orc_state *st, int l, int p, double *x,
                         scratch *s, int32_t *ids, int swap) {
    int d = c->head_dim, H = c->n_head, Hk = c->n_kv_head;
    int lb = T_LAYER0 + l * orc_layer_stride(c);
    int t0 = (c->sliding_window > 0 && p - c->sliding_window + 1 > 0) ? p - c->sliding_window + 1 : 0;
    int n = p - t0 + 1;
    double *K = malloc(sizeof(double) * (size_t)Hk * n * d);
    double *V = malloc(sizeof(double) * (size_t)Hk * n * d);
    double *rk = malloc(sizeof(double) * d), *rv = malloc(sizeof(double) * d);
    qkv(c, tab, lb, x, p, s);
    for (int j = 0; j < Hk; ++j) {
        kv_round_head(c, s->k + (size_t)j * d, d, rk);
        kv_round_head(c, s->v + (size_t)j * d, d, rv);
        for (int i = 0; i < d; ++i) {
            size_t at = ((size_t)j * st->max_ctx + (size_t)p) * d + (size_t)i;
            store_kv(st->k[l], kv_store_dt(c), at, rk[i]);
            store_kv(st->v[l], kv_store_dt(c), at, rv[i]);
        }
    }
    /* the window's cached keys and values, widened to double, [Hk][n][d] */
    for (int j = 0; j < Hk; ++j)
        for (int t = 0; t < n; ++t)
            for (int i = 0; i < d; ++i) {
                size_t src = ((size_t)j * st->max_ctx + (size_t)(t0 + t)) * d + (size_t)i;
                size_t dst = ((size_t)j * n + (size_t)t) * d + (size_t)i;
                K[dst] = rd(st->k[l], kv_store_dt(c), src);
                V[dst] = rd(st->v[l], kv_store_dt(c), src);
            }
    /* keys are the window only, so position p sits at index n-1 and W is not re-applied */
    orc_attention(s->q, K, V, H, Hk, d, n, n - 1, 0, s->o);
    attn_out(c, tab, lb, x, s);
    double gap = ffn(c, tab, lb, x, s, ids, swap);
    free(K);
    free(V);
    free(rk);
    free(rv);
    return gap;
}

static int check_step_args(const orc_config *c, const orc_state *st, int p) {
    if (p < 0 || p >= st->max_ctx) return -2;
    if (c->head_dim < 2 || c->head_dim % 2 || c->n_head % c->n_kv_head) return -4;
    return 0;
}

/* One decode step: append the token's k, v at state->pos, attend, write the
 * logits [V] and return the greedy id (or a negative error).  `route_ids`
 * (optional, [n_layer][n_expert_used]) receives the experts each layer chose,
 * `layer_gaps` (optional, [n_layer]) each layer's router k-th/(k+1)-th fp32
 * gap (+inf for dense layers), and `route_gap` (optional) the smallest of
 * them.  Bit l of `swap_mask` makes layer l (< 64) route to the (k+1)-th
 * expert in place of the k-th: the other branch of a routing near tie. */
int orc_step_ex(const orc_config *c, const void *const *tab, orc_state *st, int token,
                double *logits, int nthreads, int32_t *route_ids, double *layer_gaps,
                double *route_gap, uint64_t swap_mask) {
    int p = st->pos;
    if (token < 0 || token >= c->n_vocab) return -3;
    if (check_step_args(c, st, p)) return check_step_args(c, st, p);
    g_threads = nthreads > 0 ? nthreads : 1;
    scratch s;
    scratch_new(c, &s);
    double *x = malloc(sizeof(double) * c->n_embd);
    double gap = INFINITY;
    embed(c, tab, token, x);
    for (int l = 0; l < c->n_layer; ++l) {
        double gl = layer_step(c, tab, st, l, p, x, &s,
                               route_ids ? route_ids + (size_t)l * (c->n_expert > 0 ? c->n_expert_used : 1) : NULL,
                               l < 64 && ((swap_mask >> l) & 1));
        if (layer_gaps) layer_gaps[l] = gl;
        if (gl < gap) gap = gl;
    }
    head(c, tab, x, logits, &s);
    st->pos = p + 1;
    if (route_gap) *route_gap = gap;
    free(x);
    scratch_free(&s);
    return orc_argmax(logits, c->n_vocab);
}

/* The step's parts, for checking a deep model one layer at a time from
 * inputs given by the caller (a layer is a function of its input x, the
 * cache and the position).  orc_embed: x_out [E] = the token's embedding row.
 * orc_layer: x_out = layer l applied to x_in at position pos (the layer's k,
 * v appended to the state's cache at pos; pos not moved); returns the router
 * gap as layer_step, or a value < -1e300 on a bad argument.  orc_head: the
 * logits [V] of x_in (final RMSNorm, LM head) and the greedy id.  Running
 * orc_embed, every orc_layer and orc_head in turn is orc_step. */
int orc_embed(const orc_config *c, const void *const *tab, int token, double *x_out) {
    if (token < 0 || token >= c->n_vocab) return -3;
    embed(c, tab, token, x_out);
    return 0;
}

double orc_layer(const orc_config *c, const void *const *tab, orc_state *st, int l, int pos, const double *x_in,
                 double *x_out, int nthreads, int swap, int32_t *ids) {
    if (l < 0 || l >= c->n_layer || check_step_args(c, st, pos)) return -INFINITY;
    g_threads = nthreads > 0 ? nthreads : 1;
    scratch s;
    scratch_new(c, &s);
    memcpy(x_out, x_in, sizeof(double) * (size_t)c->n_embd);
    double gap = layer_step(c, tab, st, l, pos, x_out, &s, ids, swap);
    scratch_free(&s);
    return gap;
}

int orc_head(const orc_config *c, const void *const *tab, const double *x_in, double *logits, int nthreads) {
    g_threads = nthreads > 0 ? nthreads : 1;
    scratch s;
    scratch_new(c, &s);
    head(c, tab, x_in, logits, &s);
    scratch_free(&s);
    return orc_argmax(logits, c->n_vocab);
}

int orc_step(const orc_config *c, const void *const *tab, orc_state *st, int token,
             double *logits, int nthreads, int32_t *route_ids, double *route_gap) {
    return orc_step_ex(c, tab, st, token, logits, nthreads, route_ids, NULL, route_gap, 0);
}

/* Causal forward over tokens[0..n-1] from scratch (no cache carried between
 * calls): every position's k, v are recomputed and rounded to the KV type, and
 * the logits of the last position are written.  Returns its greedy id. */
int orc_full_recompute(const orc_config *c, const void *const *tab, const int32_t *tokens, int n,
                       double *logits, int nthreads) {
    int E = c->n_embd, d = c->head_dim, H = c->n_head, Hk = c->n_kv_head;
    g_threads = nthreads > 0 ? nthreads : 1;
    for (int t = 0; t < n; ++t)
        if (tokens[t] < 0 || tokens[t] >= c->n_vocab) return -3;
    scratch s;
    scratch_new(c, &s);
    double *X = malloc(sizeof(double) * (size_t)n * E);
    double *Q = malloc(sizeof(double) * (size_t)n * H * d);
    double *K = malloc(sizeof(double) * (size_t)Hk * n * d);
    double *V = malloc(sizeof(double) * (size_t)Hk * n * d);
    for (int t = 0; t < n; ++t) embed(c, tab, tokens[t], X + (size_t)t * E);
    for (int l = 0; l < c->n_layer; ++l) {
        int lb = T_LAYER0 + l * orc_layer_stride(c);
        for (int t = 0; t < n; ++t) {
            qkv(c, tab, lb, X + (size_t)t * E, t, &s);
            memcpy(Q + (size_t)t * H * d, s.q, sizeof(double) * (size_t)H * d);
            for (int j = 0; j < Hk; ++j) {
                kv_round_head(c, s.k + (size_t)j * d, d, K + ((size_t)j * n + t) * d);
                kv_round_head(c, s.v + (size_t)j * d, d, V + ((size_t)j * n + t) * d);
            }
        }
        for (int t = 0; t < n; ++t) {
            orc_attention(Q + (size_t)t * H * d, K, V, H, Hk, d, n, t, c->sliding_window, s.o);
            attn_out(c, tab, lb, X + (size_t)t * E, &s);
            ffn(c, tab, lb, X + (size_t)t * E, &s, NULL, 0);
        }
    }
    head(c, tab, X + (size_t)(n - 1) * E, logits, &s);
    free(X);
    free(Q);
    free(K);
    free(V);
    scratch_free(&s);
    return orc_argmax(logits, c->n_vocab);
}

int orc_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
