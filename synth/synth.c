/*
 * synth.c - seeded, counter-based synthetic inputs for the decode step.
 *
 * This module only draws numbers: weights, norm gains, cached K/V, token ids
 * and slot positions.  It holds none of the decode arithmetic.  Both the
 * oracle and the HIP path consume what it writes, so the two see identical
 * stored values.
 *
 * Generator.  Element c of a stream is the SplitMix64 output for counter c
 * (Steele, Lea and Flood, "Fast splittable pseudorandom number generators",
 * OOPSLA 2014; finaliser constants of Vigna's splitmix64):
 *     state_c = key + (c + 1) * 0x9E3779B97F4A7C15
 *     out     = mix(state_c)
 * with key = mix(seed) so that nearby seeds give unrelated streams.  The
 * counter of element i of tensor t is (t << 41) + i for uniforms; a normal
 * takes the pair of counters (t << 41) + 2*(i/2) + {0, 1} and applies the
 * Box-Muller transform (cosine branch for even i, sine branch for odd i), all
 * in double with the host libm.  Any element is therefore addressable on its
 * own, which lets a caller draw any sub-range without drawing the rest.
 *
 * Storage.  A double is rounded to fp32 by the C conversion (round to nearest
 * even) and to bf16 by rounding the 8-bit significand to nearest even.
 * INT8 rows follow the symmetric per-row rule: scale = fl32(max|w| / 127) of
 * the bf16 draw, q = rint(w / scale) clamped to [-127, 127] (q = 0 when the
 * scale is 0).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SM_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
    return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed) { return sm_mix(seed + SM_GAMMA); }

static inline uint64_t draw_u64(uint64_t key, uint64_t ctr) {
    return sm_mix(key + (ctr + 1ULL) * SM_GAMMA);
}

/* uniform in [0, 1) with 53 random bits */
static inline double u01(uint64_t r) { return (double)(r >> 11) * 0x1.0p-53; }
/* uniform in (0, 1] */
static inline double u01_open0(uint64_t r) { return (double)((r >> 11) + 1ULL) * 0x1.0p-53; }

static inline uint64_t tensor_base(uint64_t tid) { return tid << 41; }

static inline double normal_at(uint64_t key, uint64_t tid, uint64_t i) {
    uint64_t c = tensor_base(tid) + 2ULL * (i >> 1);
    double u1 = u01_open0(draw_u64(key, c));
    double u2 = u01(draw_u64(key, c + 1ULL));
    double r = sqrt(-2.0 * log(u1));
    double a = 6.283185307179586476925286766559 * u2;
    return (i & 1ULL) ? r * sin(a) : r * cos(a);
}

/* round a double to bf16 (nearest even) and return its bit pattern */
static inline uint16_t bf16_bits_rne(double v) {
    if (v == 0.0 || !isfinite(v)) {
        float f = (float)v;
        uint32_t b;
        memcpy(&b, &f, 4);
        return (uint16_t)(b >> 16);
    }
    int e;
    double m = frexp(v, &e);                 /* v = m * 2^e, 0.5 <= |m| < 1 */
    double q = nearbyint(ldexp(m, 8));       /* 8 significant bits, ties to even */
    float f = (float)ldexp(q, e - 8);        /* exact in fp32 */
    uint32_t b;
    memcpy(&b, &f, 4);
    return (uint16_t)(b >> 16);
}

static inline double bf16_bits_to_double(uint16_t h) {
    uint32_t b = (uint32_t)h << 16;
    float f;
    memcpy(&f, &b, 4);
    return (double)f;
}

/* ---- simple static-partition thread pool ---------------------------------- */

typedef void (*range_fn)(void *ctx, uint64_t lo, uint64_t hi);

typedef struct {
    range_fn fn;
    void *ctx;
    uint64_t lo, hi;
} job_t;

static void *job_main(void *p) {
    job_t *j = (job_t *)p;
    j->fn(j->ctx, j->lo, j->hi);
    return NULL;
}

static void parallel_range(range_fn fn, void *ctx, uint64_t n, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if ((uint64_t)nthreads > n / 4096 + 1) nthreads = (int)(n / 4096 + 1);
    if (nthreads == 1) {
        fn(ctx, 0, n);
        return;
    }
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    job_t *jobs = (job_t *)malloc(sizeof(job_t) * (size_t)nthreads);
    uint64_t chunk = (n + (uint64_t)nthreads - 1) / (uint64_t)nthreads;
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        uint64_t lo = (uint64_t)t * chunk, hi = lo + chunk;
        if (lo >= n) break;
        if (hi > n) hi = n;
        jobs[t].fn = fn;
        jobs[t].ctx = ctx;
        jobs[t].lo = lo;
        jobs[t].hi = hi;
        if (pthread_create(&th[t], NULL, job_main, &jobs[t]) != 0) {
            job_main(&jobs[t]); /* run inline if a thread cannot start */
            th[t] = (pthread_t)0;
        }
        started = t + 1;
    }
    for (int t = 0; t < started; ++t)
        if (th[t]) pthread_join(th[t], NULL);
    free(th);
    free(jobs);
}

/* ---- normal fills ---------------------------------------------------------- */

typedef struct {
    uint64_t key, tid, start;
    double mean, std;
    int dtype; /* 0 = fp32, 1 = bf16 */
    void *out;
} normal_ctx;

static void normal_range(void *p, uint64_t lo, uint64_t hi) {
    normal_ctx *c = (normal_ctx *)p;
    for (uint64_t i = lo; i < hi; ++i) {
        double v = c->mean + c->std * normal_at(c->key, c->tid, c->start + i);
        if (c->dtype == 0)
            ((float *)c->out)[i] = (float)v;
        else
            ((uint16_t *)c->out)[i] = bf16_bits_rne(v);
    }
}

/* out[i] = storage(mean + std * N_i) for elements start .. start+n-1 of tensor tid */
void synth_normal(uint64_t seed, uint64_t tid, uint64_t start, uint64_t n, double mean,
                  double std, int dtype, void *out, int nthreads) {
    normal_ctx c = {stream_key(seed), tid, start, mean, std, dtype, out};
    parallel_range(normal_range, &c, n, nthreads);
}

/* ---- INT8 per-row quantised rows ------------------------------------------ */

typedef struct {
    uint64_t key, tid, cols;
    double std;
    int8_t *q;
    float *scale;
} int8_ctx;

static void int8_rows_range(void *p, uint64_t lo, uint64_t hi) {
    int8_ctx *c = (int8_ctx *)p;
    double *row = (double *)malloc(sizeof(double) * c->cols);
    for (uint64_t r = lo; r < hi; ++r) {
        float amax = 0.0f;
        for (uint64_t k = 0; k < c->cols; ++k) {
            double v = c->std * normal_at(c->key, c->tid, r * c->cols + k);
            row[k] = bf16_bits_to_double(bf16_bits_rne(v));
            float a = (float)fabs(row[k]);
            if (a > amax) amax = a;
        }
        float s = amax / 127.0f;
        c->scale[r] = s;
        for (uint64_t k = 0; k < c->cols; ++k) {
            int8_t q = 0;
            if (s != 0.0f) {
                double t = nearbyint(row[k] / (double)s);
                if (t > 127.0) t = 127.0;
                if (t < -127.0) t = -127.0;
                q = (int8_t)t;
            }
            c->q[r * c->cols + k] = q;
        }
    }
    free(row);
}

static void parallel_rows(range_fn fn, void *ctx, uint64_t rows, int nthreads);

void synth_int8_rows(uint64_t seed, uint64_t tid, uint64_t rows, uint64_t cols, double std,
                     int8_t *q, float *scale, int nthreads) {
    int8_ctx c = {stream_key(seed), tid, cols, std, q, scale};
    parallel_rows(int8_rows_range, &c, rows, nthreads);
}

/* rows are independent; partition rows (not elements) */
static void parallel_rows(range_fn fn, void *ctx, uint64_t rows, int nthreads) {
    if (nthreads < 1) nthreads = 1;
    if ((uint64_t)nthreads > rows) nthreads = (int)rows;
    if (nthreads <= 1) {
        fn(ctx, 0, rows);
        return;
    }
    pthread_t *th = (pthread_t *)malloc(sizeof(pthread_t) * (size_t)nthreads);
    job_t *jobs = (job_t *)malloc(sizeof(job_t) * (size_t)nthreads);
    uint64_t chunk = (rows + (uint64_t)nthreads - 1) / (uint64_t)nthreads;
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        uint64_t lo = (uint64_t)t * chunk, hi = lo + chunk;
        if (lo >= rows) break;
        if (hi > rows) hi = rows;
        jobs[t].fn = fn;
        jobs[t].ctx = ctx;
        jobs[t].lo = lo;
        jobs[t].hi = hi;
        if (pthread_create(&th[t], NULL, job_main, &jobs[t]) != 0) {
            job_main(&jobs[t]);
            th[t] = (pthread_t)0;
        }
        started = t + 1;
    }
    for (int t = 0; t < started; ++t)
        if (th[t]) pthread_join(th[t], NULL);
    free(th);
    free(jobs);
}

/* ---- integers --------------------------------------------------------------- */

/* out[i] = lo + floor(u_i * (hi - lo + 1)), u_i uniform [0,1) from counter (tid<<41)+i */
void synth_uniform_int(uint64_t seed, uint64_t tid, uint64_t n, int64_t lo, int64_t hi,
                       int32_t *out) {
    uint64_t key = stream_key(seed);
    double span = (double)(hi - lo + 1);
    for (uint64_t i = 0; i < n; ++i) {
        int64_t v = lo + (int64_t)floor(u01(draw_u64(key, tensor_base(tid) + i)) * span);
        if (v > hi) v = hi;
        out[i] = (int32_t)v;
    }
}

/* n distinct integers in [lo, hi]: successive uniform draws, repeats skipped. */
int synth_distinct_int(uint64_t seed, uint64_t tid, uint64_t n, int64_t lo, int64_t hi,
                       int32_t *out) {
    if ((uint64_t)(hi - lo + 1) < n) return -1;
    uint64_t key = stream_key(seed);
    double span = (double)(hi - lo + 1);
    uint64_t got = 0;
    for (uint64_t c = 0; got < n; ++c) {
        int64_t v = lo + (int64_t)floor(u01(draw_u64(key, tensor_base(tid) + c)) * span);
        if (v > hi) v = hi;
        int dup = 0;
        for (uint64_t j = 0; j < got; ++j)
            if (out[j] == (int32_t)v) { dup = 1; break; }
        if (!dup) out[got++] = (int32_t)v;
    }
    return 0;
}

/* raw 64-bit draw, exposed for tests of the stream definition */
uint64_t synth_draw_u64(uint64_t seed, uint64_t ctr) { return draw_u64(stream_key(seed), ctr); }

/* ---- Q8_0 block-quantised rows ---------------------------------------------
 * A checkpoint's Q8_0 rows, made from an fp32 N(0, std) draw: per block of 32,
 * d = max|w| / 127 stored as fp16 (round to nearest even), codes
 * round(w / d) clipped to [-127, 127]; 34 bytes per block (d little-endian,
 * then the codes). */

/* fp16 bits of a finite v >= 0, round to nearest even */
static uint16_t half_bits_rne(double v) {
    if (v == 0.0) return 0;
    int e;
    double m = frexp(v, &e); /* v = m * 2^e, m in [0.5, 1) */
    int E = e - 1 + 15;      /* biased exponent of 1.xxx * 2^(e-1) */
    if (E >= 1) {
        double r = nearbyint(ldexp(m, 11)); /* 11 significant bits */
        if (r == 2048.0) {
            r = 1024.0;
            E += 1;
        }
        if (E >= 31) return 0x7C00;
        return (uint16_t)((E << 10) | ((int)r - 1024));
    }
    return (uint16_t)nearbyint(ldexp(v, 24)); /* subnormal (1024 is the smallest normal) */
}

static double half_bits_value(uint16_t h) {
    int e = (h >> 10) & 31, m = h & 1023;
    return e == 0 ? ldexp((double)m, -24) : ldexp((double)(1024 + m), e - 25);
}

typedef struct {
    uint64_t key, tid, cols;
    double std;
    uint8_t *out;
} q8_ctx;

static void q8_rows_range(void *p, uint64_t lo, uint64_t hi) {
    q8_ctx *c = (q8_ctx *)p;
    const uint64_t nb = c->cols / 32;
    for (uint64_t r = lo; r < hi; ++r) {
        for (uint64_t b = 0; b < nb; ++b) {
            float w[32];
            double amax = 0.0;
            for (int i = 0; i < 32; ++i) {
                w[i] = (float)(c->std * normal_at(c->key, c->tid, r * c->cols + b * 32 + (uint64_t)i));
                if (fabs((double)w[i]) > amax) amax = fabs((double)w[i]);
            }
            uint16_t dh = half_bits_rne(amax / 127.0);
            double d = half_bits_value(dh);
            uint8_t *blk = c->out + (r * nb + b) * 34;
            blk[0] = (uint8_t)(dh & 0xFF);
            blk[1] = (uint8_t)(dh >> 8);
            for (int i = 0; i < 32; ++i) {
                double t = d > 0.0 ? nearbyint((double)w[i] / d) : 0.0;
                if (t > 127.0) t = 127.0;
                if (t < -127.0) t = -127.0;
                blk[2 + i] = (uint8_t)(int8_t)t;
            }
        }
    }
}

void synth_q8_0_rows(uint64_t seed, uint64_t tid, uint64_t rows, uint64_t cols, double std, uint8_t *out,
                     int nthreads) {
    q8_ctx c = {stream_key(seed), tid, cols, std, out};
    parallel_rows(q8_rows_range, &c, rows, nthreads);
}

/* ---- Q4_0 block-quantised rows ---------------------------------------------
 * Per block of 32 from an fp32 N(0, std) draw: m = the value of largest
 * magnitude, d = m / -8 as fp16, codes round(w / d) + 8 clipped to [0, 15];
 * 18 bytes per block: d, then byte i = code i | code (i + 16) << 4. */

static double half_bits_signed_value(uint16_t h) {
    double v = half_bits_value((uint16_t)(h & 0x7FFF));
    return (h & 0x8000) ? -v : v;
}

typedef struct {
    uint64_t key, tid, cols;
    double std;
    uint8_t *out;
} q4_ctx;

static void q4_rows_range(void *p, uint64_t lo, uint64_t hi) {
    q4_ctx *c = (q4_ctx *)p;
    const uint64_t nb = c->cols / 32;
    for (uint64_t r = lo; r < hi; ++r) {
        for (uint64_t b = 0; b < nb; ++b) {
            float w[32];
            double m = 0.0;
            for (int i = 0; i < 32; ++i) {
                w[i] = (float)(c->std * normal_at(c->key, c->tid, r * c->cols + b * 32 + (uint64_t)i));
                if (fabs((double)w[i]) > fabs(m)) m = (double)w[i];
            }
            const double dv = m / -8.0;
            uint16_t dh = half_bits_rne(fabs(dv));
            if (dv < 0) dh |= 0x8000;
            const double d = half_bits_signed_value(dh);
            uint8_t *blk = c->out + (r * nb + b) * 18;
            blk[0] = (uint8_t)(dh & 0xFF);
            blk[1] = (uint8_t)(dh >> 8);
            int code[32];
            for (int i = 0; i < 32; ++i) {
                double t = d != 0.0 ? nearbyint((double)w[i] / d) + 8.0 : 8.0;
                if (t > 15.0) t = 15.0;
                if (t < 0.0) t = 0.0;
                code[i] = (int)t;
            }
            for (int i = 0; i < 16; ++i) blk[2 + i] = (uint8_t)(code[i] | (code[i + 16] << 4));
        }
    }
}

void synth_q4_0_rows(uint64_t seed, uint64_t tid, uint64_t rows, uint64_t cols, double std, uint8_t *out,
                     int nthreads) {
    q4_ctx c = {stream_key(seed), tid, cols, std, out};
    parallel_rows(q4_rows_range, &c, rows, nthreads);
}
