// pn_small.hpp - the small kernels of the decode step (embedding, argmax,
// MoE router and combine) and the one-time set-up kernels (weight packing,
// fills, K/V scatter).  Included only by pn_lib.hip.
#pragma once
#include "pn_attn.hpp"

namespace pn {

// ---------------------------------------------------------------- small kernels

struct SlotPtrs {
    int *err[kMaxSlots];
    int pos[kMaxSlots];
};

// Sum of squares of the 16 values held by a group of 16 consecutive lanes.
__device__ __forceinline__ float group16_sumsq(float v) {
    float sq = v * v;
    sq += __shfl_xor(sq, 8, 64);
    sq += __shfl_xor(sq, 4, 64);
    sq += __shfl_xor(sq, 2, 64);
    sq += __shfl_xor(sq, 1, 64);
    return sq;
}

// x[b] = tok_embd[token[b]] (fp32 or bf16 table); a bad id uses row 0 and sets
// a flag.  Also writes the sums of squares of x per 16-element tile and the
// step's RoPE table: for rotation index i of slot b, (cos, sin) of
// pos_b * omega_i with the angle, its sine and cosine in fp64, rounded to fp32.
// One work-group of 256 threads per slot; E <= 8192.
template <int ET>
__global__ void __launch_bounds__(256) k_embed(const void *embd, const int *tokens, float *x, int E,
                                                 int V, SlotPtrs sp, float2 *rope, const double *omega,
                                                 int D, float *ssp, int ssp_ld) {
    const int b = blockIdx.x, tid = threadIdx.x;
    int tok = tokens[b];
    if (tok < 0 || tok >= V) {
        if (tid == 0) atomicOr(sp.err[b], ERR_TOKEN);
        tok = 0;
    }
    // 32 consecutive elements per thread, loaded before any store
    constexpr int EPT = 32;
    float v[EPT];
    const int k0 = tid * EPT;
    if (k0 < E) {
        if constexpr (ET == 1) {
            const u32x4 *src = reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint16_t *>(embd) +
                                                               (long long)tok * E + k0);
            u32x4 w[EPT / 8];
#pragma unroll
            for (int q = 0; q < EPT / 8; ++q) w[q] = (k0 + 8 * q < E) ? src[q] : u32x4{0, 0, 0, 0};
#pragma unroll
            for (int q = 0; q < EPT / 8; ++q)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[8 * q + 2 * e] = __uint_as_float(w[q][e] << 16);
                    v[8 * q + 2 * e + 1] = __uint_as_float(w[q][e] & 0xFFFF0000u);
                }
        } else {
            const f32x4 *src = reinterpret_cast<const f32x4 *>(reinterpret_cast<const float *>(embd) +
                                                               (long long)tok * E + k0);
            f32x4 w[EPT / 4];
#pragma unroll
            for (int q = 0; q < EPT / 4; ++q) w[q] = (k0 + 4 * q < E) ? src[q] : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < EPT / 4; ++q)
#pragma unroll
                for (int e = 0; e < 4; ++e) v[4 * q + e] = w[q][e];
        }
#pragma unroll
        for (int q = 0; q < EPT / 4; ++q)
            if (k0 + 4 * q < E)
                *reinterpret_cast<f32x4 *>(x + (long long)b * E + k0 + 4 * q) =
                    f32x4{v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]};
        // two 16-element tiles per thread
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if (k0 + 16 * h < E) {
                float sq = 0.f;
#pragma unroll
                for (int e = 0; e < 16; ++e) sq += v[16 * h + e] * v[16 * h + e];
                ssp[(long long)b * ssp_ld + (k0 >> 4) + h] = sq;
            }
        }
    }
    for (int i = tid; i < D / 2; i += 256) {
        const double phi = (double)sp.pos[b] * omega[i];
        double sn, cs;
        sincos(phi, &sn, &cs);
        rope[(long long)b * (D / 2) + i] = make_float2((float)cs, (float)sn);
    }
}

// omega_i = theta^(-2i/D) in fp64, once per model.
__global__ void __launch_bounds__(64) k_omega(double *omega, int D, double theta) {
    for (int i = threadIdx.x; i < D / 2; i += 64) omega[i] = pow(theta, -2.0 * (double)i / (double)D);
}

// argmax[b] over the LM head's per-block partials (value, lowest index on ties).
// Up to 16 partials per thread are loaded before any comparison.
__global__ void __launch_bounds__(256) k_argmax(const float *val, const int *idx, int nwg, int nb, int *out) {
    const int b = blockIdx.x, tid = threadIdx.x;
    float best = 0.f;
    int bi = -1;
    for (int base = 0; base < nwg; base += 256 * 16) {
        float vv[16];
        int ii[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int w = base + tid + 256 * u;
            ii[u] = w < nwg ? idx[(long long)w * nb + b] : -1;
            vv[u] = w < nwg ? val[(long long)w * nb + b] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const int i = ii[u];
            const float v = vv[u];
            if (i < 0) continue;
            if (bi < 0 || v > best || (v == best && i < bi)) { best = v; bi = i; }
        }
    }
    __shared__ float sv[256];
    __shared__ int si[256];
    sv[tid] = best;
    si[tid] = bi;
    lds_barrier();
    for (int o = 128; o > 0; o >>= 1) {
        if (tid < o) {
            const float v = sv[tid + o];
            const int i = si[tid + o];
            if (i >= 0 && (si[tid] < 0 || v > sv[tid] || (v == sv[tid] && i < si[tid]))) {
                sv[tid] = v;
                si[tid] = i;
            }
        }
        lds_barrier();
    }
    if (tid == 0 && out) out[b] = si[0];
}

// MoE router of one slot: xn = round_act(RMSNorm(x)*g) with the norm from the
// per-tile sums of squares; r = W_r xn; top-k by fp32 logit (ties to the lower
// index); weights = softmax over the chosen logits.  256 threads; E <= 8192,
// E a multiple of 8.
template <int RT, int AT>
__global__ void __launch_bounds__(256) k_router(const float *x, const float *gain, const void *wr, int E,
                                                 int n_expert, int k_used, float eps, const float *ssp, int ssp_ld,
                                                 int ssp_n, int *ids, float *wts, int *ids_log) {
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    extern __shared__ float xs[];  // [E]
    __shared__ float red4[4];
    __shared__ float r[64];
    // One load of 8 router weights (k .. k+7 of expert e): a 16-byte vector of
    // bf16, or two of fp32; zeros past E.
    struct WRaw { u32x4 v[2]; };
    auto load_raw = [&](int e, int k) -> WRaw {
        WRaw q{};
        if (k < E) {
            if constexpr (RT == 1) {
                q.v[0] = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const uint16_t *>(wr) + (long long)e * E + k);
            } else {
                const u32x4 *p = reinterpret_cast<const u32x4 *>(reinterpret_cast<const float *>(wr) + (long long)e * E + k);
                q.v[0] = p[0];
                q.v[1] = p[1];
            }
        }
        return q;
    };
    auto expand = [&](const WRaw &q, float (&o)[8]) {
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            if constexpr (RT == 1) {
                o[2 * h] = __uint_as_float(q.v[0][h] << 16);
                o[2 * h + 1] = __uint_as_float(q.v[0][h] & 0xFFFF0000u);
            } else {
                o[h] = __uint_as_float(q.v[0][h]);
                o[4 + h] = __uint_as_float(q.v[1][h]);
            }
        }
    };
    // The weights do not depend on x: the first 4096 inputs of this wave's
    // first two experts (w and w + 4) are loaded before x, so their round trip
    // overlaps the norm's.
    constexpr int KC = 64 * 8 * 8;  // inputs per pass of a wave
    WRaw pre0[8], pre1[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
        pre0[u] = w < n_expert ? load_raw(w, (lane + 64 * u) * 8) : WRaw{};
        pre1[u] = w + 4 < n_expert ? load_raw(w + 4, (lane + 64 * u) * 8) : WRaw{};
    }
    const float *xr = x + (long long)b * E;
    // this thread's 32 elements of x and gain, and a share of the sums of squares
    constexpr int EPT = 32;
    const int k0 = tid * EPT;
    f32x4 xv[EPT / 4], gv[EPT / 4];
#pragma unroll
    for (int q = 0; q < EPT / 4; ++q) {
        const bool in = k0 + 4 * q < E;
        xv[q] = in ? reinterpret_cast<const f32x4 *>(xr + k0)[q] : f32x4{0.f, 0.f, 0.f, 0.f};
        gv[q] = in ? reinterpret_cast<const f32x4 *>(gain + k0)[q] : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float ss = 0.f;
    for (int i = tid; i < ssp_n; i += 256) ss += ssp[(long long)b * ssp_ld + i];
    ss = block_sum<4>(ss, red4);
    const float rinv = 1.0f / sqrtf(ss / (float)E + eps);
#pragma unroll
    for (int q = 0; q < EPT / 4; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int k = k0 + 4 * q + e;
            if (k < E) {
                float v = (xv[q][e] * rinv) * gv[q][e];
                if (AT == AT_BF16) v = bf16_round(v);
                xs[k] = v;
            }
        }
    lds_barrier();
    // expert e on wave e % 4: lanes stride over E in 8-element groups; the
    // first pass of the first two takes the weights loaded above
    auto dot = [&](int e, const WRaw (*pre)[8]) -> float {
        float acc = 0.f;
        for (int base = 0; base < E; base += KC) {
            float wv[8][8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int k = base + (lane + 64 * u) * 8;
                const WRaw q = (pre && base == 0) ? (*pre)[u] : load_raw(e, k);
                expand(q, wv[u]);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int k = base + (lane + 64 * u) * 8;
                if (k < E)
#pragma unroll
                    for (int h = 0; h < 8; ++h) acc = fmaf(wv[u][h], xs[k + h], acc);
            }
        }
        return wave_sum(acc);
    };
    if (w < n_expert) {
        const float a = dot(w, &pre0);
        if (lane == 0) r[w] = a;
    }
    if (w + 4 < n_expert) {
        const float a = dot(w + 4, &pre1);
        if (lane == 0) r[w + 4] = a;
    }
    for (int e = w + 8; e < n_expert; e += 4) {
        const float a = dot(e, nullptr);
        if (lane == 0) r[e] = a;
    }
    lds_barrier();
    if (tid == 0) {
        unsigned long long used = 0ull;
        int sel[8];
        for (int a2 = 0; a2 < k_used; ++a2) {
            int best = -1;
            for (int e = 0; e < n_expert; ++e) {
                if ((used >> e) & 1ull) continue;
                if (best < 0 || r[e] > r[best]) best = e;
            }
            used |= 1ull << best;
            sel[a2] = best;
        }
        const float mx = r[sel[0]];
        float den = 0.f;
        float pe[8];
        for (int a2 = 0; a2 < k_used; ++a2) {
            pe[a2] = expf(r[sel[a2]] - mx);
            den += pe[a2];
        }
        for (int a2 = 0; a2 < k_used; ++a2) {
            ids[b * k_used + a2] = sel[a2];
            wts[b * k_used + a2] = pe[a2] / den;
            if (ids_log) ids_log[b * k_used + a2] = sel[a2];  // the caller's routing record
        }
    }
}

// x[b][r] += sum_k w[b][k] * y[b*k_used + k][r], and the new per-tile sums of squares.
__global__ void __launch_bounds__(256) k_moe_combine(float *x, const float *y, const float *wts, int E,
                                                      int k_used, float *ssp, int ssp_ld) {
    const int b = blockIdx.y;
    const int r = blockIdx.x * 256 + threadIdx.x;
    float xn = 0.f;
    if (r < E) {
        float s = 0.f;
        for (int k = 0; k < k_used; ++k) s += wts[b * k_used + k] * y[((long long)b * k_used + k) * E + r];
        xn = x[(long long)b * E + r] + s;
        x[(long long)b * E + r] = xn;
    }
    const float sq = group16_sumsq(xn);
    if ((threadIdx.x & 15) == 0 && r < E) ssp[(long long)b * ssp_ld + (r >> 4)] = sq;
}

// Source row of stored row r when each head's d rows are put in rotation-pair
// order for the NeoX RoPE: stored rows 2i, 2i+1 of a head are its rows i and
// i + d/2, which the half-split RoPE rotates together (d = 0: no reordering).
// q.k is a sum over dims, so q and k in this order give the same scores.
__host__ __device__ inline int neox_src(int r, int d) {
    if (d <= 0) return r;
    const int h = r % d;
    return r - h + (h >> 1) + (h & 1) * (d >> 1);
}

// Re-lay a row-major matrix [N][K] (element size ES) into 1 KiB tiles.
// Int8 codes are stored biased (u = q + 128); padding is the code of 0.
template <int ES>
__global__ void __launch_bounds__(256) k_pack(const uint8_t *src, int N, int K, int KT, int n_tiles,
                                               uint8_t *dst, int neox_d) {
    constexpr int EPL = 16 / ES;  // elements per lane chunk
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long total = (long long)n_tiles * KT * 64;
    if (i >= total) return;
    const int lane = (int)(i & 63);
    const long long tileid = i >> 6;
    const int nt = (int)(tileid / KT), kt = (int)(tileid % KT);
    const int row = nt * 16 + (lane & 15);
    const int k0 = kt * EPL * 4 + (lane >> 4) * EPL;
    uint8_t out[16];
#pragma unroll
    for (int e = 0; e < EPL; ++e) {
        const int k = k0 + e;
        const bool in = row < N && k < K;
#pragma unroll
        for (int bb = 0; bb < ES; ++bb) {
            uint8_t v = in ? src[((long long)neox_src(row, neox_d) * K + k) * ES + bb] : 0;
            if (ES == 1) v = (uint8_t)(v ^ 0x80u);
            out[e * ES + bb] = v;
        }
    }
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        o[q] = (uint32_t)out[4 * q] | ((uint32_t)out[4 * q + 1] << 8) | ((uint32_t)out[4 * q + 2] << 16) |
               ((uint32_t)out[4 * q + 3] << 24);
    reinterpret_cast<u32x4 *>(dst)[i] = o;
}

// Q8_0 rows (per 32-weight block: fp16 scale, 32 int8 codes; K a multiple of
// 32) into 1 KiB tiles of biased codes (u = q + 128) whose 16 bytes per lane
// follow blk_pos, and 64-byte scale tiles holding each row's two block scales.
// Blocks past K read as code 0 with scale 0.
__global__ void __launch_bounds__(256) k_pack_q8(const uint8_t *src, int N, int K, int KT, int n_tiles,
                                                  uint8_t *dst, uint8_t *sdst, int neox_d) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long total = (long long)n_tiles * KT * 64;
    if (i >= total) return;
    const int lane = (int)(i & 63);
    const long long tileid = i >> 6;
    const int nt = (int)(tileid / KT), kt = (int)(tileid % KT);
    const int row = nt * 16 + (lane & 15), g = lane >> 4;
    const int nblk = K / 32;
    const uint8_t *srow = src + (long long)(row < N ? neox_src(row, neox_d) : 0) * nblk * 34;
    uint8_t out[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int k = kt * 64 + 32 * (e >> 3) + 8 * g + (e & 7);
        const int blk = k >> 5;
        const uint8_t q = (row < N && blk < nblk) ? srow[blk * 34 + 2 + (k & 31)] : 0;
        out[e] = (uint8_t)(q ^ 0x80u);
    }
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        o[q] = (uint32_t)out[4 * q] | ((uint32_t)out[4 * q + 1] << 8) | ((uint32_t)out[4 * q + 2] << 16) |
               ((uint32_t)out[4 * q + 3] << 24);
    reinterpret_cast<u32x4 *>(dst)[i] = o;
    if (g == 0) {
        uint32_t w = 0;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int blk = 2 * kt + j;
            const uint32_t d = (row < N && blk < nblk) ? (uint32_t)srow[blk * 34] | ((uint32_t)srow[blk * 34 + 1] << 8) : 0u;
            w |= d << (16 * j);
        }
        reinterpret_cast<uint32_t *>(sdst)[tileid * 16 + (lane & 15)] = w;
    }
}

// Q4_0 rows (per 32-weight block: fp16 scale, 16 bytes whose byte i holds code
// i in its low nibble and code i + 16 in its high one; K a multiple of 32) into
// 1 KiB tiles of 16 rows x 128 k, 16 bytes per lane: word j holds the 8 codes
// of the lane's elements 8j..8j+7 (blk_pos order: block j of the tile), codes
// 0..3 in the low nibbles of its bytes and 4..7 in the high ones (the layout
// the GEMM widens with two masks and byte permutes); and 128-byte scale tiles
// holding each row's four block scales.
// Blocks past K read as code 8 (weight 0) with scale 0.
__global__ void __launch_bounds__(256) k_pack_q4(const uint8_t *src, int N, int K, int KT, int n_tiles,
                                                  uint8_t *dst, uint8_t *sdst, int neox_d) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long total = (long long)n_tiles * KT * 64;
    if (i >= total) return;
    const int lane = (int)(i & 63);
    const long long tileid = i >> 6;
    const int nt = (int)(tileid / KT), kt = (int)(tileid % KT);
    const int row = nt * 16 + (lane & 15), g = lane >> 4;
    const int nblk = K / 32;
    const uint8_t *srow = src + (long long)(row < N ? neox_src(row, neox_d) : 0) * nblk * 18;
    u32x4 w = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 32; ++e) {
        const int blk = 4 * kt + (e >> 3);
        const int kb = 8 * g + (e & 7);  // k within the block
        uint32_t code = 8u;
        if (row < N && blk < nblk) {
            const uint8_t byte = srow[blk * 18 + 2 + (kb & 15)];
            code = kb < 16 ? (byte & 15u) : (uint32_t)(byte >> 4);
        }
        const int ee = e & 7;  // codes 0..3 of a word in its bytes' low nibbles, 4..7 in the high ones
        w[e >> 3] |= code << (ee < 4 ? 8 * ee : 8 * (ee - 4) + 4);
    }
    reinterpret_cast<u32x4 *>(dst)[i] = w;
    if (g == 0) {
        uint32_t sw[2] = {0u, 0u};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int blk = 4 * kt + j;
            const uint32_t d = (row < N && blk < nblk) ? (uint32_t)srow[blk * 18] | ((uint32_t)srow[blk * 18 + 1] << 8) : 0u;
            sw[j >> 1] |= d << (16 * (j & 1));
        }
        reinterpret_cast<u32x2 *>(sdst)[tileid * 16 + (lane & 15)] = u32x2{sw[0], sw[1]};
    }
}

// Store one k (w = 0: key rows) or v (w = 1: columns) head vector of a Q4 cache
// at key `key` of its page block `base` (layout as q4kv_key_bytes says).
__device__ __forceinline__ void q4kv_put(const float *src, uint8_t *base, int key, int w, int D, int lane) {
    uint16_t *sc = reinterpret_cast<uint16_t *>(base + kPage * (D / 2));
    if (w == 0) q4kv_store(src, base + key * (D / 2), 1, sc + key * (D / 32), 1, D, lane);
    else q4kv_store(src, base + key, kPage, sc + key, kPage, D, lane);
}

// Q4 KV cache: quantise the step's new k and v rows (kv_new of the QKV
// epilogue) into the pages, one wave per (row, KV head, k or v).
__global__ void __launch_bounds__(64) k_kv_q4_append(KvQ4Args a) {
    const int b = blockIdx.x, j = blockIdx.y, w = blockIdx.z, lane = threadIdx.x;
    const int pos = a.pos[b];
    const int pg = a.pt[b][pos / kPage];
    uint8_t *base = reinterpret_cast<uint8_t *>(w ? a.kvv[b] : a.kvk[b]) +
                    ((long long)pg * a.Hk + j) * kPage * q4kv_key_bytes(a.D);
    q4kv_put(a.src + (((long long)b * 2 + w) * a.Hk + j) * a.D, base, pos % kPage, w, a.D, lane);
}

// Q4 KV cache: positions pos0..pos0+n-1 of one layer from fp32 rows k, v
// [n][Hk][D], quantised as an append quantises them.
__global__ void __launch_bounds__(64) k_kv_q4_set(char *kpool, char *vpool, const int *pt, const float *k,
                                                   const float *v, int pos0, int Hk, int D) {
    const int t = blockIdx.x, j = blockIdx.y, w = blockIdx.z, lane = threadIdx.x;
    const int pos = pos0 + t;
    uint8_t *base = reinterpret_cast<uint8_t *>(w ? vpool : kpool) +
                    ((long long)pt[pos / kPage] * Hk + j) * kPage * q4kv_key_bytes(D);
    q4kv_put((w ? v : k) + ((long long)t * Hk + j) * D, base, pos % kPage, w, D, lane);
}

__global__ void __launch_bounds__(256) k_copy_rows_f32(float *dst, const float *src, int n, int neox_d) {
    const int r = blockIdx.x * 256 + threadIdx.x;
    if (r < n) dst[r] = src[neox_src(r, neox_d)];
}

__global__ void __launch_bounds__(256) k_fill32(uint32_t *p, long long n, uint32_t v) {
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256)
        p[i] = v;
}

// A plain streaming read of n16 16-byte words: the measured read ceiling of
// HBM that the decode kernels are held to.  Each pass a work-group reads 256 *
// 8 consecutive words (32 KiB, eight nontemporal loads in flight per thread),
// then strides by the grid.  The words are folded into one xor per wave that
// is written only when it equals an arbitrary constant (almost never), so no
// load is dead and the waves do not serialise on one atomic.
__global__ void __launch_bounds__(256) k_stream_read(const u32x4 *src, long long n16, unsigned *sink) {
    constexpr int U = 8;
    const long long stride = (long long)gridDim.x * 256 * U;
    unsigned acc = 0;
    for (long long base = (long long)blockIdx.x * 256 * U + threadIdx.x; base < n16; base += stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const long long i = base + (long long)u * 256;
            v[u] = i < n16 ? __builtin_nontemporal_load(src + i) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
    if ((threadIdx.x & 63) == 0 && acc == 0x9E3779B9u) atomicXor(sink, acc);
}

__global__ void __launch_bounds__(256) k_iota(int *p, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = i;
}

__global__ void __launch_bounds__(256) k_copy_bytes(uint8_t *dst, const uint8_t *src, long long n) {
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256)
        dst[i] = src[i];
}

// Page-table writes of pooled states: entry idx[i] of table pt[i] = val[i].
constexpr int kPageSetMax = 64;
struct PageSet {
    int *pt[kPageSetMax];
    int idx[kPageSetMax], val[kPageSetMax];
    int n;
};
__global__ void __launch_bounds__(kPageSetMax) k_set_pages(PageSet p) {
    const int i = threadIdx.x;
    if (i < p.n) p.pt[i][p.idx[i]] = p.val[i];
}

// Zero pages of a shared pool before they join a state: page val[y] of every
// layer's K (z even) and V (z odd) pools, 16 bytes per thread.
__global__ void __launch_bounds__(256) k_zero_pages(char *kbase, char *vbase, size_t layer_bytes,
                                                     long long page_words, PageSet p) {
    const int layer = blockIdx.z >> 1;
    char *pool = ((blockIdx.z & 1) ? vbase : kbase) + (size_t)layer * layer_bytes;
    uint4 *pg = reinterpret_cast<uint4 *>(pool) + (long long)p.val[blockIdx.y] * page_words;
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < page_words; i += (long long)gridDim.x * 256)
        pg[i] = make_uint4(0u, 0u, 0u, 0u);
}

// Scatter K and V of positions pos0..pos0+n-1 ([n][Hk][D]) into the pages of one
// layer (each head's block of a page laid out as kv_k_off / kv_v_off say).
template <int ES>
__global__ void __launch_bounds__(256) k_set_kv(char *kpool, char *vpool, const int *pt, const char *k,
                                                 const char *v, int pos0, int n, int Hk, int D, int neox_d) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long total = (long long)n * Hk * D;
    if (i >= total) return;
    const int d = (int)(i % D);
    const int j = (int)((i / D) % Hk);
    const int t = (int)(i / ((long long)D * Hk));
    const int p = pos0 + t;
    const long long hb = ((long long)pt[p / kPage] * Hk + j) * kPage * D;
    const long long koff = hb + kv_k_off(ES == 2, p % kPage, d, D);
    const long long voff = hb + kv_v_off(ES == 2, p % kPage, d, D);
    const long long ki = i - d + neox_src(d, neox_d);  // cached dim d holds source dim neox_src(d)
    if constexpr (ES == 2) {
        reinterpret_cast<uint16_t *>(kpool)[koff] = reinterpret_cast<const uint16_t *>(k)[ki];
        reinterpret_cast<uint16_t *>(vpool)[voff] = reinterpret_cast<const uint16_t *>(v)[i];
    } else {
        reinterpret_cast<float *>(kpool)[koff] = reinterpret_cast<const float *>(k)[ki];
        reinterpret_cast<float *>(vpool)[voff] = reinterpret_cast<const float *>(v)[i];
    }
}

}  // namespace pn
