// pn_kernels.hpp - HIP kernels (gfx950) of the one-token decode step.
//
// Weight tiles.  Every matrix W[N][K] (row-major, out x in) is re-laid into
// 1 KiB tiles of 16 rows: tile (nt, kt) holds rows nt*16..nt*16+15 and TK
// consecutive k, stored as 64 lanes x 16 bytes.  Lane l holds row nt*16 +
// (l & 15) and k-group (l >> 4), i.e. the 16 bytes of k in
// [kt*TK + (l>>4)*TK/4, +TK/4).  TK is 16 for fp32, 32 for bf16 and 64 for
// int8 (stored biased, u = q + 128).  Tiles of one row block are contiguous
// in kt, so a wave streaming one row block reads whole KiB blocks.  The lane
// layout is the B operand of the 16x16 MFMA instructions, so the same tiles
// feed batch 1 and batched slots.
//
// A operand (activations).  Up to 16 rows.  A row is one (piece, slot) pair:
// with fp32 activations and bf16 weights each fp32 value is split into three
// bf16 pieces whose sum is exactly the fp32 value, so the bf16 MFMA computes
// an fp32-exact product; otherwise a row is a slot.  Int8 weights run on the
// f16 MFMA: a code u becomes the f16 1024+u by a byte permute and 1152 is
// subtracted, which leaves q exactly; the bf16 activations are converted to
// f16 (exact in the f16 normal range).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace pn {

constexpr int kPage = 64;      // tokens per KV page
constexpr int kMaxRows = 16;   // A rows of one MFMA tile
constexpr int kMaxSlots = 16;  // sequences in one batched step
constexpr int kNW = 4;         // waves per GEMM work-group
constexpr int kU = 8;          // tiles per wave per load round
constexpr int kAttnWaves = 4;  // waves per attention work-group
constexpr int kMaxG = 8;       // query heads per KV head

enum WType { WT_F32 = 0, WT_BF16 = 1, WT_I8 = 2 };
enum AType { AT_F32 = 0, AT_BF16 = 1 };
enum Pro { PRO_NORM = 0, PRO_LOAD = 1 };
enum Epi { EPI_QKV = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_LOGITS = 3, EPI_MOE_SWIGLU = 4,
           EPI_MOE_DOWN = 5 };

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__host__ __device__ constexpr int tile_k(int wt) { return wt == WT_F32 ? 16 : (wt == WT_BF16 ? 32 : 64); }
// A-fragment bytes per (k-group, row) per tile
__host__ __device__ constexpr int frag_bytes(int wt) { return wt == WT_I8 ? 32 : 16; }

// ---------------------------------------------------------------- small helpers

__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}
__device__ __forceinline__ float bf16_round(float f) { return __uint_as_float(bf16_rne_bits(f) << 16); }
__device__ __forceinline__ float bf16_bits_f32(uint32_t h) { return __uint_as_float(h << 16); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ float readlane_f(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// the sequence-level error flags of a state
enum { ERR_TOKEN = 1, ERR_NAN = 2 };

// ---------------------------------------------------------------- GEMM

struct GemmArgs {
    const uint8_t *w;       // packed tiles of matrix 0 (of expert 0)
    const uint8_t *w2;      // pair mode: packed tiles of matrix 1
    const float *sc;        // int8 row scales of matrix 0 (padded to tiles), else null
    const float *sc2;
    long long ew_stride;    // bytes between experts' packed matrices
    long long es_stride;    // floats between experts' scales
    int N;                  // logical rows (per matrix)
    int n_tiles;            // 16-row tiles per matrix
    int KT;                 // k tiles
    int K;                  // logical K
    int kc;                 // k chunks (grid.y)
    int ktc;                // tiles per chunk
    int B;                  // dense: slots
    const float *x;         // PRO_NORM: residual [slot][K]
    const float *gain;      // PRO_NORM: [K]
    float eps;
    const void *a;          // PRO_LOAD: activation rows [row][lda]
    int lda;
    const int *route_ids;   // MoE: [slot][n_used] expert ids
    int n_slots;            // MoE: slots in the step
    int n_used;
    float *part;            // split-K partial tiles
    int *cnt;               // split-K arrival counters (self-resetting)
    float *out_f32;         // RESID: x; LOGITS: logits (nullable); MOE_DOWN: y rows
    void *out_act;          // SWIGLU / MOE_SWIGLU: hidden rows (act dtype)
    int ld_out;
    float *q_out;           // QKV: q [slot][Hq*D]
    int Hq, Hk, D;
    int kv_es;              // QKV: bytes per cached element (2 = bf16, 4 = fp32)
    double theta;
    float *am_val;          // LOGITS: per-WG best value [wg][slot]
    int *am_idx;
    int *err[kMaxSlots];    // per slot error flags
    int pos[kMaxSlots];
    char *kvk[kMaxSlots];   // per slot: K pool of this layer
    char *kvv[kMaxSlots];
    const int *pt[kMaxSlots];
};

template <int WT>
__device__ __forceinline__ void mfma_tile(f32x4 &acc, const u32x4 &wv, const uint8_t *afrag, bool live) {
    if constexpr (WT == WT_BF16) {
        u32x4 av = live ? *reinterpret_cast<const u32x4 *>(afrag) : u32x4{0, 0, 0, 0};
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                      __builtin_bit_cast(bf16x8, wv), acc, 0, 0, 0);
    } else if constexpr (WT == WT_F32) {
        f32x4 av = live ? *reinterpret_cast<const f32x4 *>(afrag) : f32x4{0.f, 0.f, 0.f, 0.f};
        f32x4 bw = __builtin_bit_cast(f32x4, wv);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[0], bw[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[1], bw[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[2], bw[2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[3], bw[3], acc, 0, 0, 0);
    } else {
        u32x4 a0 = live ? *reinterpret_cast<const u32x4 *>(afrag) : u32x4{0, 0, 0, 0};
        u32x4 a1 = live ? *reinterpret_cast<const u32x4 *>(afrag + 16) : u32x4{0, 0, 0, 0};
        const f16x2 off = {(_Float16)1152.0f, (_Float16)1152.0f};
        u32x4 b0, b1;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            uint32_t lo = __builtin_amdgcn_perm(0x64646464u, wv[i], 0x04010400u);
            uint32_t hi = __builtin_amdgcn_perm(0x64646464u, wv[i], 0x04030402u);
            f16x2 flo = __builtin_bit_cast(f16x2, lo) - off;
            f16x2 fhi = __builtin_bit_cast(f16x2, hi) - off;
            uint32_t ulo = __builtin_bit_cast(uint32_t, flo), uhi = __builtin_bit_cast(uint32_t, fhi);
            if (i < 2) { b0[2 * i] = ulo; b0[2 * i + 1] = uhi; }
            else { b1[2 * (i - 2)] = ulo; b1[2 * (i - 2) + 1] = uhi; }
        }
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a0),
                                                     __builtin_bit_cast(f16x8, b0), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a1),
                                                     __builtin_bit_cast(f16x8, b1), acc, 0, 0, 0);
    }
}

// Store activation value v of (slot b, chunk-local k index kk) into the LDS A fragments.
template <int WT, int AT>
__device__ __forceinline__ void put_a(uint8_t *sa, int rows, int nb, int b, int kk, float v) {
    constexpr int TK = tile_k(WT);
    constexpr int FB = frag_bytes(WT);
    constexpr int EPG = TK / 4;  // elements per (k-group) per tile
    const int tt = kk / TK, kin = kk % TK, gq = kin / EPG, el = kin % EPG;
    if constexpr (WT == WT_F32) {
        *reinterpret_cast<float *>(sa + ((tt * 4 + gq) * rows + b) * FB + el * 4) = v;
    } else if constexpr (WT == WT_I8) {
        *reinterpret_cast<_Float16 *>(sa + ((tt * 4 + gq) * rows + b) * FB + el * 2) = (_Float16)v;
    } else if constexpr (AT == AT_BF16) {
        *reinterpret_cast<uint16_t *>(sa + ((tt * 4 + gq) * rows + b) * FB + el * 2) =
            (uint16_t)bf16_rne_bits(v);
    } else {
        // three bf16 pieces with p0 + p1 + p2 == v exactly
        float p0 = bf16_round(v);
        float r1 = v - p0;
        float p1 = bf16_round(r1);
        float p2 = bf16_round(r1 - p1);
        *reinterpret_cast<uint16_t *>(sa + ((tt * 4 + gq) * rows + b) * FB + el * 2) = (uint16_t)bf16_rne_bits(p0);
        *reinterpret_cast<uint16_t *>(sa + ((tt * 4 + gq) * rows + nb + b) * FB + el * 2) = (uint16_t)bf16_rne_bits(p1);
        *reinterpret_cast<uint16_t *>(sa + ((tt * 4 + gq) * rows + 2 * nb + b) * FB + el * 2) = (uint16_t)bf16_rne_bits(p2);
    }
}

// Block-wide deterministic sum of one float per thread (256 threads).
__device__ __forceinline__ float block_sum256(float v, float *red4) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red4[w] = v;
    __syncthreads();
    return (red4[0] + red4[1]) + (red4[2] + red4[3]);
}

// RoPE of the pair (y0, y1) at rotation index i of a head of width D, position pos.
__device__ __forceinline__ void rope_pair(float &y0, float &y1, int i, int D, int pos, double theta) {
    double w = pow(theta, -2.0 * (double)i / (double)D);
    double phi = (double)pos * w;
    double s, c;
    sincos(phi, &s, &c);
    float cf = (float)c, sf = (float)s;
    float a = y0, b = y1;
    y0 = a * cf - b * sf;
    y1 = a * sf + b * cf;
}

template <int AT>
__device__ __forceinline__ void store_act(void *base, long long idx, float v) {
    if constexpr (AT == AT_BF16)
        reinterpret_cast<uint16_t *>(base)[idx] = (uint16_t)bf16_rne_bits(v);
    else
        reinterpret_cast<float *>(base)[idx] = v;
}

template <int AT>
__device__ __forceinline__ float load_act(const void *base, long long idx) {
    if constexpr (AT == AT_BF16)
        return bf16_bits_f32(reinterpret_cast<const uint16_t *>(base)[idx]);
    else
        return reinterpret_cast<const float *>(base)[idx];
}

// Skinny GEMM Y[rows][N] = A[rows][K] * W[N][K]^T for rows <= 16, fused with a
// prologue that builds A and an epilogue that consumes Y.
// grid: x = row-block (NTW tiles), y = k chunk, z = expert (MoE) ; 256 threads.
// NTW = 2 with PAIR: tile x of matrices w and w2 (gate/up).  NTW = 2 without
// PAIR: tiles 2x and 2x+1 of w.
template <int WT, int AT, int PRO, int EPI, int NTW, bool PAIR>
__global__ void __launch_bounds__(256) k_gemm(GemmArgs g) {
    constexpr int TK = tile_k(WT);
    constexpr int FB = frag_bytes(WT);
    constexpr int PIECES = (WT == WT_BF16 && AT == AT_F32) ? 3 : 1;
    constexpr bool MOE = (EPI == EPI_MOE_SWIGLU || EPI == EPI_MOE_DOWN);
    extern __shared__ __align__(16) uint8_t smem[];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int bx = blockIdx.x, chunk = blockIdx.y, ex = blockIdx.z;

    __shared__ int s_ent[kMaxSlots];   // MoE: entry (slot*n_used + k) of each gathered row
    __shared__ int s_nb;
    __shared__ float s_rinv[kMaxSlots];
    __shared__ float s_red4[4];
    __shared__ int s_last;

    if constexpr (MOE) {
        if (tid == 0) {
            int n = 0;
            for (int b = 0; b < g.n_slots; ++b)
                for (int k = 0; k < g.n_used; ++k)
                    if (g.route_ids[b * g.n_used + k] == ex) s_ent[n++] = b * g.n_used + k;
            s_nb = n;
        }
        __syncthreads();
    }
    const int nb = MOE ? s_nb : g.B;
    if (nb == 0) return;
    const int rows = nb * PIECES;

    const int c0 = chunk * g.ktc;
    const int c1 = min(g.KT, c0 + g.ktc);
    const int clen = c1 - c0;
    const int per = (clen + kNW - 1) / kNW;
    const int wt0 = c0 + min(clen, wave * per);
    const int wt1 = c0 + min(clen, (wave + 1) * per);

    // matrix tile bases
    const uint8_t *wbase[NTW];
    bool wlive[NTW];
#pragma unroll
    for (int mt = 0; mt < NTW; ++mt) {
        int nt = PAIR ? bx : bx * NTW + mt;
        wlive[mt] = nt < g.n_tiles;
        const uint8_t *m = (PAIR && mt == 1) ? g.w2 : g.w;
        wbase[mt] = m + (long long)ex * g.ew_stride + ((long long)nt * g.KT) * 1024 + lane * 16;
    }

    // first load round, issued before the prologue so it overlaps it
    u32x4 wr[NTW][kU];
    int t = wt0;
    {
        int n = min(kU, wt1 - t);
#pragma unroll
        for (int i = 0; i < kU; ++i)
#pragma unroll
            for (int mt = 0; mt < NTW; ++mt)
                if (i < n && wlive[mt])
                    wr[mt][i] = __builtin_nontemporal_load(
                        reinterpret_cast<const u32x4 *>(wbase[mt] + (long long)(t + i) * 1024));
    }

    // ---- prologue: A fragments of this chunk into LDS
    uint8_t *sa = smem;
    const int klo = c0 * TK;
    const int klen = clen * TK;
    if constexpr (PRO == PRO_NORM) {
        for (int b = 0; b < nb; ++b) {
            const int sb = MOE ? s_ent[b] / g.n_used : b;
            const float *xr = g.x + (long long)sb * g.K;
            float ss = 0.f;
            for (int k = tid; k < g.K; k += 256) ss += xr[k] * xr[k];
            ss = block_sum256(ss, s_red4);
            if (tid == 0) s_rinv[b] = 1.0f / sqrtf(ss / (float)g.K + g.eps);
        }
        __syncthreads();
        for (int idx = tid; idx < nb * klen; idx += 256) {
            const int b = idx / klen, kk = idx - b * klen, k = klo + kk;
            const int sb = MOE ? s_ent[b] / g.n_used : b;
            float v = 0.f;
            if (k < g.K) {
                v = (g.x[(long long)sb * g.K + k] * s_rinv[b]) * g.gain[k];
                if (AT == AT_BF16) v = bf16_round(v);
            }
            put_a<WT, AT>(sa, rows, nb, b, kk, v);
        }
    } else {
        for (int idx = tid; idx < nb * klen; idx += 256) {
            const int b = idx / klen, kk = idx - b * klen, k = klo + kk;
            const long long ar = MOE ? s_ent[b] : b;
            float v = (k < g.K) ? load_act<AT>(g.a, ar * g.lda + k) : 0.f;
            put_a<WT, AT>(sa, rows, nb, b, kk, v);
        }
    }
    __syncthreads();

    // ---- main loop
    f32x4 acc[NTW];
#pragma unroll
    for (int mt = 0; mt < NTW; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int am = lane & 15, ag = lane >> 4;
    const bool alive = am < rows;
    while (t < wt1) {
        const int n = min(kU, wt1 - t);
#pragma unroll
        for (int i = 0; i < kU; ++i) {
            if (i < n) {
                const uint8_t *af = sa + (((t - c0 + i) * 4 + ag) * rows + am) * FB;
#pragma unroll
                for (int mt = 0; mt < NTW; ++mt)
                    if (wlive[mt]) mfma_tile<WT>(acc[mt], wr[mt][i], af, alive);
            }
        }
        t += n;
        if (t < wt1) {
            const int n2 = min(kU, wt1 - t);
#pragma unroll
            for (int i = 0; i < kU; ++i)
#pragma unroll
                for (int mt = 0; mt < NTW; ++mt)
                    if (i < n2 && wlive[mt])
                        wr[mt][i] = __builtin_nontemporal_load(
                            reinterpret_cast<const u32x4 *>(wbase[mt] + (long long)(t + i) * 1024));
        }
    }

    // ---- reduce the waves' tiles: red[wave][mt][m][n]
    const int abytes = g.ktc * 4 * rows * FB;
    float *red = reinterpret_cast<float *>(smem + ((abytes + 255) & ~255));
    float *C = red + kNW * NTW * 256;
#pragma unroll
    for (int mt = 0; mt < NTW; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[(wave * NTW + mt) * 256 + (4 * ag + i) * 16 + am] = acc[mt][i];
    __syncthreads();
    for (int idx = tid; idx < NTW * 256; idx += 256) {
        float s = 0.f;
#pragma unroll
        for (int w = 0; w < kNW; ++w) s += red[w * NTW * 256 + idx];
        C[idx] = s;
    }

    if (g.kc > 1) {
        const long long tg = (long long)ex * gridDim.x + bx;
        float *mine = g.part + (tg * g.kc + chunk) * (NTW * 256);
        for (int idx = tid; idx < NTW * 256; idx += 256) mine[idx] = C[idx];
        __threadfence();
        __syncthreads();
        if (tid == 0) s_last = (atomicAdd(&g.cnt[tg], 1) == g.kc - 1);
        __syncthreads();
        if (!s_last) return;
        __threadfence();
        for (int idx = tid; idx < NTW * 256; idx += 256) {
            float s = 0.f;
            for (int c = 0; c < g.kc; ++c)
                s += __builtin_nontemporal_load(g.part + (tg * g.kc + c) * (NTW * 256) + idx);
            C[idx] = s;
        }
        if (tid == 0) g.cnt[tg] = 0;
    }
    __syncthreads();

    // ---- epilogue.  Y[mt][b][n] = sum over pieces of C[mt][piece*nb + b][n]
    auto Y = [&](int mt, int b, int n) -> float {
        float v = C[mt * 256 + b * 16 + n];
        if constexpr (PIECES == 3) v += C[mt * 256 + (nb + b) * 16 + n] + C[mt * 256 + (2 * nb + b) * 16 + n];
        return v;
    };
    auto scale_of = [&](int mt, int r) -> float {
        if constexpr (WT == WT_I8) {
            const float *s = (PAIR && mt == 1) ? g.sc2 : g.sc;
            return s[(long long)ex * g.es_stride + r];
        } else {
            return 1.0f;
        }
    };

    if constexpr (EPI == EPI_QKV) {
        const int hd = g.Hq * g.D, kd = g.Hk * g.D;
        for (int idx = tid; idx < nb * 8; idx += 256) {
            const int b = idx >> 3, n0 = (idx & 7) * 2;
            const int r0 = bx * 16 + n0;
            if (r0 >= g.N) continue;
            float y0 = Y(0, b, n0) * scale_of(0, r0);
            float y1 = Y(0, b, n0 + 1) * scale_of(0, r0 + 1);
            const int pos = g.pos[b];
            if (r0 < hd) {
                rope_pair(y0, y1, (r0 % g.D) >> 1, g.D, pos, g.theta);
                g.q_out[(long long)b * hd + r0] = y0;
                g.q_out[(long long)b * hd + r0 + 1] = y1;
            } else {
                const bool isk = r0 < hd + kd;
                const int rr = isk ? r0 - hd : r0 - hd - kd;
                const int j = rr / g.D, dd = rr % g.D;
                if (isk) rope_pair(y0, y1, dd >> 1, g.D, pos, g.theta);
                const int page = g.pt[b][pos / kPage];
                const long long off = (((long long)page * g.Hk + j) * kPage + (pos % kPage)) * g.D + dd;
                char *base = isk ? g.kvk[b] : g.kvv[b];
                if (g.kv_es == 2) {
                    uint32_t pk = bf16_rne_bits(y0) | (bf16_rne_bits(y1) << 16);
                    *reinterpret_cast<uint32_t *>(base + off * 2) = pk;
                } else {
                    reinterpret_cast<float *>(base)[off] = y0;
                    reinterpret_cast<float *>(base)[off + 1] = y1;
                }
            }
        }
    } else if constexpr (EPI == EPI_RESID) {
        for (int idx = tid; idx < nb * 16; idx += 256) {
            const int b = idx >> 4, n = idx & 15, r = bx * 16 + n;
            if (r < g.N) g.out_f32[(long long)b * g.ld_out + r] += Y(0, b, n) * scale_of(0, r);
        }
    } else if constexpr (EPI == EPI_SWIGLU || EPI == EPI_MOE_SWIGLU) {
        for (int idx = tid; idx < nb * 16; idx += 256) {
            const int b = idx >> 4, n = idx & 15, r = bx * 16 + n;
            if (r >= g.N) continue;
            const float gt = Y(0, b, n) * scale_of(0, r);
            const float up = Y(1, b, n) * scale_of(1, r);
            const float h = (gt / (1.0f + expf(-gt))) * up;
            const long long row = MOE ? s_ent[b] : b;
            store_act<AT>(g.out_act, row * g.ld_out + r, h);
        }
    } else if constexpr (EPI == EPI_MOE_DOWN) {
        for (int idx = tid; idx < nb * 16; idx += 256) {
            const int b = idx >> 4, n = idx & 15, r = bx * 16 + n;
            if (r < g.N) g.out_f32[(long long)s_ent[b] * g.ld_out + r] = Y(0, b, n) * scale_of(0, r);
        }
    } else if constexpr (EPI == EPI_LOGITS) {
        float *L = red;  // reuse: logits of this block [slot][NTW*16]
        for (int idx = tid; idx < nb * NTW * 16; idx += 256) {
            const int b = idx / (NTW * 16), c = idx % (NTW * 16), mt = c >> 4, n = c & 15;
            const int r = (bx * NTW + mt) * 16 + n;
            float v = 0.f;
            if (r < g.N) {
                v = Y(mt, b, n) * scale_of(mt, r);
                if (g.out_f32) g.out_f32[(long long)b * g.N + r] = v;
            }
            L[idx] = v;
        }
        __syncthreads();
        for (int b = tid; b < nb; b += 256) {
            float best = 0.f;
            int bi = -1;
            bool nan = false;
            for (int c = 0; c < NTW * 16; ++c) {
                const int r = bx * NTW * 16 + c;
                if (r >= g.N) break;
                const float v = L[b * NTW * 16 + c];
                if (v != v) { nan = true; continue; }
                if (bi < 0 || v > best) { best = v; bi = r; }
            }
            g.am_val[(long long)bx * nb + b] = best;
            g.am_idx[(long long)bx * nb + b] = bi;
            if (nan) atomicOr(g.err[b], ERR_NAN);
        }
    }
}

// ---------------------------------------------------------------- attention

struct AttnArgs {
    const float *q;   // [slot][Hq*D]
    void *o;          // [slot][Hq*D] act dtype
    int Hq, Hk, G, kps;
    float scale;
    int pos[kMaxSlots], t0[kMaxSlots], nsplit[kMaxSlots], s_cap[kMaxSlots];
    const char *kvk[kMaxSlots], *kvv[kMaxSlots];
    const int *pt[kMaxSlots];
    float *part[kMaxSlots];  // [Hk][s_cap][G][D+2]
    int *cnt[kMaxSlots];     // [Hk]
};

template <int KV>
__device__ __forceinline__ float kv_at(const char *base, long long i) {
    if constexpr (KV == 1) return bf16_bits_f32(reinterpret_cast<const uint16_t *>(base)[i]);
    else return reinterpret_cast<const float *>(base)[i];
}

// Split-K flash decode.  grid: x = split, y = kv head, z = slot; 256 threads.
// Each split covers kps keys of the slot's window; each wave takes 64-key
// chunks with an online softmax.  For q.k a lane owns one key and reads its
// whole K row; for p.v a lane owns D/64 (at least one) consecutive dimensions
// and reads one value row per key.  All K and V loads of a chunk are issued
// before any arithmetic, so a wave keeps a whole chunk in flight.  Waves, then
// splits, are merged in a fixed order, so results do not depend on timing.
template <int D, int KV, int AT>
__global__ void __launch_bounds__(256) k_attn(AttnArgs a) {
    constexpr int VE = D >= 64 ? D / 64 : 1;   // value elements per lane
    constexpr int VL = D / VE;                 // lanes holding values
    constexpr int ES = KV == 1 ? 2 : 4;
    constexpr int KVEC = 16 / ES;              // K elements per 16-byte load
    constexpr int NKL = D / KVEC;              // 16-byte loads per K row
    constexpr int VCH = (VE * ES > 4) ? 32 : 64;  // keys whose V is held at once
    typedef typename std::conditional<VE * ES == 2, uint16_t,
            typename std::conditional<VE * ES == 4, uint32_t, unsigned long long>::type>::type vword;
    const int s = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
    if (s >= a.nsplit[b]) return;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int G = a.G;
    const int pos = a.pos[b];
    const int kb = a.t0[b] + s * a.kps;
    const int ke = min(kb + a.kps, pos + 1);

    __shared__ float qs[kMaxG][D];
    __shared__ float wm[kAttnWaves][kMaxG], wl[kAttnWaves][kMaxG];
    __shared__ float wacc[kAttnWaves][kMaxG][D];
    __shared__ int s_last;

    for (int idx = tid; idx < G * D; idx += 256)
        qs[idx / D][idx % D] = a.q[(long long)b * a.Hq * D + (long long)(j * G) * D + idx] * a.scale;
    __syncthreads();

    const char *Kb = a.kvk[b];
    const char *Vb = a.kvv[b];
    const int *pt = a.pt[b];
    const bool vlane = lane < VL;

    float m[kMaxG], l[kMaxG], acc[kMaxG][VE];
#pragma unroll
    for (int g = 0; g < kMaxG; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[g][e] = 0.f;
    }

    for (int cs = kb + w * 64; cs < ke; cs += kAttnWaves * 64) {
        const int t = cs + lane;
        const bool valid = t < ke;
        const int tt = valid ? t : cs;  // invalid lanes read a valid key and get weight 0
        const int off = ((pt[tt / kPage] * a.Hk + j) * kPage + (tt % kPage)) * D;  // element offset
        // issue the chunk's loads: this lane's K row, then the first V rows
        u32x4 kreg[NKL];
        const u32x4 *kp = reinterpret_cast<const u32x4 *>(Kb + (long long)off * ES);
#pragma unroll
        for (int c = 0; c < NKL; ++c) kreg[c] = kp[c];
        vword vreg[VCH];
        const vword *vbase = reinterpret_cast<const vword *>(Vb) + (vlane ? lane : 0);
#pragma unroll
        for (int u = 0; u < VCH; ++u)
            vreg[u] = vbase[__builtin_amdgcn_readlane(off, u) / VE];
        // q.k for this lane's key
        float sc[kMaxG];
#pragma unroll
        for (int g = 0; g < kMaxG; ++g) sc[g] = 0.f;
#pragma unroll
        for (int c = 0; c < NKL; ++c) {
            float kf[KVEC];
            if constexpr (KV == 1) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    kf[2 * e] = __uint_as_float(kreg[c][e] << 16);
                    kf[2 * e + 1] = __uint_as_float(kreg[c][e] & 0xFFFF0000u);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) kf[e] = __uint_as_float(kreg[c][e]);
            }
#pragma unroll
            for (int g = 0; g < kMaxG; ++g)
                if (g < G)
#pragma unroll
                    for (int e = 0; e < KVEC; ++e) sc[g] = fmaf(qs[g][c * KVEC + e], kf[e], sc[g]);
            __builtin_amdgcn_sched_barrier(0);
        }
        // online softmax update
        float p[kMaxG];
#pragma unroll
        for (int g = 0; g < kMaxG; ++g) {
            p[g] = 0.f;
            if (g < G) {
                const float sv = valid ? sc[g] : -INFINITY;
                const float mn = fmaxf(m[g], wave_max(sv));
                const float alpha = expf(m[g] - mn);
                p[g] = valid ? expf(sv - mn) : 0.f;
                l[g] = l[g] * alpha + wave_sum(p[g]);
#pragma unroll
                for (int e = 0; e < VE; ++e) acc[g][e] *= alpha;
                m[g] = mn;
            }
        }
        // p.v
#pragma unroll
        for (int vb = 0; vb < 64; vb += VCH) {
            if (vb > 0) {
#pragma unroll
                for (int u = 0; u < VCH; ++u)
                    vreg[u] = vbase[__builtin_amdgcn_readlane(off, vb + u) / VE];
            }
#pragma unroll
            for (int u = 0; u < VCH; ++u) {
                float v[VE];
                if constexpr (KV == 1) {
                    if constexpr (VE == 2) {
                        v[0] = __uint_as_float((uint32_t)vreg[u] << 16);
                        v[1] = __uint_as_float((uint32_t)vreg[u] & 0xFFFF0000u);
                    } else {
                        v[0] = __uint_as_float((uint32_t)vreg[u] << 16);
                    }
                } else {
                    if constexpr (VE == 2) {
                        v[0] = __uint_as_float((uint32_t)(vreg[u] & 0xFFFFFFFFull));
                        v[1] = __uint_as_float((uint32_t)(vreg[u] >> 32));
                    } else {
                        v[0] = __uint_as_float((uint32_t)vreg[u]);
                    }
                }
#pragma unroll
                for (int g = 0; g < kMaxG; ++g) {
                    if (g < G) {
                        const float pg = readlane_f(p[g], vb + u);
#pragma unroll
                        for (int e = 0; e < VE; ++e) acc[g][e] = fmaf(pg, v[e], acc[g][e]);
                    }
                }
            }
        }
    }

    // merge the waves
    if (lane == 0)
        for (int g = 0; g < G; ++g) { wm[w][g] = m[g]; wl[w][g] = l[g]; }
#pragma unroll
    for (int g = 0; g < kMaxG; ++g)
        if (g < G && vlane)
#pragma unroll
            for (int e = 0; e < VE; ++e) wacc[w][g][lane * VE + e] = acc[g][e];
    __syncthreads();

    const int ns = a.nsplit[b];
    float *part = a.part[b];
    for (int idx = tid; idx < G * D; idx += 256) {
        const int g = idx / D, d = idx % D;
        float M = wm[0][g];
        for (int x = 1; x < kAttnWaves; ++x) M = fmaxf(M, wm[x][g]);
        float L = 0.f, A = 0.f;
        for (int x = 0; x < kAttnWaves; ++x) {
            const float f = expf(wm[x][g] - M);
            L += wl[x][g] * f;
            A += wacc[x][g][d] * f;
        }
        if (ns == 1) {
            store_act<AT>(a.o, (long long)b * a.Hq * D + (long long)(j * G + g) * D + d, A / L);
        } else {
            float *pp = part + (((long long)j * a.s_cap[b] + s) * G + g) * (D + 2);
            if (d == 0) { pp[0] = M; pp[1] = L; }
            pp[2 + d] = A;
        }
    }
    if (ns == 1) return;
    __threadfence();
    __syncthreads();
    if (tid == 0) s_last = (atomicAdd(&a.cnt[b][j], 1) == ns - 1);
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    for (int idx = tid; idx < G * D; idx += 256) {
        const int g = idx / D, d = idx % D;
        const float *p0 = part + ((long long)j * a.s_cap[b] * G + g) * (D + 2);
        const long long sstride = (long long)G * (D + 2);
        float M = -INFINITY;
        for (int x = 0; x < ns; ++x) M = fmaxf(M, __builtin_nontemporal_load(p0 + x * sstride));
        float L = 0.f, A = 0.f;
        for (int x = 0; x < ns; ++x) {
            const float *px = p0 + x * sstride;
            const float f = expf(__builtin_nontemporal_load(px) - M);
            L += __builtin_nontemporal_load(px + 1) * f;
            A += __builtin_nontemporal_load(px + 2 + d) * f;
        }
        store_act<AT>(a.o, (long long)b * a.Hq * D + (long long)(j * G + g) * D + d, A / L);
    }
    if (tid == 0) a.cnt[b][j] = 0;
}

// ---------------------------------------------------------------- small kernels

struct SlotPtrs {
    int *err[kMaxSlots];
};

// x[b] = tok_embd[token[b]] (fp32 or bf16 table); bad ids use row 0 and set a flag.
template <int ET>
__global__ void __launch_bounds__(256) k_embed(const void *embd, const int *tokens, float *x, int E,
                                                 int V, SlotPtrs sp) {
    const int b = blockIdx.x;
    int tok = tokens[b];
    if (tok < 0 || tok >= V) {
        if (threadIdx.x == 0) atomicOr(sp.err[b], ERR_TOKEN);
        tok = 0;
    }
    for (int k = threadIdx.x; k < E; k += 256) {
        float v;
        if constexpr (ET == 1)
            v = bf16_bits_f32(reinterpret_cast<const uint16_t *>(embd)[(long long)tok * E + k]);
        else
            v = reinterpret_cast<const float *>(embd)[(long long)tok * E + k];
        x[(long long)b * E + k] = v;
    }
}

// argmax[b] over the LM head's per-block partials (value, lowest index on ties).
__global__ void __launch_bounds__(256) k_argmax(const float *val, const int *idx, int nwg, int nb,
                                                 int *out) {
    const int b = blockIdx.x, tid = threadIdx.x;
    float best = 0.f;
    int bi = -1;
    for (int w = tid; w < nwg; w += 256) {
        const int i = idx[(long long)w * nb + b];
        const float v = val[(long long)w * nb + b];
        if (i < 0) continue;
        if (bi < 0 || v > best || (v == best && i < bi)) { best = v; bi = i; }
    }
    __shared__ float sv[256];
    __shared__ int si[256];
    sv[tid] = best;
    si[tid] = bi;
    __syncthreads();
    for (int o = 128; o > 0; o >>= 1) {
        if (tid < o) {
            const float v = sv[tid + o];
            const int i = si[tid + o];
            if (i >= 0 && (si[tid] < 0 || v > sv[tid] || (v == sv[tid] && i < si[tid]))) {
                sv[tid] = v;
                si[tid] = i;
            }
        }
        __syncthreads();
    }
    if (tid == 0 && out) out[b] = si[0];
}

// MoE router of one slot: xn = round_act(RMSNorm(x)*g); r = W_r xn; top-k (ties
// to the lower index); weights = softmax over the chosen logits.
template <int RT, int AT>
__global__ void __launch_bounds__(256) k_router(const float *x, const float *gain, const void *wr,
                                                 int E, int n_expert, int k_used, float eps,
                                                 int *ids, float *wts) {
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    extern __shared__ float xs[];  // [E]
    __shared__ float red4[4];
    __shared__ float r[64];
    const float *xr = x + (long long)b * E;
    float ss = 0.f;
    for (int k = tid; k < E; k += 256) ss += xr[k] * xr[k];
    ss = block_sum256(ss, red4);
    const float rinv = 1.0f / sqrtf(ss / (float)E + eps);
    for (int k = tid; k < E; k += 256) {
        float v = (xr[k] * rinv) * gain[k];
        if (AT == AT_BF16) v = bf16_round(v);
        xs[k] = v;
    }
    __syncthreads();
    for (int e = w; e < n_expert; e += 4) {
        float acc = 0.f;
        for (int k = lane; k < E; k += 64) {
            float wv;
            if constexpr (RT == 1)
                wv = bf16_bits_f32(reinterpret_cast<const uint16_t *>(wr)[(long long)e * E + k]);
            else
                wv = reinterpret_cast<const float *>(wr)[(long long)e * E + k];
            acc = fmaf(wv, xs[k], acc);
        }
        acc = wave_sum(acc);
        if (lane == 0) r[e] = acc;
    }
    __syncthreads();
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
        }
    }
}

// x[b][r] += sum_k w[b][k] * y[b*k_used + k][r]
__global__ void __launch_bounds__(256) k_moe_combine(float *x, const float *y, const float *wts,
                                                      int E, int k_used) {
    const int b = blockIdx.y;
    const int r = blockIdx.x * 256 + threadIdx.x;
    if (r >= E) return;
    float s = 0.f;
    for (int k = 0; k < k_used; ++k)
        s += wts[b * k_used + k] * y[((long long)b * k_used + k) * E + r];
    x[(long long)b * E + r] += s;
}

// Re-lay a row-major matrix [N][K] (element size ES) into 1 KiB tiles.
// Int8 codes are stored biased (u = q + 128); padding is the code of 0.
template <int ES>
__global__ void __launch_bounds__(256) k_pack(const uint8_t *src, int N, int K, int KT, int n_tiles,
                                               uint8_t *dst) {
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
            uint8_t v = in ? src[((long long)row * K + k) * ES + bb] : 0;
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

__global__ void __launch_bounds__(256) k_fill32(uint32_t *p, long long n, uint32_t v) {
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256)
        p[i] = v;
}

__global__ void __launch_bounds__(256) k_iota(int *p, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = i;
}

__global__ void __launch_bounds__(256) k_copy_bytes(uint8_t *dst, const uint8_t *src, long long n) {
    for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256)
        dst[i] = src[i];
}

// Scatter K and V of positions pos0..pos0+n-1 ([n][Hk][D]) into the pages of one layer.
template <int ES>
__global__ void __launch_bounds__(256) k_set_kv(char *kpool, char *vpool, const int *pt, const char *k,
                                                 const char *v, int pos0, int n, int Hk, int D) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long total = (long long)n * Hk * D;
    if (i >= total) return;
    const int d = (int)(i % D);
    const int j = (int)((i / D) % Hk);
    const int t = (int)(i / ((long long)D * Hk));
    const int p = pos0 + t;
    const long long off = (((long long)pt[p / kPage] * Hk + j) * kPage + (p % kPage)) * D + d;
    if constexpr (ES == 2) {
        reinterpret_cast<uint16_t *>(kpool)[off] = reinterpret_cast<const uint16_t *>(k)[i];
        reinterpret_cast<uint16_t *>(vpool)[off] = reinterpret_cast<const uint16_t *>(v)[i];
    } else {
        reinterpret_cast<float *>(kpool)[off] = reinterpret_cast<const float *>(k)[i];
        reinterpret_cast<float *>(vpool)[off] = reinterpret_cast<const float *>(v)[i];
    }
}

}  // namespace pn
