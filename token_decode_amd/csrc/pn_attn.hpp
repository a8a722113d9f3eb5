// pn_attn.hpp - split-K flash-decode attention over the paged KV cache and
// the split merge, with the Q4 KV-cache helpers (included by the attention
// units and the engine; the GEMM units need none of it).
#pragma once

#include "pn_kernels.hpp"

namespace pn {

// ---------------------------------------------------------------- attention

struct AttnArgs {
    const float *q;   // [slot][Hq*D]
    float *o;         // attention output [slot][Hq*D] (fp32; the O projection rounds it)
    int Hq, Hk;
    float scale;      // 1/sqrt(D) * log2(e): scores are kept in the base-2 domain
    int pos[kMaxSlots];     // the slot's current position (its last key)
    int lo[kMaxSlots];      // first key inside the window
    int origin[kMaxSlots];  // lo rounded down to a page: the window's np pages start there
    int np[kMaxSlots];      // split s of nsplit takes pages [s*np/nsplit, (s+1)*np/nsplit)
    int nsplit[kMaxSlots], s_cap[kMaxSlots];
    const char *kvk[kMaxSlots], *kvv[kMaxSlots];
    const int *pt[kMaxSlots];
    float *part[kMaxSlots];  // [Hk][s_cap][G][D+4]: running max (base 2), sum, 2 pad, unnormalised output
    unsigned kv_bytes[kMaxSlots];  // bytes of one layer's K (and of its V) pool
    int pt_ident[kMaxSlots];       // 1: the slot's page table is the identity (logical page = physical)
    int kind;                // bf16 cache: 0 = vector units (k_attn), 1 = matrix cores (k_attn_mfma)
    // rows > 0: the grid's slots are `rows` prefill rows of one state, row b at
    // position p0 + b; the per-slot entries 0 hold that state's pages, page
    // table and split capacity; window, lo, origin, np come from the position
    // (window 0 = none), nsplit = min(ns_rows, np), and row b's split scratch
    // starts part_row floats after row b - 1's
    int rows, p0, window, ns_rows;
    long long part_row;
    // rows mode, bf16 cache on the matrix cores: tile > 1 puts `tile` (= 16 / G)
    // consecutive rows in one work-group, their heads in the 16 columns, so
    // the rows share every K and V load (one split; no merge)
    int tile;
    // decode over a bf16 cache on the matrix cores: waves per work-group (4, or
    // 8 for G <= 4: two pages per chunk)
    int waves;
};

// One slot's (or prefill row's) attention geometry.
struct AttnRow {
    int pos, lo, origin, np, nsplit, s_cap;
    const char *kvk, *kvv;
    const int *pt;
    float *part;
    unsigned kv_bytes;
    int pt_ident;
};
__device__ __forceinline__ AttnRow attn_row(const AttnArgs &a, int b) {
    AttnRow r;
    if (a.rows > 0) {
        r.pos = a.p0 + b;
        r.lo = a.window > 0 ? max(0, r.pos - a.window + 1) : 0;
        r.origin = r.lo / kPage * kPage;
        r.np = (r.pos + 1 - r.origin + kPage - 1) / kPage;
        r.nsplit = min(a.ns_rows, r.np);
        r.s_cap = a.s_cap[0];
        r.kvk = a.kvk[0];
        r.kvv = a.kvv[0];
        r.pt = a.pt[0];
        r.part = a.part[0] + (long long)b * a.part_row;
        r.kv_bytes = a.kv_bytes[0];
        r.pt_ident = a.pt_ident[0];
    } else {
        r.pos = a.pos[b];
        r.lo = a.lo[b];
        r.origin = a.origin[b];
        r.np = a.np[b];
        r.nsplit = a.nsplit[b];
        r.s_cap = a.s_cap[b];
        r.kvk = a.kvk[b];
        r.kvv = a.kvv[b];
        r.pt = a.pt[b];
        r.part = a.part[b];
        r.kv_bytes = a.kv_bytes[b];
        r.pt_ident = a.pt_ident[b];
    }
    return r;
}

// Split-K flash decode for G query heads per KV head.  Decode attention
// moves few bytes per work-group, and one compute unit only pulls a small
// share of HBM bandwidth, so the window is cut into many short splits (a
// multiple of 64 keys each, aligned to pages) spread over the whole chip;
// k_attn_merge then folds the splits together.
//
// grid: x = split, y = kv head, z = slot; 256 threads (4 waves).  A split is
// walked in page-aligned chunks of 64 keys, 16 per wave, so a wave's keys sit
// in one page (one scalar page-table load).  For q.k four lanes share a key,
// each taking the 16-byte pieces dq, dq+4, dq+8, ... of its row (so every
// load instruction of the four lanes covers 64 contiguous bytes) and two DPP
// steps finish the dot product; for p.v a lane owns D/64 (at least one)
// consecutive dimensions and reads one value row per key, with the 16 key
// weights broadcast through LDS.  All K and V loads of a chunk are issued
// before any arithmetic; in multi-chunk splits the next chunk is in flight
// while the current one is scored.  Keys outside [lo, pos] are masked (their
// rows are clamped into the window, so masked lanes read valid data).  Each
// wave keeps a running (max, sum, output); the waves merge in a fixed order.
// A single-split slot writes the output; otherwise the split's (max, sum,
// unnormalised output) goes to the state's split scratch.
constexpr int kAttnWaves = 4;
constexpr int kAttnChunk = kAttnWaves * 16;  // keys per chunk, and the split granularity
constexpr int kMaxSplits = 256;              // splits per (slot, kv head)
static_assert(kAttnChunk == kPage, "a chunk is one page of keys");

__device__ __forceinline__ float quad_sum(float v) {
    v += dpp_f<kDppXor1, 0xF>(0.f, v);
    v += dpp_f<kDppXor2, 0xF>(0.f, v);
    return v;
}
// max over the 64 lanes of a value that is uniform within each quad of lanes
__device__ __forceinline__ float wave_max_q(float v) {
    v = fmaxf(v, dpp_f<kDppHalfMirror, 0xF>(-INFINITY, v));
    v = fmaxf(v, dpp_f<kDppMirror, 0xF>(-INFINITY, v));
    v = fmaxf(v, dpp_f<kDppBcast15, 0xA>(-INFINITY, v));
    v = fmaxf(v, dpp_f<kDppBcast31, 0xC>(-INFINITY, v));
    return readlane_f(v, 63);
}
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Q4 KV cache: per page and KV head, the 64 keys' codes (dims 2i, 2i+1 in the
// low and high nibbles of byte i) and their block scales (fp16; a block is 32
// dims, value = d * (code - 8)).  K by key rows: codes [key][D/2], then scales
// [key][D/32].  V by columns, so a lane reads one byte column of 16 keys at
// once: codes [D/2][key], then scales [D/32][key].  Each key owns its bytes.
__host__ __device__ constexpr int q4kv_key_bytes(int D) { return D / 2 + D / 16; }

// Quantise one head vector src[D] into a key's codes and scales (one wave; lane l
// < D/2 takes dims 2l, 2l+1, 16 lanes a block); byte l goes to codes[l * cs],
// block scale b to scales[b * ss].  Per block: m = the element of largest
// magnitude (the lowest index on ties), d = fp16(m / -8), code = clamp(rint(x /
// d) + 8, 0, 15), all codes 8 when d is 0; fp32 throughout.
__device__ __forceinline__ void q4kv_store(const float *src, uint8_t *codes, int cs, uint16_t *scales, int ss, int D,
                                           int lane) {
    const bool on = lane < D / 2;
    const float v0 = on ? src[2 * lane] : 0.f, v1 = on ? src[2 * lane + 1] : 0.f;
    float m = fabsf(v1) > fabsf(v0) ? v1 : v0;
    int mi = fabsf(v1) > fabsf(v0) ? 2 * lane + 1 : 2 * lane;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
        const float om = __shfl_xor(m, o, 64);
        const int oi = __shfl_xor(mi, o, 64);
        if (fabsf(om) > fabsf(m) || (fabsf(om) == fabsf(m) && oi < mi)) {
            m = om;
            mi = oi;
        }
    }
    const _Float16 dh = (_Float16)(m / -8.0f);
    const float dd = (float)dh;
    uint32_t c0 = 8u, c1 = 8u;
    if (dd != 0.f) {
        c0 = (uint32_t)fminf(fmaxf(rintf(v0 / dd) + 8.f, 0.f), 15.f);
        c1 = (uint32_t)fminf(fmaxf(rintf(v1 / dd) + 8.f, 0.f), 15.f);
    }
    if (on) {
        codes[lane * cs] = (uint8_t)(c0 | (c1 << 4));
        if ((lane & 15) == 0) scales[(lane / 16) * ss] = __builtin_bit_cast(uint16_t, dh);
    }
}

// the new rows of a Q4 KV cache and where they go
struct KvQ4Args {
    const float *src;  // [row][2][Hk][D]: k then v
    char *kvk[kMaxSlots];
    char *kvv[kMaxSlots];
    const int *pt[kMaxSlots];
    int pos[kMaxSlots];
    int Hk, D;
};

template <int D, int KV>
struct AttnShape {
    // KV: 0 fp32, 1 bf16, 2 Q4 (values widened to fp32 as they are loaded)
    static constexpr int ES = KV == 1 ? 2 : 4;       // bytes per cached (or widened) element
    static constexpr int VE = D >= 64 ? D / 64 : 1;  // value elements per lane
    static constexpr int VL = D / VE;                // lanes holding values
    // 16-byte K registers per lane (Q4: the codes of the lane's quarter of the
    // dims, then the block scale)
    static constexpr int NKL = KV == 2 ? 2 : D * ES / 64;
    static constexpr int KVEC = 16 / ES;             // K elements per load (fp32 / bf16)
    typedef typename std::conditional<VE * ES == 2, uint16_t,
            typename std::conditional<VE * ES == 4, uint32_t, unsigned long long>::type>::type vword;
    // double-buffer a chunk's rows when both copies fit the register budget
    static constexpr bool PREF = (NKL * 4 + 16 * (int)sizeof(vword) / 4) <= 40;
};

// Issue the K and V loads of one wave's 16 keys k0..k0+15 (k0 a multiple of
// 16, w-uniform), which lie in physical page pg.  K rows are clamped into
// [lo, kl], which keeps them inside that page and inside the written window;
// a lane gathers the 16 keys of each of its V dimensions (one run for an fp32
// cache, four 8-byte pieces for a bf16 one), and keys outside [lo, kl] read
// zeros (their weights are 0, and 0 * NaN would not be).
template <int D, int KV>
__device__ __forceinline__ void attn_load(const AttnArgs &a, const AttnRow &R, int j, int pg, int k0, int lo, int kl, int kq,
                                          int dq, int lane, u32x4 (&kr)[AttnShape<D, KV>::NKL],
                                          typename AttnShape<D, KV>::vword (&vr)[16]) {
    typedef AttnShape<D, KV> S;
    const long long hb = ((long long)pg * a.Hk + j) * kPage * D;  // the head's block of the page
    const int tq = min(max(k0 + kq, lo), kl);
    const int dl = (lane < S::VL ? lane : 0) * S::VE;
    uint32_t col[S::VE][16];
    if constexpr (KV == 2) {
        // Q4 block of the head (q4kv_*): codes [key][D/2] then scales [key][D/32]
        const uint8_t *kb = reinterpret_cast<const uint8_t *>(R.kvk) + ((long long)pg * a.Hk + j) * kPage * q4kv_key_bytes(D);
        const uint8_t *krow = kb + (tq % kPage) * (D / 2) + dq * (D / 8);  // the lane's quarter: D/8 bytes
        if constexpr (D == 128) {
            kr[0] = *reinterpret_cast<const u32x4 *>(krow);
        } else if constexpr (D == 64) {
            const u32x2 t = *reinterpret_cast<const u32x2 *>(krow);
            kr[0] = u32x4{t[0], t[1], 0u, 0u};
        } else {
            kr[0] = u32x4{*reinterpret_cast<const uint32_t *>(krow), 0u, 0u, 0u};
        }
        const uint16_t *ks = reinterpret_cast<const uint16_t *>(kb + kPage * (D / 2)) + (tq % kPage) * (D / 32) +
                             dq * (D / 4) / 32;
        kr[1] = u32x4{(uint32_t)*ks, 0u, 0u, 0u};
        // values: the lane's byte column for the 16 keys (one 16-byte load) and
        // their scales of its block (32 bytes), widened to fp32 here
        const uint8_t *vb = reinterpret_cast<const uint8_t *>(R.kvv) + ((long long)pg * a.Hk + j) * kPage * q4kv_key_bytes(D);
        const int key0 = k0 % kPage;
        const u32x4 cw = *reinterpret_cast<const u32x4 *>(vb + (dl / 2) * kPage + key0);
        const u32x4 *vs = reinterpret_cast<const u32x4 *>(vb + kPage * (D / 2) + ((dl / 32) * kPage + key0) * 2);
        const u32x4 s0 = vs[0], s1 = vs[1];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            const uint32_t byte = (cw[u / 4] >> (8 * (u % 4))) & 0xFFu;
            const uint32_t sw = u < 8 ? s0[(u % 8) / 2] : s1[(u % 8) / 2];
            const float sc = (u & 1) ? half_hi(sw) : half_lo(sw);
#pragma unroll
            for (int e = 0; e < S::VE; ++e) {
                const int code = (int)(((dl + e) & 1) ? byte >> 4 : byte & 15u);
                col[e][u] = __float_as_uint(sc * (float)(code - 8));
            }
        }
    } else if constexpr (KV == 1) {
        // tiled (kv_k_off / kv_v_off): piece dq + 4c of key row tq % 16 is 16 bytes of
        // the group's 1 KiB step c; the 4 keys 4q..4q+3 of a dim are 8 contiguous bytes
        // (next to the same keys of dim + 16 or dim - 16)
        const uint8_t *gk = reinterpret_cast<const uint8_t *>(R.kvk) + (hb + (long long)(k0 % kPage) * D) * 2;
#pragma unroll
        for (int c = 0; c < S::NKL; ++c)
            kr[c] = *reinterpret_cast<const u32x4 *>(gk + c * 1024 + (dq * 16 + tq % 16) * 16);
        const uint8_t *gv = reinterpret_cast<const uint8_t *>(R.kvv) + (hb + (long long)(k0 % kPage) * D) * 2;
#pragma unroll
        for (int e = 0; e < S::VE; ++e) {
            const int d = dl + e;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u32x2 t = *reinterpret_cast<const u32x2 *>(
                    gv + (((d / 32) * 64 + q * 16 + d % 16) * 8 + ((d % 32) / 16) * 4) * 2);
                col[e][4 * q] = t[0] & 0xFFFFu;
                col[e][4 * q + 1] = t[0] >> 16;
                col[e][4 * q + 2] = t[1] & 0xFFFFu;
                col[e][4 * q + 3] = t[1] >> 16;
            }
        }
    } else {
        // rows for K, columns for V
        const u32x4 *kp = reinterpret_cast<const u32x4 *>(R.kvk + (hb + (long long)(tq % kPage) * D + dq * S::KVEC) * S::ES);
#pragma unroll
        for (int c = 0; c < S::NKL; ++c) kr[c] = kp[4 * c];
        constexpr int NV = 16 * S::ES / 16;  // 16-byte loads per column run
#pragma unroll
        for (int e = 0; e < S::VE; ++e) {
            const u32x4 *vp = reinterpret_cast<const u32x4 *>(
                R.kvv + (hb + (long long)(dl + e) * kPage + k0 % kPage) * S::ES);
#pragma unroll
            for (int c = 0; c < NV; ++c) {
                const u32x4 t = vp[c];
#pragma unroll
                for (int q = 0; q < 4; ++q) col[e][4 * c + q] = t[q];
            }
        }
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
        const bool in = k0 + u >= lo && k0 + u <= kl;
        unsigned long long w = 0;
#pragma unroll
        for (int e = 0; e < S::VE; ++e) w |= (unsigned long long)(in ? col[e][u] : 0u) << (8 * S::ES * e);
        vr[u] = (typename S::vword)w;
    }
}

// Score one wave's 16 keys k0..k0+15 (valid: lo <= key < ke, at least one)
// and fold them into the running (m, l, acc) of its G query heads.  pw is the
// wave's LDS slice for the key weights.
template <int D, int KV, int G>
__device__ __forceinline__ void attn_chunk(const float (*qs)[D], float (*pw)[16],
                                           const u32x4 (&kr)[AttnShape<D, KV>::NKL],
                                           const typename AttnShape<D, KV>::vword (&vr)[16], int k0, int lo,
                                           int ke, int kq, int dq, float (&m)[G], float (&l)[G],
                                           float (&acc)[G][AttnShape<D, KV>::VE]) {
    typedef AttnShape<D, KV> S;
    float sc[G];
#pragma unroll
    for (int g = 0; g < G; ++g) sc[g] = 0.f;
    if constexpr (KV == 2) {
        // Q4: the lane's D/4 dims from 4-bit codes (dim 2i in the low nibble of
        // byte i, 2i + 1 in the high one), times the block scale
        constexpr int QD = D / 4;
        const float dsc = half_lo(kr[1][0]);
        float t[G];
#pragma unroll
        for (int g = 0; g < G; ++g) t[g] = 0.f;
#pragma unroll
        for (int i = 0; i < QD; ++i) {
            const float kf = (float)((int)((kr[0][i / 8] >> (4 * (i % 8))) & 15u) - 8);
#pragma unroll
            for (int g = 0; g < G; ++g) t[g] = fmaf(qs[g][dq * QD + i], kf, t[g]);
        }
#pragma unroll
        for (int g = 0; g < G; ++g) sc[g] = t[g] * dsc;
    } else {
#pragma unroll
        for (int c = 0; c < S::NKL; ++c) {
            float kf[S::KVEC];
            if constexpr (KV == 1) {
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    kf[2 * e] = __uint_as_float(kr[c][e] << 16);
                    kf[2 * e + 1] = __uint_as_float(kr[c][e] & 0xFFFF0000u);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e) kf[e] = __uint_as_float(kr[c][e]);
            }
#pragma unroll
            for (int g = 0; g < G; ++g)
#pragma unroll
                for (int e = 0; e < S::KVEC; ++e) sc[g] = fmaf(qs[g][(4 * c + dq) * S::KVEC + e], kf[e], sc[g]);
        }
    }
    const int key = k0 + kq;
    const bool valid = key >= lo && key < ke;
    float p[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        sc[g] = quad_sum(sc[g]);
        const float mx = fmaxf(m[g], wave_max_q(valid ? sc[g] : -INFINITY));
        const float f = exp2_fast(m[g] - mx);  // 0 on the wave's first chunk
        p[g] = valid ? exp2_fast(sc[g] - mx) : 0.f;
        m[g] = mx;
        l[g] *= f;
#pragma unroll
        for (int e = 0; e < S::VE; ++e) acc[g][e] *= f;
    }
    // the 16 key weights of each head to every lane, through the wave's LDS slice
    if (dq == 0)
#pragma unroll
        for (int g = 0; g < G; ++g) pw[g][kq] = p[g];
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float pg[16];
#pragma unroll
        for (int u = 0; u < 16; u += 4) {
            const f32x4 t = *reinterpret_cast<const f32x4 *>(&pw[g][u]);
            pg[u] = t[0]; pg[u + 1] = t[1]; pg[u + 2] = t[2]; pg[u + 3] = t[3];
        }
        float ls = 0.f;
#pragma unroll
        for (int u = 0; u < 16; ++u) ls += pg[u];
        l[g] += ls;
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            float v[S::VE];
            if constexpr (KV == 1) {
                v[0] = __uint_as_float((uint32_t)vr[u] << 16);
                if constexpr (S::VE == 2) v[1] = __uint_as_float((uint32_t)vr[u] & 0xFFFF0000u);
            } else {
                v[0] = __uint_as_float((uint32_t)((unsigned long long)vr[u] & 0xFFFFFFFFull));
                if constexpr (S::VE == 2) v[1] = __uint_as_float((uint32_t)((unsigned long long)vr[u] >> 32));
            }
#pragma unroll
            for (int e = 0; e < S::VE; ++e) acc[g][e] = fmaf(pg[u], v[e], acc[g][e]);
        }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

template <int D, int KV, int G>
__global__ void __launch_bounds__(256) k_attn(AttnArgs a) {
    typedef AttnShape<D, KV> S;
    constexpr int NWV = kAttnWaves;
    const int s = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
    const AttnRow R = attn_row(a, b);
    if (s >= R.nsplit) return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lo = R.lo;
    const int np = R.np, ns_b = R.nsplit;
    const int kb = R.origin + (int)((long long)s * np / ns_b) * kPage;
    const int ke = min(R.origin + (int)((long long)(s + 1) * np / ns_b) * kPage, R.pos + 1);
    const int kl = ke - 1;

    __shared__ __align__(16) float qs[G][D];
    __shared__ __align__(16) float pws[NWV][G][16];
    __shared__ float wm[NWV][G], wl[NWV][G];
    __shared__ float wacc[NWV][G][D];

    const int kq = lane >> 2, dq = lane & 3;
    // the split's pages, one chunk (= page) per lane, looked up once; chunk ci
    // past the split's last reads the last one (its loads are clamped there)
    const int nch = (ke - kb + kAttnChunk - 1) / kAttnChunk;
    // (an identity table needs no load: the K/V loads can go out at once)
    const int *ptb = R.pt + kb / kPage;
    const int vpg = R.pt_ident ? kb / kPage + min(lane, nch - 1) : ptb[min(lane, nch - 1)];
    auto page_of = [&](int ci) -> int {
        ci = min(ci, nch - 1);
        if (R.pt_ident) return kb / kPage + ci;
        return ci < 64 ? __builtin_amdgcn_readlane(vpg, ci) : ptb[ci];
    };
    u32x4 kc[S::NKL], kn[S::NKL];
    typename S::vword vc[16], vn[16];
    attn_load<D, KV>(a, R, j, page_of(0), kb + w * 16, lo, kl, kq, dq, lane, kc, vc);
    {
        const f32x4 *q4 = reinterpret_cast<const f32x4 *>(a.q + (long long)b * a.Hq * D + (long long)(j * G) * D);
        for (int i = tid; i < G * D / 4; i += 256) {
            const f32x4 v = q4[i];
            const int g = (i * 4) / D, d = (i * 4) % D;
#pragma unroll
            for (int e = 0; e < 4; ++e) qs[g][d + e] = v[e] * a.scale;
        }
    }
    lds_barrier();

    float m[G], l[G], acc[G][S::VE];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int e = 0; e < S::VE; ++e) acc[g][e] = 0.f;
    }
    // a wave's 16 keys take part when at least one lies in [lo, ke)
    if (ke - kb <= kAttnChunk) {
        const int k0 = kb + w * 16;
        if (k0 + 15 >= lo && k0 < ke) attn_chunk<D, KV, G>(qs, pws[w], kc, vc, k0, lo, ke, kq, dq, m, l, acc);
    } else {
        for (int c0 = kb, ci = 0; c0 < ke; c0 += kAttnChunk, ++ci) {
            const int k0 = c0 + w * 16;
            if constexpr (S::PREF) {
                // next chunk in flight (clamped into the split past its end)
                attn_load<D, KV>(a, R, j, page_of(ci + 1), k0 + kAttnChunk, lo, kl, kq, dq, lane, kn, vn);
            } else if (c0 != kb) {
                attn_load<D, KV>(a, R, j, page_of(ci), k0, lo, kl, kq, dq, lane, kc, vc);
            }
            if (k0 + 15 >= lo && k0 < ke) attn_chunk<D, KV, G>(qs, pws[w], kc, vc, k0, lo, ke, kq, dq, m, l, acc);
            if constexpr (S::PREF) {
#pragma unroll
                for (int c = 0; c < S::NKL; ++c) kc[c] = kn[c];
#pragma unroll
                for (int u = 0; u < 16; ++u) vc[u] = vn[u];
            }
        }
    }

    // merge the waves in wave order (a wave with no keys has m = -inf, l = 0)
    if (lane == 0)
#pragma unroll
        for (int g = 0; g < G; ++g) { wm[w][g] = m[g]; wl[w][g] = l[g]; }
    if (lane < S::VL)
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int e = 0; e < S::VE; ++e) wacc[w][g][lane * S::VE + e] = acc[g][e];
    lds_barrier();

    const int ns = R.nsplit;
    for (int idx = tid; idx < G * D; idx += 256) {
        const int g = idx / D, d = idx % D;
        float M = wm[0][g];
#pragma unroll
        for (int x = 1; x < NWV; ++x) M = fmaxf(M, wm[x][g]);
        float L = 0.f, A = 0.f;
#pragma unroll
        for (int x = 0; x < NWV; ++x) {
            const float f = exp2_fast(wm[x][g] - M);
            L += wl[x][g] * f;
            A += wacc[x][g][d] * f;
        }
        if (ns == 1) {
            a.o[(long long)b * a.Hq * D + (long long)(j * G + g) * D + d] = A / L;
        } else {
            float *pp = R.part + (((long long)j * R.s_cap + s) * G + g) * (D + 4);
            if (d == 0) { pp[0] = M; pp[1] = L; }
            pp[4 + d] = A;
        }
    }
}

// Piece pc (0..2) of x's exact three-piece bf16 split (x == p0 + p1 + p2:
// 24 mantissa bits), as bits.
__device__ __forceinline__ uint32_t bf16_piece(float x, int pc) {
    const float p0 = bf16_round(x);
    const float r1 = x - p0;
    const float p1 = bf16_round(r1);
    const float p2 = bf16_round(r1 - p1);
    return bf16_rne_bits(pc == 0 ? p0 : (pc == 1 ? p1 : p2));  // (already a bf16 value)
}
// Piece pc of x and of y packed low, high; zero when !on.
__device__ __forceinline__ uint32_t bf16_piece2(float x, float y, int pc, bool on) {
    return on ? (bf16_piece(x, pc) | (bf16_piece(y, pc) << 16)) : 0u;
}
// Rotation by N lanes within each row of 16 lanes.
template <int N>
__device__ __forceinline__ float row_ror(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x120 + N, 0xF, 0xF, false));
}
// The sum of lanes c, c+4, c+8, c+12 of a row of 16, the same value in all
// four: (v_c + v_c+8) + (v_c+4 + v_c+12), whose adds are commutative.
__device__ __forceinline__ float sum_stride4(float v) {
    const float t = v + row_ror<8>(v);
    return t + row_ror<4>(t);
}

// The same split-K flash decode as k_attn for a bf16 cache, on the matrix
// cores.  A wave's 16 keys form one 16x16 score tile per KV head:
//   S^T[key][c] = sum_d K[key][d] * Q[c][d]
// with K fragments as the A operand (16x16x32 steps over d; the cache stores
// them in that order, see kv_k_off, so each load reads 1 KiB) and the scaled
// fp32 query split into three exact bf16 pieces (the products are exact, the
// sums fp32).  With G <= 4 the pieces are columns of the tile: column c =
// 4p + g holds piece p of head g (p = 3 and heads past G are zero), so one
// step per 32 dims scores all pieces, and a head's score is its four columns
// added across lanes (sum_stride4, the same value in each).  With more heads
// the columns are the heads and the same accumulator adds three steps, one
// per piece.  The tile leaves lane l holding column l%16 and keys
// 4*(l/16)..+3, which is the B-operand layout of a 16x16x16 step over keys,
// so the softmax stays in the lane and the weights, again as three bf16
// pieces (in the columns, or in three steps), feed
//   O^T[d][c] += sum_key V^T[d][key] * P^T[key][c]
// with V fragments (stored in operand order too, see kv_v_off: two fragments
// per 16-byte lane load, 1 KiB per load) as the A operand; a head's output is
// again the sum of its piece columns.  Keys of a fragment outside the window
// are zeroed (their weight is 0, and 0 * NaN is not) and rows of K outside it
// are masked after the scores.  A lane keeps the running max of its column's
// head; the max moves only when a chunk's exceeds it by more than 8 (base 2,
// so every weight stays below 2^8), and the output is rescaled only when it
// moved for a head that had keys: both sides of the final division use the
// same max, so this changes rounding only.  The running sum covers the lane's
// own keys and is added over the four lanes of a column at the end.  The
// query's loads go out before the first K/V loads, its pieces sit in LDS; K
// and V rotate through three register buffers, so two chunks are in flight
// while one is scored.
//
// TR > 1 (prefill rows, TR = 16 / G): the work-group takes TR consecutive rows
// of the chunk, column c = G*r + g holding head g of row r (pieces in three
// steps), so the rows share each K and V load.  Every column keeps its own
// key range [lo, pos] of its row; the pages cover the first row's window
// start to the last row's position, in one split, and V is zeroed only past
// that range (inside it every key holds data, masked per column by its zero
// weight).  A column that meets a 16-key group with none of its keys before it
// has had any keeps max -inf and sum 0.
//
// NWV = 8 (decode, G <= 4): a work-group of 8 waves walks chunks of two
// pages, wave w taking 16 keys of page w / 4: twice the keys in flight per
// work-group, for few, long splits (the split combine then runs in the O
// projection's prologue).
template <int D, int G, int TR = 1, int NWV = kAttnWaves>
__global__ void __launch_bounds__(NWV * 64) k_attn_mfma(AttnArgs a) {
    static_assert(G <= 16 && TR * G <= 16, "one 16-column tile of query heads");
    static_assert(NWV % 4 == 0 && (NWV == kAttnWaves || TR == 1), "whole pages per chunk; tiled rows use 4 waves");
    constexpr bool PC = G <= 4 && TR == 1;  // pieces in the columns
    constexpr int NP = PC ? 1 : 3;  // steps per 32 dims and per 16 keys
    constexpr int NC = TR * G;      // columns holding a (row, head)
    constexpr int CHK = NWV * 16;   // keys per chunk (one 16-key group per wave)
    constexpr int PPC = NWV / 4;    // pages per chunk
    constexpr int KS = D / 32;  // 16x16x32 steps over d
    constexpr int DT = D / 16;  // 16-row output tiles over d
    constexpr int QU = (KS + NWV - 1) / NWV;  // query steps per wave
    const int s = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
    // tiled: rows b0 .. b0 + nr - 1 (R: the first row's window start and pages)
    const int b0 = TR > 1 ? b * TR : b;
    const int nr = TR > 1 ? min(TR, a.rows - b0) : 1;
    const AttnRow R = attn_row(a, b0);
    const int posl = TR > 1 ? a.p0 + b0 + nr - 1 : R.pos;  // the last key of the work-group
    const int ns_b = TR > 1 ? 1 : R.nsplit;
    if (s >= ns_b) return;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int r16 = lane & 15, q4 = lane >> 4;
    // the lane's column: piece pc of head gc (PC), head r16, or (TR > 1) head gc of row cr
    const int cr = TR > 1 ? r16 / G : 0;
    const int pc = PC ? r16 >> 2 : 0, gc = PC ? r16 & 3 : (TR > 1 ? r16 % G : r16);
    const bool hc = gc < G && pc < 3 && cr < nr;  // the column holds a head (and a piece)
    const int lo = R.lo;
    const int np = TR > 1 ? (posl + 1 - R.origin + kPage - 1) / kPage : R.np;
    const int kb = R.origin + (int)((long long)s * np / ns_b) * kPage;
    const int ke = min(R.origin + (int)((long long)(s + 1) * np / ns_b) * kPage, posl + 1);
    // the column's own key range (columns past the rows take the last row's)
    const int cpos = TR > 1 ? a.p0 + b0 + min(cr, nr - 1) : R.pos;
    const int clo = TR > 1 ? (a.window > 0 ? max(0, cpos - a.window + 1) : 0) : lo;

    __shared__ __align__(16) u32x4 qsh[NP][KS][64];  // B operands of the query pieces, by lane
    __shared__ float wm[NWV][16], wl[NWV][16];
    __shared__ float wacc[NWV][NC][D];

    // the split's chunks and pages; its pages one per lane, looked up once
    const int nch = (ke - kb + CHK - 1) / CHK;
    const int npg = (ke - kb + kPage - 1) / kPage;
    // (an identity table needs no load: the K/V loads can go out at once)
    const int *ptb = R.pt + kb / kPage;
    const int vpg = R.pt_ident ? kb / kPage + min(lane, npg - 1) : ptb[min(lane, npg - 1)];
    // page pi of the split (pi is wave-uniform)
    auto page_of = [&](int pi) -> int {
        pi = min(pi, npg - 1);
        if (R.pt_ident) return kb / kPage + pi;
        return pi < 64 ? __builtin_amdgcn_readlane(vpg, pi) : ptb[pi];
    };
    // buffer loads over the layer's pools: an offset past the pool reads zeros
    // without a memory access, which is how chunks past the split are loaded.
    // Their base offset is 2^31: a layer's pool is smaller (the host refuses
    // 2 GiB), and adding the fragment steps (under 8 KiB) keeps every such
    // offset past the pool without wrapping round to the pool's start.
    constexpr unsigned kPast = 0x80000000u;
    constexpr int kRsrcWord3 = 0x00020000;  // raw (untyped) access
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(R.kvk), (short)0, (int)R.kv_bytes, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(R.kvv), (short)0, (int)R.kv_bytes, kRsrcWord3);
    auto load = [&](int ci, u32x4 (&kr)[KS], u32x2 (&vr)[DT]) {
        // the wave's 16-key group of its page's head block (16 * D elements of K and of V)
        const int pi = ci * PPC + w / 4;
        const unsigned gb = (unsigned)((((long long)page_of(pi) * a.Hk + j) * kPage + (w % 4) * 16) * D * 2);
        const unsigned ko = pi < npg ? gb + lane * 16 : kPast;
        const unsigned vo = pi < npg ? gb + lane * 16 : kPast;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kr[ks] = __builtin_amdgcn_raw_buffer_load_b128(rk, (int)(ko + ks * 1024), 0, 0);
        // one 16-byte load per lane holds its fragments of output tiles 2p and 2p + 1
#pragma unroll
        for (int dp = 0; dp < DT / 2; ++dp) {
            const u32x4 t = __builtin_amdgcn_raw_buffer_load_b128(rv, (int)(vo + dp * 1024), 0, 0);
            vr[2 * dp] = u32x2{t[0], t[1]};
            vr[2 * dp + 1] = u32x2{t[2], t[3]};
        }
    };
    // the query's loads first (wave w: steps w, w+4, ...; lane l: its column's
    // head, d = ks*32 + 8*q4..+7), so its pieces are made while K and V load
    float qx[QU][8];
#pragma unroll
    for (int u = 0; u < QU; ++u) {
        const int ks = min(w + u * NWV, KS - 1);
        const int qrow = TR > 1 ? b0 + min(cr, nr - 1) : b;
        const float *qp = a.q + (long long)qrow * a.Hq * D + (long long)(j * G + min(gc, G - 1)) * D + ks * 32 + 8 * q4;
        const f32x4 x0 = *reinterpret_cast<const f32x4 *>(qp);
        const f32x4 x1 = *reinterpret_cast<const f32x4 *>(qp + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            qx[u][e] = x0[e];
            qx[u][4 + e] = x1[e];
        }
    }
    u32x4 k0r[KS], k1r[KS], k2r[KS];
    u32x2 v0r[DT], v1r[DT], v2r[DT];
    load(0, k0r, v0r);
    load(1, k1r, v1r);  // (past a one-chunk split: zeros without a memory access; the count of loads stays fixed)
#pragma unroll
    for (int u = 0; u < QU; ++u) {
        const int ks = w + u * NWV;
        if (ks >= KS) break;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
            u32x4 pq;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                pq[e] = bf16_piece2(qx[u][2 * e] * a.scale, qx[u][2 * e + 1] * a.scale, PC ? pc : p, hc);
            qsh[p][ks][lane] = pq;
        }
    }
    lds_barrier();

    float m = -INFINITY, l = 0.f;
    f32x4 acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // one wave chunk: keys k0..k0+15 with at least one in [lo, ke) (none past the split)
    auto chunk = [&](int ci, const u32x4 (&kr)[KS], const u32x2 (&vr)[DT]) {
        const int k0 = kb + ci * CHK + w * 16;
        if (ci >= nch || k0 + 15 < lo || k0 >= ke) return;
        f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int p = 0; p < NP; ++p)
                sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[ks]),
                                                             __builtin_bit_cast(bf16x8, qsh[p][ks][lane]), sc, 0, 0,
                                                             0);
        const int key0 = k0 + 4 * q4;
        float sv[4];
        bool vin[4], cin[4];  // in the work-group's range (V holds data); in the column's
        float cm = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            vin[i] = key0 + i >= lo && key0 + i < ke;
            cin[i] = TR > 1 ? key0 + i >= clo && key0 + i <= cpos : vin[i];
            const float full = PC ? sum_stride4(sc[i]) : sc[i];  // the head's score
            sv[i] = cin[i] ? full : -INFINITY;
            cm = fmaxf(cm, sv[i]);
        }
        cm = fmaxf(cm, __shfl_xor(cm, 16, 64));
        cm = fmaxf(cm, __shfl_xor(cm, 32, 64));
        const float mn = cm > m + 8.f ? cm : m;
        // 1 where the max stays, 0 on the wave's first chunk (tiled: 1 while a column has no keys)
        const float f = (TR > 1 && mn == -INFINITY) ? 1.f : exp2_fast(m - mn);
        const bool rescale = __builtin_amdgcn_ballot_w64(mn != m && m != -INFINITY) != 0;
        float pv[4], ps = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pv[i] = cin[i] ? exp2_fast(sv[i] - mn) : 0.f;
            ps += pv[i];
        }
        l = l * f + ps;
        m = mn;
        u32x2 pb[NP];
#pragma unroll
        for (int p = 0; p < NP; ++p)
#pragma unroll
            for (int h = 0; h < 2; ++h) pb[p][h] = bf16_piece2(pv[2 * h], pv[2 * h + 1], PC ? pc : p, hc);
        // keys outside the window read zeros from V (their weight is 0, and 0 * NaN is not)
        const bool all_in = __builtin_amdgcn_ballot_w64(!(vin[0] && vin[1] && vin[2] && vin[3])) == 0;
        u32x2 vm[DT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) vm[dt] = vr[dt];
        if (!all_in) {  // (wave-uniform: a window's edge chunks only)
            const uint32_t m0 = (vin[0] ? 0xFFFFu : 0u) | (vin[1] ? 0xFFFF0000u : 0u);
            const uint32_t m1 = (vin[2] ? 0xFFFFu : 0u) | (vin[3] ? 0xFFFF0000u : 0u);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) vm[dt] = u32x2{vm[dt][0] & m0, vm[dt][1] & m1};
        }
        if (rescale) {  // (wave-uniform)
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) acc[dt] = acc[dt] * f;
        }
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int p = 0; p < NP; ++p)
                acc[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, vm[dt]),
                                                                    __builtin_bit_cast(s16x4, pb[p]), acc[dt], 0, 0, 0);
    };

    if (nch == 1) {
        chunk(0, k0r, v0r);
    } else {
        // chunk ci lives in buffer ci % 3; the loads of chunk ci + 2 go out before
        // chunk ci is scored.  Every round issues the same loads (chunks past the
        // split read zeros without touching memory), so the waits stay exact.
        for (int ci = 0; ci < nch; ci += 3) {
            load(ci + 2, k2r, v2r);
            chunk(ci, k0r, v0r);
            load(ci + 3, k0r, v0r);
            chunk(ci + 1, k1r, v1r);
            load(ci + 4, k1r, v1r);
            chunk(ci + 2, k2r, v2r);
        }
    }
    // the lane's sum covers its own keys: add the column's four lanes
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    if constexpr (PC) {  // a head's output: its piece columns added (columns 0..G-1 hold them)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[dt][i] = sum_stride4(acc[dt][i]);
    }

    // merge the waves in wave order (a wave with no keys has m = -inf, l = 0);
    // columns 0..G-1 are the heads (with PC: piece 0 of each, holding the sums)
    if (q4 == 0) {
        wm[w][r16] = m;
        wl[w][r16] = l;
    }
    if (r16 < NC)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) wacc[w][r16][dt * 16 + 4 * q4 + i] = acc[dt][i];
    lds_barrier();

    const int ns = ns_b;
    for (int idx = tid; idx < NC * D; idx += NWV * 64) {
        const int g = idx / D, d = idx % D;  // (tiled: column g = G * row + head)
        if (TR > 1 && g / G >= nr) continue;
        float M = wm[0][g];
#pragma unroll
        for (int x = 1; x < NWV; ++x) M = fmaxf(M, wm[x][g]);
        float L = 0.f, A = 0.f;
#pragma unroll
        for (int x = 0; x < NWV; ++x) {
            const float f = exp2_fast(wm[x][g] - M);
            L += wl[x][g] * f;
            A += wacc[x][g][d] * f;
        }
        if (TR > 1) {
            a.o[(long long)(b0 + g / G) * a.Hq * D + (long long)(j * G + g % G) * D + d] = A / L;
        } else if (ns == 1) {
            a.o[(long long)b * a.Hq * D + (long long)(j * G + g) * D + d] = A / L;
        } else {
            float *pp = R.part + (((long long)j * R.s_cap + s) * G + g) * (D + 4);
            if (d == 0) { pp[0] = M; pp[1] = L; }
            pp[4 + d] = A;
        }
    }
}

// Fold the splits of one (slot, query head) together.  grid: x = query head,
// y = slot; 256 threads.  Wave w owns splits w, w+4, w+8, ...: it issues the
// loads of their unnormalised outputs together with the (max, sum) pairs, so
// the kernel waits for memory once.  Every split's weight exp2(M_s - M) / L
// is then formed from the pairs (thread s holds split s) and kept in LDS, each
// wave sums its splits' weighted outputs, and the four partial sums are added
// in wave order.  Slots with one split were finished by k_attn.
template <int D, int G, int NB>
__device__ __forceinline__ void attn_merge_body(const AttnArgs &a, const AttnRow &R, int h, int b, int ns) {
    constexpr int VE = D >= 64 ? D / 64 : 1;
    constexpr int VL = D / VE;
    constexpr int NWV = 4;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int j = h / G, g = h % G;
    const long long stride = (long long)G * (D + 4);  // floats between consecutive splits
    const float *base = R.part + ((long long)j * R.s_cap * G + g) * (D + 4);

    __shared__ float fs[kMaxSplits];
    __shared__ float red[NWV][2];
    __shared__ float pacc[NWV][D];

    // issue everything: this thread's (max, sum) pair and the wave's outputs
    // (split indices clamped to the last split, so every load is in bounds)
    const int dl = (lane < VL ? lane : 0) * VE;
    const f32x2 ml = *reinterpret_cast<const f32x2 *>(base + min(tid, ns - 1) * stride);
    float v[NB][VE];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
        const float *px = base + min(w + u * NWV, ns - 1) * stride + 4 + dl;
        if constexpr (VE == 2) {
            const f32x2 t = *reinterpret_cast<const f32x2 *>(px);
            v[u][0] = t[0];
            v[u][1] = t[1];
        } else {
            v[u][0] = *px;
        }
    }
    const float Ms = tid < ns ? ml[0] : -INFINITY;
    float mx = wave_max(Ms);
    if (lane == 0) red[w][0] = mx;
    lds_barrier();
    mx = fmaxf(fmaxf(red[0][0], red[1][0]), fmaxf(red[2][0], red[3][0]));
    const float f = tid < ns ? exp2_fast(Ms - mx) : 0.f;
    const float ls = wave_sum(tid < ns ? f * ml[1] : 0.f);
    if (lane == 0) red[w][1] = ls;
    lds_barrier();
    const float L = (red[0][1] + red[1][1]) + (red[2][1] + red[3][1]);
    fs[tid] = f / L;  // 0 past the last split
    lds_barrier();

    float acc[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[e] = 0.f;
#pragma unroll
    for (int u = 0; u < NB; ++u) {
        const int sx = w + u * NWV;
        // a clamped (repeated) split has weight 0 here; fs is 0 past ns
        const float fw = fs[min(sx, kMaxSplits - 1)];
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[e] = sx < ns ? fmaf(fw, v[u][e], acc[e]) : acc[e];
    }
    if (lane < VL)
#pragma unroll
        for (int e = 0; e < VE; ++e) pacc[w][dl + e] = acc[e];
    lds_barrier();
    if (tid < D)
        a.o[(long long)b * a.Hq * D + (long long)h * D + tid] =
            (pacc[0][tid] + pacc[1][tid]) + (pacc[2][tid] + pacc[3][tid]);
}

template <int D, int G>
__global__ void __launch_bounds__(256) k_attn_merge(AttnArgs a) {
    const int h = blockIdx.x, b = blockIdx.y;
    const AttnRow R = attn_row(a, b);
    const int ns = R.nsplit;
    if (ns <= 1) return;
    // per-wave split count, rounded up to one of three batch depths (block-uniform)
    const int nbw = (ns + 3) / 4;
    if (nbw <= 4) attn_merge_body<D, G, 4>(a, R, h, b, ns);
    else if (nbw <= 16) attn_merge_body<D, G, 16>(a, R, h, b, ns);
    else attn_merge_body<D, G, kMaxSplits / 4>(a, R, h, b, ns);
}

}  // namespace pn
