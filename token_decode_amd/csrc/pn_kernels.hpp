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
constexpr int kNW = 16;        // waves per GEMM work-group
constexpr int kMaxG = 8;       // query heads per KV head

// Layout of one KV head's block of a page (kPage keys x D dims).  An fp32
// cache keeps K by rows [key][dim] and V by columns [dim][key].  A bf16 cache
// keeps both in the operand order of the attention's matrix-core steps, so
// that each load instruction of a wave reads one contiguous run:
//   K: [key / 16][dim / 32][((dim % 32) / 8) * 16 + key % 16][dim % 8]
//      (a 16x16x32 A fragment per 16 keys and 32 dims, 1 KiB),
//   V: [key / 16][dim / 32][((key % 16) / 4) * 16 + dim % 16][(dim % 32) / 16][key % 4]
//      (the 16x16x16 A fragments of 16 keys for dims d..d+15 and d+16..d+31,
//      interleaved per lane, so one 16-byte load per lane reads both: 1 KiB).
// Offsets are in elements from the start of the head's block.
__host__ __device__ constexpr long long kv_k_off(bool tiled, int key, int d, int D) {
    return tiled ? ((long long)((key / 16) * (D / 32) + d / 32) * 64 + ((d % 32) / 8) * 16 + key % 16) * 8 + d % 8
                 : (long long)key * D + d;
}
__host__ __device__ constexpr long long kv_v_off(bool tiled, int key, int d, int D) {
    return tiled ? ((long long)((key / 16) * (D / 32) + d / 32) * 64 + ((key % 16) / 4) * 16 + d % 16) * 8 +
                       ((d % 32) / 16) * 4 + key % 4
                 : (long long)d * kPage + key;
}

// Elements between dim d and d + 1 (d even) of one key in the V layout.
__host__ __device__ constexpr int kv_v_dim_step(bool tiled) { return tiled ? 8 : kPage; }
static_assert(kv_v_off(true, 5, 7, 64) == kv_v_off(true, 5, 6, 64) + kv_v_dim_step(true), "dim step (tiled)");
static_assert(kv_v_off(false, 5, 7, 64) == kv_v_off(false, 5, 6, 64) + kv_v_dim_step(false), "dim step");
static_assert(kv_v_off(true, 17, 31, 128) == kv_v_off(true, 17, 30, 128) + kv_v_dim_step(true), "dim step (tiled)");

// WT_Q8 / WT_Q4: Q8_0 / Q4_0 block-quantised weights (per row, blocks of 32
// along K with one fp16 scale each, and int8 / 4-bit codes)
enum WType { WT_F32 = 0, WT_BF16 = 1, WT_I8 = 2, WT_Q8 = 3, WT_Q4 = 4 };
enum AType { AT_F32 = 0, AT_BF16 = 1 };
enum Pro { PRO_NORM = 0, PRO_LOAD = 1, PRO_CONV = 2, PRO_MERGE = 3 };  // CONV: A = round_act(fp32 rows), no norm
// MERGE (one slot, wave-local): A = round_act(the attention output), its splits
// combined in the prologue from their (max, sum, unnormalised output)
constexpr int kMergeSplits = 8;  // the most attention splits per head the MERGE prologue combines
enum Epi { EPI_QKV = 0, EPI_RESID = 1, EPI_SWIGLU = 2, EPI_LOGITS = 3, EPI_MOE_SWIGLU = 4,
           EPI_MOE_DOWN = 5 };

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__host__ __device__ constexpr int tile_k(int wt) {
    return wt == WT_F32 ? 16 : (wt == WT_BF16 ? 32 : (wt == WT_Q4 ? 128 : 64));
}
// int8 and block-quantised weights are widened to f16 and meet f16 activations
__host__ __device__ constexpr bool f16_a(int wt) { return wt == WT_I8 || wt == WT_Q8 || wt == WT_Q4; }
// block-quantised weights: one fp16 scale per 32 weights of a row
__host__ __device__ constexpr bool blockq(int wt) { return wt == WT_Q8 || wt == WT_Q4; }
// the scale words of one block-quantised tile per lane: its row's fp16 block
// scales (two for Q8_0, four for Q4_0)
template <int WT>
using SReg = typename std::conditional<WT == WT_Q4, u32x2, uint32_t>::type;
// A-fragment bytes per (k-group, row) per tile: a quarter of a tile row's k
__host__ __device__ constexpr int frag_bytes(int wt) { return wt == WT_Q4 ? 64 : (f16_a(wt) ? 32 : 16); }
// 16-byte vectors per A fragment, and 32-wide blocks per tile row (block formats)
__host__ __device__ constexpr int frag_vecs(int wt) { return frag_bytes(wt) / 16; }
__host__ __device__ constexpr int tile_blocks(int wt) { return tile_k(wt) / 32; }
// Block-quantised tiles (16 rows x 64 k for Q8_0, x 128 k for Q4_0: two or four
// 32-wide blocks per row) order each row's k so that MFMA step j of a tile
// covers exactly block j: element e of k-group g (the g-th quarter of the
// tile's positions, 8 per block) is k = 32 (e / 8) + 8 g + e % 8.  blk_pos
// gives the position of k in its tile; A-ready rows of these GEMMs use the
// same order.
__host__ __device__ constexpr int blk_pos(int nblk, int k) {
    return ((k & 31) >> 3) * (8 * nblk) + ((k >> 5) << 3) + (k & 7);
}

// ---------------------------------------------------------------- small helpers

__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}
__device__ __forceinline__ float bf16_round(float f) { return __uint_as_float(bf16_rne_bits(f) << 16); }
__device__ __forceinline__ float bf16_bits_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Wave-wide reductions over the 64 lanes with DPP moves (no LDS traffic); the
// combining order is fixed and the result is read from lane 63, so every lane
// gets the same value.
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within a row
constexpr int kDppBcast15 = 0x142;    // lane 15 of the previous row
constexpr int kDppBcast31 = 0x143;    // lane 31 to rows 2 and 3

template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_f(float ident, float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(ident), __float_as_int(v), CTRL, ROWS, 0xF, false));
}

__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_f<kDppXor1, 0xF>(0.f, v);
    v += dpp_f<kDppXor2, 0xF>(0.f, v);
    v += dpp_f<kDppHalfMirror, 0xF>(0.f, v);
    v += dpp_f<kDppMirror, 0xF>(0.f, v);
    v += dpp_f<kDppBcast15, 0xA>(0.f, v);
    v += dpp_f<kDppBcast31, 0xC>(0.f, v);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_f<kDppXor1, 0xF>(-INFINITY, v));
    v = fmaxf(v, dpp_f<kDppXor2, 0xF>(-INFINITY, v));
    v = fmaxf(v, dpp_f<kDppHalfMirror, 0xF>(-INFINITY, v));
    v = fmaxf(v, dpp_f<kDppMirror, 0xF>(-INFINITY, v));
    v = fmaxf(v, dpp_f<kDppBcast15, 0xA>(-INFINITY, v));
    v = fmaxf(v, dpp_f<kDppBcast31, 0xC>(-INFINITY, v));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Work-group barrier for LDS data only.  __syncthreads() also waits for every
// outstanding global load of the wave (vmcnt(0)), which would drain the weight
// rounds kept in flight across a block's reduction; these barriers only order
// LDS accesses, so they wait for LDS operations alone.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ float readlane_f(float v, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

// the sequence-level error flags of a state
enum { ERR_TOKEN = 1, ERR_NAN = 2 };

// ---------------------------------------------------------------- GEMM

// "A-ready" activation buffers.  A producer (attention combine, SwiGLU) writes
// the next GEMM's input already in the element type its MFMA consumes, so
// the consuming waves load their fragments straight from memory:
//   bf16 weights, fp32 act: 3 planes of bf16 pieces (sum = the fp32 value)
//   bf16 weights, bf16 act: 1 plane of bf16
//   int8 weights (bf16 act): 1 plane of f16
//   Q8_0 / Q4_0 weights (bf16 act): 1 plane of f16, each tile's k in blk_pos order
//   fp32 weights:           1 plane of fp32 (bf16-rounded when act is bf16)
// Plane p of row r starts at element p*plane + r*ld; rows are zero-padded to
// a whole number of k tiles.
template <int WT, int AT>
struct AReady {
    static constexpr int PIECES = (WT == WT_BF16 && AT == AT_F32) ? 3 : 1;
    static constexpr int ES = WT == WT_F32 ? 4 : 2;
    __device__ static void store(void *base, long long plane, long long idx, float v) {
        if constexpr (AT == AT_BF16) v = bf16_round(v);
        if constexpr (WT == WT_F32) {
            reinterpret_cast<float *>(base)[idx] = v;
        } else if constexpr (f16_a(WT)) {
            // (rows and planes hold whole tiles, so idx % TK is the k within the tile)
            if constexpr (blockq(WT)) {
                constexpr int TK = tile_k(WT);
                idx = (idx & ~(long long)(TK - 1)) | blk_pos(tile_blocks(WT), (int)(idx & (TK - 1)));
            }
            reinterpret_cast<_Float16 *>(base)[idx] = (_Float16)v;
        } else if constexpr (PIECES == 1) {
            reinterpret_cast<uint16_t *>(base)[idx] = (uint16_t)bf16_rne_bits(v);
        } else {
            const float p0 = bf16_round(v);
            const float r1 = v - p0;
            const float p1 = bf16_round(r1);
            const float p2 = bf16_round(r1 - p1);
            uint16_t *b = reinterpret_cast<uint16_t *>(base);
            b[idx] = (uint16_t)bf16_rne_bits(p0);
            b[plane + idx] = (uint16_t)bf16_rne_bits(p1);
            b[2 * plane + idx] = (uint16_t)bf16_rne_bits(p2);
        }
    }
};

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
    int B;                  // dense: slots
    int nblk;               // row blocks of NTW tiles (per expert)
    int tpw;                // the most row blocks a work-group takes (work-group x takes
                            // blocks [x*nblk/gx, (x+1)*nblk/gx) of its expert)
    const float *x;         // PRO_NORM: residual [slot][K]
    const float *gain;      // PRO_NORM: [K]
    float eps;
    float *ssp;             // sums of squares of x per 16-element tile [slot][ssp_ld]
    int ssp_ld, ssp_n;      // (read by the norm prologue, written by the residual epilogue)
    const void *a;          // PRO_LOAD: A-ready activation planes
    long long a_plane;      // PRO_LOAD: elements per plane
    int lda;                // PRO_LOAD: elements per row (padded K)
    const int *route_ids;   // MoE: [slot][n_used] expert ids
    int n_slots;            // MoE: slots in the step
    int n_used;
    float *out_f32;         // RESID: x; LOGITS: logits (nullable); MOE_DOWN: y rows
    void *out_act;          // SWIGLU / MOE_SWIGLU: A-ready hidden planes
    long long out_plane;    // elements per output plane
    int ld_out;
    float *q_out;           // QKV: q [slot][Hq*D]
    const float *bias;      // QKV: biases [N] in packed row order, or null
    float *kv_new;          // QKV with a Q4 cache: the new k, v rows [slot][2][Hk][D] fp32 (then
                            // quantised into the pages by k_kv_q4); null: append to the cache here
    int Hq, Hk, D;
    int kv_es;              // QKV: bytes per cached element (2 = bf16, 4 = fp32)
    const float2 *rope;     // QKV: (cos, sin) per slot and rotation index [slot][D/2]
    float *am_val;          // LOGITS: per-WG best value [wg][slot]
    int *am_idx;
    int *err[kMaxSlots];    // per slot error flags
    int pos[kMaxSlots];
    char *kvk[kMaxSlots];   // per slot: K pool of this layer
    char *kvv[kMaxSlots];
    const int *pt[kMaxSlots];
    // MERGE prologue: slot 0's attention splits, [Hk][s_cap][G][D+4] floats each
    // (max, sum, 2 pad, unnormalised output); with one split the output is in x
    const float *part;
    int nsplit, s_cap;
};

// fp16 halves of a 32-bit word as floats
__device__ __forceinline__ float half_lo(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (unsigned short)(w & 0xFFFFu));
}
__device__ __forceinline__ float half_hi(uint32_t w) { return (float)__builtin_bit_cast(_Float16, (unsigned short)(w >> 16)); }

// One weight tile times one A fragment.  a holds this lane's A values of the
// tile: 4 fp32, 8 bf16, or 16 / 32 f16 of row (lane & 15).
template <int WT>
__device__ __forceinline__ void mfma_tile(f32x4 &acc, const u32x4 &wv, const u32x4 (&a)[frag_vecs(WT)],
                                          SReg<WT> sv) {
    if constexpr (WT == WT_BF16) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[0]),
                                                      __builtin_bit_cast(bf16x8, wv), acc, 0, 0, 0);
    } else if constexpr (WT == WT_F32) {
        const f32x4 av = __builtin_bit_cast(f32x4, a[0]);
        const f32x4 bw = __builtin_bit_cast(f32x4, wv);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[0], bw[0], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[1], bw[1], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[2], bw[2], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[3], bw[3], acc, 0, 0, 0);
    } else {
        constexpr int NS = frag_vecs(WT);  // f16 MFMA steps per tile (one per block for block formats)
        u32x4 b[NS];
        if constexpr (WT == WT_Q4) {
            // word j holds the 8 codes of step j: codes 0..3 in the low nibbles of
            // its bytes, 4..7 in the high ones.  Two masks give a byte per code, a
            // byte permute pairs them into f16 (1024 + c), minus 1032 leaves c - 8
            // exactly
            const f16x2 off = {(_Float16)1032.0f, (_Float16)1032.0f};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t lo = wv[j] & 0x0F0F0F0Fu, hi = (wv[j] >> 4) & 0x0F0F0F0Fu;
                const uint32_t p[4] = {__builtin_amdgcn_perm(0x64646464u, lo, 0x04010400u),
                                       __builtin_amdgcn_perm(0x64646464u, lo, 0x04030402u),
                                       __builtin_amdgcn_perm(0x64646464u, hi, 0x04010400u),
                                       __builtin_amdgcn_perm(0x64646464u, hi, 0x04030402u)};
#pragma unroll
                for (int q = 0; q < 4; ++q) b[j][q] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, p[q]) - off);
            }
        } else {
            const f16x2 off = {(_Float16)1152.0f, (_Float16)1152.0f};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // byte u -> f16 (1024 + u); minus 1152 leaves the signed code exactly
                const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, wv[i], 0x04010400u);
                const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, wv[i], 0x04030402u);
                b[i >> 1][2 * (i & 1)] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, lo) - off);
                b[i >> 1][2 * (i & 1) + 1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, hi) - off);
            }
        }
        if constexpr (blockq(WT)) {
            // one step per 32-wide block from zero, scaled by the block's fp16
            // scale of this lane's weight row (the output column the lane holds)
            const f32x4 z = {0.f, 0.f, 0.f, 0.f};
            f32x4 t[NS];
#pragma unroll
            for (int j = 0; j < NS; ++j)
                t[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a[j]),
                                                              __builtin_bit_cast(f16x8, b[j]), z, 0, 0, 0);
            // the scales are taken out of their words by shifts and masks: a bit
            // cast of the second word of a two-word vector to f16x2 was compiled
            // here from the first word for both (every block read blocks 0, 1's scales)
            float d[NS];
            if constexpr (NS == 2) {
                d[0] = half_lo(sv);
                d[1] = half_hi(sv);
            } else {
                const uint32_t w0 = sv[0], w1 = sv[1];
                d[0] = half_lo(w0);
                d[1] = half_hi(w0);
                d[2] = half_lo(w1);
                d[3] = half_hi(w1);
            }
#pragma unroll
            for (int j = 0; j < NS; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] = fmaf(d[j], t[j][i], acc[i]);
        } else {
#pragma unroll
            for (int j = 0; j < NS; ++j)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a[j]),
                                                             __builtin_bit_cast(f16x8, b[j]), acc, 0, 0, 0);
        }
    }
}

// Block-wide deterministic sum of one float per thread.
template <int NW>
__device__ __forceinline__ float block_sum(float v, float *redw) {
    v = wave_sum(v);
    const int w = threadIdx.x >> 6;
    lds_barrier();
    if ((threadIdx.x & 63) == 0) redw[w] = v;
    lds_barrier();
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NW; ++i) s += redw[i];
    return s;
}

// RoPE of the pair (y0, y1) by the angle whose (cos, sin) is cs.
__device__ __forceinline__ void rope_pair(float &y0, float &y1, float2 cs) {
    const float a = y0, b = y1;
    y0 = a * cs.x - b * cs.y;
    y1 = a * cs.y + b * cs.x;
}

// Issue the weight loads of one round: KU tiles of each matrix, always the
// same number of loads (tiles past `last` re-read tile `last`), so the
// compiler can wait for exactly the rounds it needs.
template <int WT, int NTW, int KU>
__device__ __forceinline__ void issue_w(u32x4 (&wr)[NTW][KU], const uint8_t *const (&wbase)[NTW], int t_at,
                                        int last) {
#pragma unroll
    for (int i = 0; i < KU; ++i) {
        const int t = min(t_at + i, last);
#pragma unroll
        for (int mt = 0; mt < NTW; ++mt)
            wr[mt][i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(wbase[mt] + (long long)t * 1024));
    }
}

// Block formats: the scales of the same tiles, one word (Q8_0) or two (Q4_0)
// per lane: its weight row's block scales (scale tiles of 4 bytes per block
// and row, [row][block]).
template <int WT, int NTW, int KU>
__device__ __forceinline__ void issue_s(SReg<WT> (&sr)[NTW][KU], const uint8_t *const (&sbase)[NTW], int t_at,
                                        int last) {
    constexpr int SB = 16 * 2 * tile_blocks(WT);  // bytes of one scale tile
#pragma unroll
    for (int i = 0; i < KU; ++i) {
        const int t = min(t_at + i, last);
#pragma unroll
        for (int mt = 0; mt < NTW; ++mt)
            sr[mt][i] = __builtin_nontemporal_load(reinterpret_cast<const SReg<WT> *>(sbase[mt] + (long long)t * SB));
    }
}

// Issue the direct A-fragment loads of one round (A-ready input not staged in
// LDS), with the same clamping.  `arow` is a valid address on every lane; rows
// past `rows` read row 0 and use zeros.
template <int WT, int AT, int KU>
__device__ __forceinline__ void issue_a(u32x4 (&ar)[KU][frag_vecs(WT)], const uint8_t *arow, bool alive,
                                        int t_at, int last) {
    constexpr int TK = tile_k(WT);
#pragma unroll
    for (int i = 0; i < KU; ++i) {
        const int t = min(t_at + i, last);
        const uint8_t *p = arow + (long long)t * TK * AReady<WT, AT>::ES;
#pragma unroll
        for (int v = 0; v < frag_vecs(WT); ++v) {
            const u32x4 x = *reinterpret_cast<const u32x4 *>(p + 16 * v);
            ar[i][v] = alive ? x : u32x4{0, 0, 0, 0};
        }
    }
}

// MFMA over one round: tiles t_at..t_at+n-1 with A from LDS fragments or registers.
// With A in LDS the round is branch-free: lanes past the A rows and tiles past
// n read zero fragments (at zoff), which add nothing; so the compiler can
// overlap one tile's matrix-core steps with the next tile's arithmetic.  A
// dead tile (past the matrix) is multiplied too (it re-reads a live tile of
// its block, and the epilogues store rows below N only), except in the block
// formats, whose scaled steps take more registers when not branched over.
template <int WT, int NTW, int KU, bool ALDS>
__device__ __forceinline__ void compute_round(f32x4 (&acc)[NTW], const u32x4 (&wr)[NTW][KU],
                                              const SReg<WT> (&sr)[NTW][KU], const u32x4 (&ar)[KU][frag_vecs(WT)],
                                              const uint8_t *sa, int zoff, int a_step, int a_base,
                                              const bool (&wlive)[NTW], int t_loc, int n) {
    constexpr int AV = frag_vecs(WT);
#pragma unroll
    for (int i = 0; i < KU; ++i) {
        if constexpr (ALDS) {
            // this lane's fragment of tile t_loc + i: a_base + t * a_step (a dead lane's
            // a_step is 0 and its a_base the zero block); tiles past n read the zero block
            const uint8_t *af = sa + (i < n ? (t_loc + i) * a_step + a_base : zoff);
            u32x4 a[AV];
#pragma unroll
            for (int v = 0; v < AV; ++v) a[v] = *reinterpret_cast<const u32x4 *>(af + 16 * v);
#pragma unroll
            for (int mt = 0; mt < NTW; ++mt)
                if (!blockq(WT) || wlive[mt]) mfma_tile<WT>(acc[mt], wr[mt][i], a, sr[mt][i]);
        } else if (i < n) {
#pragma unroll
            for (int mt = 0; mt < NTW; ++mt)
                if (!blockq(WT) || wlive[mt]) mfma_tile<WT>(acc[mt], wr[mt][i], ar[i], sr[mt][i]);
        }
    }
}

// Write the A values of 8 consecutive k (k0..k0+7, k0 a multiple of 8) of slot
// b into the LDS fragments [kt][k-group][row][FB bytes].
template <int WT, int AT>
__device__ __forceinline__ void put_a8(uint8_t *sa, int rows, int nb, int b, int k0, const float (&v)[8]) {
    constexpr int TK = tile_k(WT);
    constexpr int FB = frag_bytes(WT);
    constexpr int EPG = TK / 4;
    const int kt = k0 / TK, kin = k0 % TK;
    if constexpr (WT == WT_F32) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int gq = kin / EPG + h;
            *reinterpret_cast<f32x4 *>(sa + ((kt * 4 + gq) * rows + b) * FB) =
                f32x4{v[4 * h], v[4 * h + 1], v[4 * h + 2], v[4 * h + 3]};
        }
    } else if constexpr (f16_a(WT)) {
        // k0..k0+7 are 8 consecutive positions in both orders (int8: k; block formats: blk_pos)
        const int pos = blockq(WT) ? blk_pos(tile_blocks(WT), kin) : kin;
        const int gq = pos / EPG, el = pos % EPG;
        u32x4 o;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            o[q] = __builtin_bit_cast(uint32_t, f16x2{(_Float16)v[2 * q], (_Float16)v[2 * q + 1]});
        *reinterpret_cast<u32x4 *>(sa + ((kt * 4 + gq) * rows + b) * FB + el * 2) = o;
    } else {
        const int gq = kin / EPG;
        uint8_t *dst = sa + ((kt * 4 + gq) * rows + b) * FB;
        if constexpr (AReady<WT, AT>::PIECES == 1) {
            u32x4 o;
#pragma unroll
            for (int q = 0; q < 4; ++q) o[q] = bf16_rne_bits(v[2 * q]) | (bf16_rne_bits(v[2 * q + 1]) << 16);
            *reinterpret_cast<u32x4 *>(dst) = o;
        } else {
            u32x4 o0, o1, o2;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                uint32_t w0[2], w1[2], w2[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const float x = v[2 * q + h];
                    const float p0 = bf16_round(x);
                    const float r1 = x - p0;
                    const float p1 = bf16_round(r1);
                    const float p2 = bf16_round(r1 - p1);
                    w0[h] = bf16_rne_bits(p0);
                    w1[h] = bf16_rne_bits(p1);
                    w2[h] = bf16_rne_bits(p2);
                }
                o0[q] = w0[0] | (w0[1] << 16);
                o1[q] = w1[0] | (w1[1] << 16);
                o2[q] = w2[0] | (w2[1] << 16);
            }
            *reinterpret_cast<u32x4 *>(dst) = o0;
            *reinterpret_cast<u32x4 *>(dst + nb * FB) = o1;
            *reinterpret_cast<u32x4 *>(dst + 2 * nb * FB) = o2;
        }
    }
}

// Write the A values of 4 consecutive k (k0..k0+3, k0 a multiple of 4) of slot
// b into the LDS fragments: half of put_a8's fragment.
template <int WT, int AT>
__device__ __forceinline__ void put_a4(uint8_t *sa, int rows, int nb, int b, int k0, const float (&v)[4]) {
    constexpr int TK = tile_k(WT);
    constexpr int FB = frag_bytes(WT);
    constexpr int EPG = TK / 4;
    const int kt = k0 / TK, kin = k0 % TK;
    if constexpr (WT == WT_F32) {
        *reinterpret_cast<f32x4 *>(sa + ((kt * 4 + kin / EPG) * rows + b) * FB) = f32x4{v[0], v[1], v[2], v[3]};
    } else if constexpr (f16_a(WT)) {
        // 4-aligned runs of k are 4 consecutive positions in both orders
        const int pos = blockq(WT) ? blk_pos(tile_blocks(WT), kin) : kin;
        const int gq = pos / EPG, el = pos % EPG;
        u32x2 o;
#pragma unroll
        for (int q = 0; q < 2; ++q)
            o[q] = __builtin_bit_cast(uint32_t, f16x2{(_Float16)v[2 * q], (_Float16)v[2 * q + 1]});
        *reinterpret_cast<u32x2 *>(sa + ((kt * 4 + gq) * rows + b) * FB + el * 2) = o;
    } else {
        const int gq = kin / EPG, el = kin % EPG;
        uint8_t *dst = sa + ((kt * 4 + gq) * rows + b) * FB + el * 2;
        if constexpr (AReady<WT, AT>::PIECES == 1) {
            u32x2 o;
#pragma unroll
            for (int q = 0; q < 2; ++q) o[q] = bf16_rne_bits(v[2 * q]) | (bf16_rne_bits(v[2 * q + 1]) << 16);
            *reinterpret_cast<u32x2 *>(dst) = o;
        } else {
            u32x2 o0, o1, o2;
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                uint32_t w0[2], w1[2], w2[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const float x = v[2 * q + h];
                    const float p0 = bf16_round(x);
                    const float r1 = x - p0;
                    const float p1 = bf16_round(r1);
                    const float p2 = bf16_round(r1 - p1);
                    w0[h] = bf16_rne_bits(p0);
                    w1[h] = bf16_rne_bits(p1);
                    w2[h] = bf16_rne_bits(p2);
                }
                o0[q] = w0[0] | (w0[1] << 16);
                o1[q] = w1[0] | (w1[1] << 16);
                o2[q] = w2[0] | (w2[1] << 16);
            }
            *reinterpret_cast<u32x2 *>(dst) = o0;
            *reinterpret_cast<u32x2 *>(dst + nb * FB) = o1;
            *reinterpret_cast<u32x2 *>(dst + 2 * nb * FB) = o2;
        }
    }
}

// Prologue register budgets of a GEMM variant.  x-prologue: 8-element chunks
// per thread per batch (its first batch's loads go out before any weight
// load): for the norm prologue four rows of 4096 with 16 waves, one with 8
// (more would cost the occupancy of 8-wave groups), two with 4.  A-ready
// staging: fragments per thread per batch, enough for A in one batch up to the
// LDS staging limit (96 KiB) where the registers allow.
__host__ __device__ constexpr int gemm_ch(int nw, int pro) { return (nw == 8 || pro == PRO_CONV) ? 1 : 2; }
__host__ __device__ constexpr int gemm_cha(int wt, int nw) {
    return (96 * 1024 / frag_bytes(wt) + nw * 64 - 1) / (nw * 64) < 12
               ? (96 * 1024 / frag_bytes(wt) + nw * 64 - 1) / (nw * 64)
               : 12;
}
__host__ __device__ constexpr int gemm_spw(int nw) { return (kMaxSlots + nw - 1) / nw; }

// Whether the wave-local prologue fits: each wave loads the A slice of its own
// k tiles (nb slots of x for the norm / conversion prologue, rows A-ready rows
// otherwise) in one batch of the prologue registers.
__host__ __device__ constexpr bool gemm_wave_local_fits(int wt, int pro, int nw, int nb, int rows, int KT) {
    const int per = (KT + nw - 1) / nw;
    if (pro == PRO_NORM || pro == PRO_CONV) {
        const int cpr = (per * tile_k(wt) / 8 + 63) / 64 > 1 ? (per * tile_k(wt) / 8 + 63) / 64 : 1;
        return nb <= gemm_spw(nw) && nb * cpr <= gemm_ch(nw, pro);
    }
    const int cpr = (per * 4 + 63) / 64 > 1 ? (per * 4 + 63) / 64 : 1;
    return rows * cpr <= gemm_cha(wt, nw);
}

// The wave-local conversion prologue over several slots (WL = 2: the O
// projection of a batched step).  Each wave loads its own k tiles of every
// slot's attention output: 64-lane loads of 8-element chunks run over (slot,
// chunk) pairs, so with npr chunks per slot and npr dividing 64 a lane keeps
// one chunk column and takes slot (64 c + lane) / npr in load c.  (The same
// form for the norm prologue, with every slot's sums of squares and the gains
// in registers, spilled in the 16-wave gate/up and LM-head kernels and made
// them slower; it made no difference to QKV.)
constexpr int kWaveRowsMax = 8;  // slots
constexpr int kWaveRowsCh = 4;   // chunk loads per lane
__host__ __device__ constexpr bool gemm_wave_rows_fits(int wt, int pro, int nw, int nb, int KT) {
    const int per = (KT + nw - 1) / nw;
    const int npr = per * tile_k(wt) / 8;
    return pro == PRO_CONV && nb >= 1 && nb <= kWaveRowsMax && npr >= 1 && npr <= 64 && 64 % npr == 0 &&
           nb * npr <= kWaveRowsCh * 64;
}

// Skinny GEMM Y[rows][N] = A[rows][K] * W[N][K]^T for rows <= 16, fused with a
// prologue that supplies A and an epilogue that consumes Y.
// A row block is NTW weight tiles: with PAIR, tile blk of matrices w and w2
// (gate and up); without, tiles NTW*blk .. NTW*blk+NTW-1 of w.  Work-group x
// owns the consecutive row blocks [x*tpw, x*tpw + tpw) (grid z = expert for
// MoE); its NW waves split K and reduce through LDS, so every work-group owns
// whole output tiles.
// A comes from LDS (ALDS: the prologue builds it there once for all the
// group's blocks) or, for large A-ready inputs, straight from memory.
// Memory accesses are issued early: the prologue's loads first, then two
// rounds of weight tiles and the epilogue's inputs, so one round trip covers
// the prologue; weight rounds then ping-pong between two register buffers, and
// the next block's first rounds are in flight during this block's reduction
// and epilogue.
// WL: 0 = the work-group's shared prologue, 1 = wave-local for one batch of
// the prologue registers, 2 = the wave-local conversion prologue over up to
// kWaveRowsMax slots (gemm_wave_rows_fits).
template <int WT, int AT, int PRO, int EPI, int NTW, bool PAIR, int NW, bool ALDS, int WL>
__global__ void __launch_bounds__(NW * 64) k_gemm(GemmArgs g) {
    static_assert(PRO == PRO_LOAD || ALDS, "the norm prologue stages A in LDS");
    static_assert(!WL || ALDS, "the wave-local prologue stages A in LDS");
    static_assert(PRO != PRO_MERGE || (WL == 1 && EPI == EPI_RESID), "the split combine runs in the wave-local prologue");
    static_assert(WL != 2 || PRO == PRO_CONV, "the several-slot wave-local prologue converts x");
    constexpr bool XPRO = PRO == PRO_NORM || PRO == PRO_CONV;  // A built from fp32 rows in g.x
    constexpr bool MPRO = PRO == PRO_MERGE;
    constexpr int NT = NW * 64;
    constexpr int TK = tile_k(WT);
    constexpr int FB = frag_bytes(WT);
    // tiles per matrix per round: two rounds in flight keep 8 KiB per wave
    // outstanding within a 128-register budget (16 waves per CU)
    constexpr int KU = 4 / NTW;
    constexpr int PIECES = AReady<WT, AT>::PIECES;
    constexpr bool MOE = (EPI == EPI_MOE_SWIGLU || EPI == EPI_MOE_DOWN);
    // x-prologue: 8-element chunks per thread per batch (its first batch's loads
    // go out before any weight load): for the norm prologue four rows of 4096
    // with 16 waves, one with 8 (more would cost the occupancy of 8-wave
    // groups), two with 4
    constexpr int CH = WL == 2 ? kWaveRowsCh : gemm_ch(NW, PRO);
    constexpr int CHA = gemm_cha(WT, NW);
    constexpr int SPW = gemm_spw(NW);  // norm prologue: slots whose sums of squares a wave reads
    constexpr int ES = AReady<WT, AT>::ES;
    extern __shared__ __align__(16) uint8_t smem[];

    // (the wave index is uniform: read from lane 0 it lives in a scalar register, so the
    // k range, round counts and tile addresses derived from it are scalar too)
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int ex = blockIdx.z;
    // an equal share (+-1) of the expert's blocks per work-group
    const int blk0 = (int)((long long)blockIdx.x * g.nblk / gridDim.x);
    const int blk1 = (int)((long long)(blockIdx.x + 1) * g.nblk / gridDim.x);
    if (blk0 >= blk1) return;

    __shared__ int s_ent[kMaxSlots];   // MoE: entry (slot*n_used + k) of each gathered row
    __shared__ int s_nb;
    __shared__ float s_rinv[kMaxSlots];

    if constexpr (MOE) {
        if (tid == 0) {
            int n = 0;
            for (int b = 0; b < g.n_slots; ++b)
                for (int k = 0; k < g.n_used; ++k)
                    if (g.route_ids[b * g.n_used + k] == ex) s_ent[n++] = b * g.n_used + k;
            s_nb = n;
        }
        lds_barrier();
    }
    const int nb = MOE ? s_nb : g.B;
    if (nb == 0) return;
    const int rows = nb * PIECES;
    const int am = lane & 15, ag = lane >> 4;
    const bool alive = am < rows;
    uint8_t *sa = smem;  // A fragments [kt][k-group][row][FB bytes], then 256 zero bytes
    const int zoff = ALDS ? (g.KT * 4 * rows * FB + 255) & ~255 : 0;
    const int abytes = ALDS ? zoff + 256 : 0;
    float *red = reinterpret_cast<float *>(smem + abytes);  // [wave][mt][m][n]
    // The zero block: lanes past the A rows, and tiles past the end of a round,
    // read their A fragments here, so a round has no branches.  Every wave
    // writes it before its own reads (a wave's LDS operations run in order; all
    // writers write zeros).
    if (ALDS && lane < 16) *reinterpret_cast<u32x4 *>(sa + zoff + lane * 16) = u32x4{0, 0, 0, 0};
    // LDS offset of this lane's A fragment of k tile t: a_base + t * a_step
    const int a_step = alive ? 4 * rows * FB : 0;
    const int a_base = alive ? (ag * rows + am) * FB : zoff;
    float *C = red + NW * NTW * 256;                          // [mt][m][n]

    // ---- phase 1: the prologue's loads, all issued before any weight load and
    // with a fixed count (addresses clamped, values selected), so that waiting
    // for them never waits for weights
    const int n8 = g.KT * TK / 8;  // 8-element chunks per A row
    // the k tiles of this wave (the waves split K evenly; the last ones may be short or empty)
    const int per = (g.KT + NW - 1) / NW;
    const int wt0 = min(g.KT, wave * per);
    const int wt1 = min(g.KT, wt0 + per);
    // Wave-local prologue: when the A slice of this wave's k tiles fits the
    // registers below, each wave loads and stages only that slice (and works out
    // the norm factors itself), so no wave waits at a work-group barrier for
    // another wave's prologue loads.  The condition is uniform over the group.
    // Load c of a lane covers A row c / cpr, items (c % cpr) * 64 + lane of the
    // row's slice (8-element chunks of x, or A fragments); the divisions are
    // scalar.
    const int nchw = (wt1 - wt0) * TK / 8;  // 8-element chunks of this wave's tiles, per A row
    const int nfw = (wt1 - wt0) * 4;        // A fragments of this wave's tiles, per A row
    const int cpr = XPRO ? max(1, (per * TK / 8 + 63) / 64) : max(1, (per * 4 + 63) / 64);
    constexpr bool wl = WL == 1;
    // WL = 2: chunks per slot (one wave's share, the same for every wave) and
    // this lane's chunk column
    const int npr = per * TK / 8;
    const int jr = WL == 2 ? lane % npr : 0;
    float xv[CH][8], gv[CH][8];
    float ssv[SPW][8];
    u32x4 st[CHA][frag_vecs(WT)];
    if constexpr (WL == 2) {
        const int k0 = wt0 * TK + jr * 8;
        const bool jin = jr < nchw && k0 < g.K;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int b = (c * 64 + lane) / npr;
            const bool in = jin && b < nb;
            const f32x4 *xp = reinterpret_cast<const f32x4 *>(g.x + (long long)(in ? b : 0) * g.K + (in ? k0 : 0));
            // (values of chunks past the rows or K are never used)
            const f32x4 x0 = xp[0], x1 = xp[1];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xv[c][e] = x0[e];
                xv[c][4 + e] = x1[e];
            }
        }
    } else if constexpr (XPRO) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            int b, k0;
            if constexpr (wl) {
                const int j = (c % cpr) * 64 + lane;
                b = j < nchw ? c / cpr : nb;
                k0 = wt0 * TK + j * 8;
            } else {
                const int ch = tid + c * NT;
                b = ch / n8;
                k0 = (ch - b * n8) * 8;
            }
            const bool in = b < nb && k0 < g.K;
            const int sb = in ? (MOE ? s_ent[b] / g.n_used : b) : 0;
            const f32x4 *xp = reinterpret_cast<const f32x4 *>(g.x + (long long)sb * g.K + (in ? k0 : 0));
            // (values of chunks past the rows or K are never used)
            const f32x4 x0 = xp[0], x1 = xp[1];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xv[c][e] = x0[e];
                xv[c][4 + e] = x1[e];
            }
            if constexpr (PRO == PRO_NORM) {
                const f32x4 *gp = reinterpret_cast<const f32x4 *>(g.gain + (in ? k0 : 0));
                const f32x4 g0 = gp[0], g1 = gp[1];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    gv[c][e] = g0[e];
                    gv[c][4 + e] = g1[e];
                }
            }
        }
    }
    if constexpr (PRO == PRO_NORM) {
        // the per-16-element sums of squares of slots wave, wave+NW, ... (at most
        // 512 of them: K <= 8192); wave-local: of every slot
#pragma unroll
        for (int q = 0; q < SPW; ++q) {
            const int b = WL ? q : wave + q * NW;
            const int sb = b < nb ? (MOE ? s_ent[b] / g.n_used : b) : 0;
            const float *sp = g.ssp + (long long)sb * g.ssp_ld;
#pragma unroll
            for (int u = 0; u < 8; ++u) ssv[q][u] = sp[min(lane + 64 * u, g.ssp_n - 1)];  // masked in phase 3
        }
    }
    if constexpr (PRO == PRO_LOAD && ALDS) {
        const int chunksA = g.KT * 4;
#pragma unroll
        for (int c = 0; c < CHA; ++c) {
            int m, f;
            if constexpr (wl) {
                const int j = (c % cpr) * 64 + lane;
                m = j < nfw ? c / cpr : rows;
                f = wt0 * 4 + j;
            } else {
                const int idx = tid + c * NT;
                m = idx / chunksA;
                f = idx - m * chunksA;
            }
            const bool in = m < rows;
            const int s = in ? m / nb : 0, b = in ? m - s * nb : 0;
            const long long r = MOE ? s_ent[b] : b;
            const uint8_t *src = reinterpret_cast<const uint8_t *>(g.a) +
                                 ((long long)s * g.a_plane + r * g.lda + (long long)(in ? f : 0) * (TK / 4)) * ES;
#pragma unroll
            for (int v = 0; v < frag_vecs(WT); ++v)  // (rows past A are never stored)
                st[c][v] = *reinterpret_cast<const u32x4 *>(src + 16 * v);
        }
    }

    // The split-combine prologue (one slot): lane l takes the 4 consecutive k
    // wt0*TK + 4l .. +3 of this wave's slice, dims dd.. of query head h.  It
    // loads every split's (max, sum) and its 4 unnormalised outputs (split
    // indices clamped to the last split), or with one split the attention
    // output itself.
    constexpr int SMX = MPRO ? kMergeSplits : 1;
    f32x2 mml[SMX];
    f32x4 mov[SMX];
    const int mk0 = wt0 * TK + 4 * lane;
    const bool mslice = MPRO && 4 * lane < (wt1 - wt0) * TK;  // this lane's 4 k are in the wave's tiles
    const bool min_ = mslice && mk0 < g.K;                      // ... and below K (the rest of a tile is 0)
    if constexpr (MPRO) {
        const int kk = min_ ? mk0 : 0;
        if (g.nsplit <= 1) {
            mov[0] = *reinterpret_cast<const f32x4 *>(g.x + kk);
        } else {
            const int G = g.Hq / g.Hk;
            const int h = kk / g.D, dd = kk - h * g.D;
            const int jh = h / G, gh = h - jh * G;
            const long long sst = (long long)G * (g.D + 4);  // floats between consecutive splits
            const float *pb = g.part + ((long long)jh * g.s_cap * G + gh) * (g.D + 4);
#pragma unroll
            for (int sx = 0; sx < SMX; ++sx) {
                const float *ps = pb + min(sx, g.nsplit - 1) * sst;
                mml[sx] = *reinterpret_cast<const f32x2 *>(ps);
                mov[sx] = *reinterpret_cast<const f32x4 *>(ps + 4 + dd);
            }
        }
    }

    // epilogue inputs of one block, loaded early by the threads that use them
    // (row r of slot b: the old x for the residual, the (cos, sin) for RoPE,
    // the int8 row scales)
    struct EpIn { float x, s0, s1, b0, b1; float2 cs; int page; };
    auto epi_load = [&](int blk) -> EpIn {
        EpIn e{0.f, 1.f, 1.f, 0.f, 0.f, make_float2(1.f, 0.f), 0};
        if constexpr (EPI == EPI_RESID) {
            if (tid < nb * 16) {
                const int b = tid >> 4, r = blk * 16 + (tid & 15);
                if (r < g.N) e.x = g.out_f32[(long long)b * g.ld_out + r];
                if constexpr (WT == WT_I8) e.s0 = r < g.N ? g.sc[r] : 0.f;
            }
        } else if constexpr (EPI == EPI_QKV) {
            if (tid < nb * 8) {
                const int b = tid >> 3, r0 = blk * 16 + (tid & 7) * 2;
                e.page = g.pt[b][g.pos[b] / kPage];  // the page the k, v rows are appended to
                if (r0 < g.N) {
                    e.cs = g.rope[(long long)b * (g.D / 2) + ((r0 % g.D) >> 1)];
                    if constexpr (WT == WT_I8) { e.s0 = g.sc[r0]; e.s1 = g.sc[r0 + 1]; }
                    if (g.bias) { e.b0 = g.bias[r0]; e.b1 = g.bias[r0 + 1]; }
                }
            }
        } else if constexpr (EPI == EPI_SWIGLU || EPI == EPI_MOE_SWIGLU || EPI == EPI_MOE_DOWN) {
            if constexpr (WT == WT_I8) {
                if (tid < nb * 16) {
                    const int r = blk * 16 + (tid & 15);
                    if (r < g.N) {
                        e.s0 = g.sc[(long long)ex * g.es_stride + r];
                        if constexpr (PAIR) e.s1 = g.sc2[(long long)ex * g.es_stride + r];
                    }
                }
            }
        } else if constexpr (EPI == EPI_LOGITS) {
            if constexpr (WT == WT_I8) {
                if (tid < nb * NTW * 16) {
                    const int c = tid % (NTW * 16);
                    const int r = blk * NTW * 16 + c;
                    if (r < g.N) e.s0 = g.sc[r];
                }
            }
        }
        return e;
    };
    EpIn epc = epi_load(blk0);

    // ---- phase 2: the first block's first two weight rounds (and direct A fragments)
    const int last = max(wt1 - 1, 0);             // clamp target of every load of this wave
    const int rounds = (wt1 - wt0 + KU - 1) / KU;  // rounds with at least one tile
    const uint8_t *mbase[NTW];
#pragma unroll
    for (int mt = 0; mt < NTW; ++mt)
        mbase[mt] = ((PAIR && mt == 1) ? g.w2 : g.w) + (long long)ex * g.ew_stride + lane * 16;
    // block formats: scale tiles (2 bytes per block and row) after each weight
    // tile's scales; this lane reads its row's
    constexpr int SB = 16 * 2 * tile_blocks(WT);
    const uint8_t *sbase0[NTW];
#pragma unroll
    for (int mt = 0; mt < NTW; ++mt)
        sbase0[mt] = reinterpret_cast<const uint8_t *>((PAIR && mt == 1) ? g.sc2 : g.sc) +
                     (long long)ex * g.es_stride * 4 + am * (SB / 16);
    const uint8_t *sbase[NTW];
    auto block_ptrs = [&](int blk, const uint8_t *(&wbase)[NTW], bool (&wlive)[NTW]) {
#pragma unroll
        for (int mt = 0; mt < NTW; ++mt) {
            const int nt = PAIR ? blk : blk * NTW + mt;
            wlive[mt] = nt < g.n_tiles;
            // a dead tile (past the matrix) re-reads the block's first tile
            const long long t0 = (long long)(wlive[mt] ? nt : (PAIR ? blk : blk * NTW)) * g.KT;
            wbase[mt] = mbase[mt] + t0 * 1024;
            if constexpr (blockq(WT)) sbase[mt] = sbase0[mt] + t0 * SB;
        }
    };
    const uint8_t *arow = nullptr;
    if constexpr (!ALDS) {
        long long r = 0, sp = 0;
        if (alive) {
            const int s = am / nb, b = am - s * nb;
            r = MOE ? s_ent[b] : b;
            sp = s;
        }
        arow = reinterpret_cast<const uint8_t *>(g.a) + (sp * g.a_plane + r * g.lda + ag * (TK / 4)) * ES;
    }
    // NR register rounds rotate (NR - 1 in flight while one is multiplied).
    // Three rounds for the 16-wave groups fit their 128 registers with no spill
    // but made every such kernel slower (8 slots: QKV 15.2 -> 16.9 us, gate/up
    // 41.2 -> 43.1 us): the weight stream is not short of loads in flight.
    constexpr int NR = 2;
    u32x4 wr[NR][NTW][KU];
    u32x4 ar[NR][KU][frag_vecs(WT)];
    const uint8_t *wbase[NTW];
    bool wlive[NTW];
    block_ptrs(blk0, wbase, wlive);
    SReg<WT> sr[NR][NTW][KU];  // block scales of the rounds in wr
#pragma unroll
    for (int q = 0; q < NR; ++q)
#pragma unroll
        for (int mt = 0; mt < NTW; ++mt)
#pragma unroll
            for (int i = 0; i < KU; ++i) sr[q][mt][i] = SReg<WT>{};
    auto issue_first = [&]() {
        if constexpr (blockq(WT)) {
#pragma unroll
            for (int q = 0; q < NR; ++q) issue_s<WT, NTW, KU>(sr[q], sbase, wt0 + q * KU, last);
        }
#pragma unroll
        for (int q = 0; q < NR; ++q) {
            issue_w<WT, NTW, KU>(wr[q], wbase, wt0 + q * KU, last);
            if constexpr (!ALDS) issue_a<WT, AT, KU>(ar[q], arow, alive, wt0 + q * KU, last);
        }
    };
    issue_first();


    // ---- phase 3: the prologue's arithmetic
    if constexpr (WL == 2) {
        // this wave's chunks of every slot, straight into LDS
        const int k0 = wt0 * TK + jr * 8;
        if (jr < nchw) {
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                const int b = (c * 64 + lane) / npr;
                if (b >= nb) continue;
                float v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = (k0 + e < g.K) ? xv[c][e] : 0.f;
                if constexpr (AT == AT_BF16) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] = bf16_round(v[e]);
                }
                put_a8<WT, AT>(sa, rows, nb, b, k0, v);
            }
        }
    } else if constexpr (XPRO) {
        if constexpr (wl) {
            // this wave's tiles of every slot: norm factors from all the slot's
            // sums of squares (same order as below), then straight into LDS
            float ri[SPW];
#pragma unroll
            for (int q = 0; q < SPW; ++q) {
                ri[q] = 1.f;
                if constexpr (PRO == PRO_NORM) {
                    if (q < nb) {
                        float v[8];
#pragma unroll
                        for (int u = 0; u < 8; ++u) v[u] = lane + 64 * u < g.ssp_n ? ssv[q][u] : 0.f;
                        float ss = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
                        ss = wave_sum(ss);
                        ri[q] = 1.0f / sqrtf(ss / (float)g.K + g.eps);
                    }
                }
            }
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                const int b = c / cpr, j = (c % cpr) * 64 + lane;
                if (b >= nb || j >= nchw) continue;
                const int k0 = wt0 * TK + j * 8;
                float rb = ri[0];
#pragma unroll
                for (int q = 1; q < SPW; ++q) rb = b == q ? ri[q] : rb;
                float v[8];
                if constexpr (PRO == PRO_NORM) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] = (k0 + e < g.K) ? (xv[c][e] * rb) * gv[c][e] : 0.f;
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] = (k0 + e < g.K) ? xv[c][e] : 0.f;
                }
                if constexpr (AT == AT_BF16) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) v[e] = bf16_round(v[e]);
                }
                put_a8<WT, AT>(sa, rows, nb, b, k0, v);
            }
        } else {
            if constexpr (PRO == PRO_NORM) {
#pragma unroll
                for (int q = 0; q < SPW; ++q) {
                    const int b = wave + q * NW;
                    if (b < nb) {
                        // fixed summation order: per lane, then the wave reduction
                        float v[8];
#pragma unroll
                        for (int u = 0; u < 8; ++u) v[u] = lane + 64 * u < g.ssp_n ? ssv[q][u] : 0.f;
                        float ss = ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
                        ss = wave_sum(ss);
                        if (lane == 0) s_rinv[b] = 1.0f / sqrtf(ss / (float)g.K + g.eps);
                    }
                }
                lds_barrier();
            }
            // batch 0 comes from the phase-1 registers; later batches (more rows
            // than one batch covers) load their own, after the weights
            auto stage_x = [&](int base) {
#pragma unroll
                for (int c = 0; c < CH; ++c) {
                    const int ch = base + tid + c * NT;
                    const int b = ch / n8, k0 = (ch - b * n8) * 8;
                    if (b >= nb) continue;
                    float v[8];
                    if constexpr (PRO == PRO_NORM) {
                        const float ri = s_rinv[b];
#pragma unroll
                        for (int e = 0; e < 8; ++e) v[e] = (k0 + e < g.K) ? (xv[c][e] * ri) * gv[c][e] : 0.f;
                    } else {
#pragma unroll
                        for (int e = 0; e < 8; ++e) v[e] = (k0 + e < g.K) ? xv[c][e] : 0.f;
                    }
                    if constexpr (AT == AT_BF16) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) v[e] = bf16_round(v[e]);
                    }
                    put_a8<WT, AT>(sa, rows, nb, b, k0, v);
                }
            };
            stage_x(0);
            for (int base = CH * NT; base < nb * n8; base += CH * NT) {
#pragma unroll
                for (int c = 0; c < CH; ++c) {
                    const int ch = base + tid + c * NT;
                    const int b = ch / n8, k0 = (ch - b * n8) * 8;
                    const bool in = b < nb && k0 < g.K;
                    const int sb = in ? (MOE ? s_ent[b] / g.n_used : b) : 0;
                    const f32x4 *xp = reinterpret_cast<const f32x4 *>(g.x + (long long)sb * g.K + (in ? k0 : 0));
                    const f32x4 x0 = xp[0], x1 = xp[1];
#pragma unroll
                    for (int e = 0; e < 4; ++e) { xv[c][e] = x0[e]; xv[c][4 + e] = x1[e]; }
                    if constexpr (PRO == PRO_NORM) {
                        const f32x4 *gp = reinterpret_cast<const f32x4 *>(g.gain + (in ? k0 : 0));
                        const f32x4 g0 = gp[0], g1 = gp[1];
#pragma unroll
                        for (int e = 0; e < 4; ++e) { gv[c][e] = g0[e]; gv[c][4 + e] = g1[e]; }
                    }
                }
                stage_x(base);
            }
            lds_barrier();
        }
    } else if constexpr (MPRO) {
        // weights exp2(M_s - M) per split, the head's sum L, and the combined
        // output sum_s (w_s / L) o_s, in split order; straight into LDS (zeros
        // past K)
        if (mslice) {
            float v[4] = {0.f, 0.f, 0.f, 0.f};
            if (!min_) {
            } else if (g.nsplit <= 1) {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = mov[0][e];
            } else {
                float M = -INFINITY;
#pragma unroll
                for (int sx = 0; sx < SMX; ++sx) M = sx < g.nsplit ? fmaxf(M, mml[sx][0]) : M;
                float f[SMX], L = 0.f;
#pragma unroll
                for (int sx = 0; sx < SMX; ++sx) {
                    f[sx] = sx < g.nsplit ? __builtin_amdgcn_exp2f(mml[sx][0] - M) : 0.f;
                    L = sx < g.nsplit ? fmaf(f[sx], mml[sx][1], L) : L;
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = 0.f;
#pragma unroll
                for (int sx = 0; sx < SMX; ++sx) {
                    const float fw = f[sx] / L;
#pragma unroll
                    for (int e = 0; e < 4; ++e) v[e] = sx < g.nsplit ? fmaf(fw, mov[sx][e], v[e]) : v[e];
                }
            }
            if constexpr (AT == AT_BF16) {
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = bf16_round(v[e]);
            }
            put_a4<WT, AT>(sa, rows, nb, 0, mk0, v);
        }
    } else if constexpr (ALDS) {
        if constexpr (wl) {
            // this wave's fragments of every row, straight into LDS
#pragma unroll
            for (int c = 0; c < CHA; ++c) {
                const int m = c / cpr, j = (c % cpr) * 64 + lane;
                if (m >= rows || j >= nfw) continue;
                const int f = wt0 * 4 + j;
                uint8_t *dst = sa + (f * rows + m) * FB;
#pragma unroll
                for (int v = 0; v < frag_vecs(WT); ++v) *reinterpret_cast<u32x4 *>(dst + 16 * v) = st[c][v];
            }
        } else {
            const int chunksA = g.KT * 4;  // fragments per A row
            auto stage_a = [&](int base) {
#pragma unroll
                for (int c = 0; c < CHA; ++c) {
                    const int idx = base + tid + c * NT;
                    const int m = idx / chunksA, f = idx - m * chunksA;
                    if (m >= rows) continue;
                    uint8_t *dst = sa + (f * rows + m) * FB;
#pragma unroll
                    for (int v = 0; v < frag_vecs(WT); ++v) *reinterpret_cast<u32x4 *>(dst + 16 * v) = st[c][v];
                }
            };
            stage_a(0);  // from the phase-1 registers
            for (int base = CHA * NT; base < rows * chunksA; base += CHA * NT) {
#pragma unroll
                for (int c = 0; c < CHA; ++c) {
                    const int idx = base + tid + c * NT;
                    const int m = idx / chunksA, f = idx - m * chunksA;
                    const bool in = m < rows;
                    const int s = in ? m / nb : 0, b = in ? m - s * nb : 0;
                    const long long r = MOE ? s_ent[b] : b;
                    const uint8_t *src = reinterpret_cast<const uint8_t *>(g.a) +
                                         ((long long)s * g.a_plane + r * g.lda + (long long)(in ? f : 0) * (TK / 4)) * ES;
#pragma unroll
                    for (int v = 0; v < frag_vecs(WT); ++v) st[c][v] = *reinterpret_cast<const u32x4 *>(src + 16 * v);
                }
                stage_a(base);
            }
            lds_barrier();
        }
    }

    for (int blk = blk0; blk < blk1; ++blk) {
        // ---- main loop of this block: weight rounds rotate through the NR
        // register buffers.  Every round issues the same loads (clamped past the
        // end), so the waits are exact and NR - 1 rounds are always in flight.
        f32x4 acc[NTW];
#pragma unroll
        for (int mt = 0; mt < NTW; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int r = 0; r < rounds; r += NR) {
#pragma unroll
            for (int q = 0; q < NR; ++q) {
                if (r + q < rounds) {
                    const int ta = wt0 + (r + q) * KU;
                    compute_round<WT, NTW, KU, ALDS>(acc, wr[q], sr[q], ar[q], sa, zoff, a_step, a_base, wlive, ta,
                                                     min(KU, wt1 - ta));
                    if (r + q + NR < rounds) {
                        if constexpr (blockq(WT)) issue_s<WT, NTW, KU>(sr[q], sbase, ta + NR * KU, last);
                        issue_w<WT, NTW, KU>(wr[q], wbase, ta + NR * KU, last);
                        if constexpr (!ALDS) issue_a<WT, AT, KU>(ar[q], arow, alive, ta + NR * KU, last);
                    }
                }
            }
        }
        // the next block's first rounds and epilogue inputs go out before this block's epilogue
        EpIn epn = epc;
        if (blk + 1 < blk1) {
            block_ptrs(blk + 1, wbase, wlive);
            epn = epi_load(blk + 1);
            issue_first();
        }

        // ---- reduce the waves' tiles: red[wave][mt][m][n], then C[mt][m][n]
#pragma unroll
        for (int mt = 0; mt < NTW; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) red[(wave * NTW + mt) * 256 + (4 * ag + i) * 16 + am] = acc[mt][i];
        lds_barrier();
        for (int idx = tid; idx < NTW * 256; idx += NT) {
            float sum = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) sum += red[w * NTW * 256 + idx];
            C[idx] = sum;
        }
        lds_barrier();

        // ---- epilogue.  Y[mt][b][n] = sum over pieces of C[mt][piece*nb + b][n]
        auto Y = [&](int mt, int b, int n) -> float {
            float v = C[mt * 256 + b * 16 + n];
            if constexpr (PIECES == 3) v += C[mt * 256 + (nb + b) * 16 + n] + C[mt * 256 + (2 * nb + b) * 16 + n];
            return v;
        };
        if constexpr (EPI == EPI_QKV) {
            const int hd = g.Hq * g.D, kd = g.Hk * g.D;
            if (tid < nb * 8) {
                const int b = tid >> 3, n0 = (tid & 7) * 2;
                const int r0 = blk * 16 + n0;
                if (r0 < g.N) {
                    float y0 = Y(0, b, n0) * epc.s0;
                    float y1 = Y(0, b, n0 + 1) * epc.s1;
                    if (g.bias) {
                        y0 += epc.b0;
                        y1 += epc.b1;
                    }
                    const int pos = g.pos[b];
                    if (r0 < hd) {
                        rope_pair(y0, y1, epc.cs);
                        g.q_out[(long long)b * hd + r0] = y0;
                        g.q_out[(long long)b * hd + r0 + 1] = y1;
                    } else {
                        const bool isk = r0 < hd + kd;
                        const int rr = isk ? r0 - hd : r0 - hd - kd;
                        const int j = rr / g.D, dd = rr % g.D;
                        if (isk) rope_pair(y0, y1, epc.cs);
                        // the head's block of the page (layouts as kv_k_off / kv_v_off)
                        const long long hb = ((long long)epc.page * g.Hk + j) * kPage * g.D;
                        const int t = pos % kPage;
                        const bool tiled = g.kv_es == 2;
                        if (g.kv_new) {
                            float *kn = g.kv_new + (((long long)b * 2 + (isk ? 0 : 1)) * g.Hk + j) * g.D + dd;
                            kn[0] = y0;
                            kn[1] = y1;
                        } else if (isk) {
                            // dd, dd + 1 are adjacent in both K layouts
                            const long long off = hb + kv_k_off(tiled, t, dd, g.D);
                            if (tiled) {
                                const uint32_t pk = bf16_rne_bits(y0) | (bf16_rne_bits(y1) << 16);
                                *reinterpret_cast<uint32_t *>(g.kvk[b] + off * 2) = pk;
                            } else {
                                reinterpret_cast<float *>(g.kvk[b])[off] = y0;
                                reinterpret_cast<float *>(g.kvk[b])[off + 1] = y1;
                            }
                        } else {
                            // dd is even: dd + 1 sits one dim further in either layout
                            const long long o0 = hb + kv_v_off(tiled, t, dd, g.D);
                            const long long o1 = o0 + kv_v_dim_step(tiled);
                            if (tiled) {
                                reinterpret_cast<uint16_t *>(g.kvv[b])[o0] = (uint16_t)bf16_rne_bits(y0);
                                reinterpret_cast<uint16_t *>(g.kvv[b])[o1] = (uint16_t)bf16_rne_bits(y1);
                            } else {
                                reinterpret_cast<float *>(g.kvv[b])[o0] = y0;
                                reinterpret_cast<float *>(g.kvv[b])[o1] = y1;
                            }
                        }
                    }
                }
            }
        } else if constexpr (EPI == EPI_RESID) {
            // x += y; then this tile's sum of squares of the new x for the next norm
            if (tid < nb * 16) {
                const int b = tid >> 4, n = tid & 15, r = blk * 16 + n;
                float xn = 0.f;
                if (r < g.N) {
                    xn = epc.x + Y(0, b, n) * epc.s0;
                    g.out_f32[(long long)b * g.ld_out + r] = xn;
                }
                float sq = xn * xn;
                sq += __shfl_xor(sq, 8, 64);
                sq += __shfl_xor(sq, 4, 64);
                sq += __shfl_xor(sq, 2, 64);
                sq += __shfl_xor(sq, 1, 64);
                if (n == 0) g.ssp[(long long)b * g.ssp_ld + blk] = sq;
            }
        } else if constexpr (EPI == EPI_SWIGLU || EPI == EPI_MOE_SWIGLU) {
            if (tid < nb * 16) {
                const int b = tid >> 4, n = tid & 15, r = blk * 16 + n;
                if (r < g.N) {
                    const float gt = Y(0, b, n) * epc.s0;
                    const float up = Y(1, b, n) * epc.s1;
                    const float h = (gt / (1.0f + expf(-gt))) * up;
                    const long long row = MOE ? s_ent[b] : b;
                    AReady<WT, AT>::store(g.out_act, g.out_plane, row * g.ld_out + r, h);
                }
            }
        } else if constexpr (EPI == EPI_MOE_DOWN) {
            if (tid < nb * 16) {
                const int b = tid >> 4, n = tid & 15, r = blk * 16 + n;
                if (r < g.N) g.out_f32[(long long)s_ent[b] * g.ld_out + r] = Y(0, b, n) * epc.s0;
            }
        } else if constexpr (EPI == EPI_LOGITS) {
            // the block's logits, and per slot the (value, lowest index) max over
            // its 32 rows by a shuffle reduction within the slot's half-wave
            // (NaN rows are skipped and flag the slot)
            static_assert(NTW * 16 == 32, "one half-wave per slot");
            if (tid < nb * 32) {
                const int b = tid >> 5, c = tid & 31, mt = c >> 4, n = c & 15;
                const int r = (blk * NTW + mt) * 16 + n;
                float v = 0.f;
                int vi = -1;
                bool nan = false;
                if (r < g.N) {
                    const float y = Y(mt, b, n) * epc.s0;
                    if (g.out_f32) g.out_f32[(long long)b * g.N + r] = y;
                    if (y != y) {
                        nan = true;
                    } else {
                        v = y;
                        vi = r;
                    }
                }
#pragma unroll
                for (int o = 16; o > 0; o >>= 1) {
                    const float ov = __shfl_xor(v, o, 64);
                    const int oi = __shfl_xor(vi, o, 64);
                    if (oi >= 0 && (vi < 0 || ov > v || (ov == v && oi < vi))) {
                        v = ov;
                        vi = oi;
                    }
                }
                const unsigned long long bal = __ballot(nan);
                if (c == 0) {
                    g.am_val[(long long)blk * nb + b] = v;
                    g.am_idx[(long long)blk * nb + b] = vi;
                    if ((bal >> (lane & 32)) & 0xFFFFFFFFull) atomicOr(g.err[b], ERR_NAN);
                }
            }
        }
        epc = epn;
        lds_barrier();  // red and C are reused by the next block
    }
}

}  // namespace pn
