// pn_wide.hpp - prefill of many prompt rows of one sequence at once ("Engine
// Architecture", chunked prefill: the prompt's positions go through each layer
// together, so every weight is read once per chunk).  Included only by
// pn_lib.hip.
//
// The decode GEMM takes at most 16 rows, so a chunk there re-reads every
// weight each 16 tokens.  Here a chunk of up to kWideRows rows goes through
// each projection as one matrix product on the matrix cores (k_wgemm), with
// the steps around it as plain row kernels: RMSNorm into MFMA-ready planes,
// RoPE + K/V append, SwiGLU, the residual add and the per-row argmax.  Dense
// models with bf16, int8 or Q8_0 weights and an fp32 or bf16 cache take this
// path.
#pragma once
#include "pn_kernels.hpp"

namespace pn {

constexpr int kWideRows = 256;   // most rows of one wide chunk
constexpr int kWideSplitMax = 8; // most K splits of one wide GEMM

// Y_s[r][n] = sum over k in split s of A[r][k] * W[n][k], for the P planes of
// A (the bf16 pieces whose sum is the fp32 input, or one bf16 plane); int8
// weights: times the row scale sc[n]; Q8_0 weights: each 32-wide block's
// product times that block's scale of row n.
//   W: packed tiles [n_tiles][KT][1 KiB]; bf16: 16 rows x 32 k, lane l holds
//      row l & 15, k 8*(l >> 4) .. +7 (the 16x16x32 operand layout); int8:
//      16 rows x 64 k of biased codes, lane l row l & 15, k 16*(l >> 4) .. +15;
//      Q8_0: the same, with each lane's first 8 codes in block 0 of the tile
//      and its last 8 in block 1 (blk_pos order), and the scale tiles
//      [n_tiles][KT][16 rows][2 blocks] fp16 at sc.
//   A: planes [P][rows][lda] bf16 (int8 and Q8_0 weights: one plane of f16,
//      Q8_0 in blk_pos order), lda >= KT * tile width, zero from K up to lda.
//   Y: split s, matrix z at y[z] + s * y_split, [r][ldy] fp32; rows < R and
//      n < N are written.
// grid: one dimension, work-group id = (W group * A groups + A group) * nzs +
// zs, with zs = matrix * nsplit + split varying fastest: work-groups are
// dealt to the XCDs in id order, so with 8 (or 4) values of zs each XCD's L2
// holds the A slice of one split instead of all of A; a W group is WGW tiles
// (8, 14 or 16: 128, 224 or 256 rows), an A group 128 rows; 512 threads (two
// waves per SIMD: one computes while the other waits on LDS).  Wave w
// computes weight tiles (WGW/2)*(w & 1) .. +WGW/2-1 against row tiles
// 2*(w >> 1), +1 of the group (WGW accumulators): the wider group reads a
// third fewer LDS bytes per output, for products with rows enough to fill the
// chip without splitting K; 14 tiles fill whole rounds of compute units where
// 16 would not.  A k step's WGW weight and 8*NA row fragments (1 KiB each) go
// from memory straight into a ring of LDS stages (each wave loads an eighth
// of them, rounded up); S - 1 steps are in flight while the work-group computes one, at
// one barrier per step, so the loads in flight take no registers.  Tiles past
// n_tiles and rows past R load clamped (in bounds) and are not stored.
struct WGemmArgs {
    const uint8_t *w[2];
    const float *sc[2];  // int8 weights: the rows' scales (padded to tiles); Q8_0: the scale tiles; else null
    float *y[2];
    long long y_split;  // floats between the splits' outputs
    const uint16_t *a;
    long long a_plane;  // elements between the planes of A
    int lda, R, N, n_tiles, KT, ldy, nsplit;
    int nzs, gx;  // matrices * nsplit; A groups
    // Grouped experts (ecnt null: one product over R rows).  Work-groups
    // [e * per_e, (e + 1) * per_e) are expert e's: its rows are the ecnt[e]
    // packed rows of A from row eoff[e] (at most R), its outputs the same rows
    // of y, its matrices start ew bytes per expert after w[z], its scales es
    // bytes per expert after sc[z].  A group past the expert's rows does no work.
    const int *ecnt, *eoff;
    long long ew, es;
    int per_e;
};

// Row fragments per row tile and k step: the P bf16 planes, or for int8 and
// block-quantised weights (f16 rows) the 32-wide blocks of the step's tile:
// two for int8 and Q8_0 (64-wide tiles), four for Q4_0 (128-wide).
__host__ __device__ constexpr int wgemm_na(int WT, int P) {
    return WT == WT_Q4 ? 4 : ((WT == WT_I8 || WT == WT_Q8) ? 2 : P);
}
// Block formats: bytes of one weight tile's scale tile per k step (16 rows x
// the tile's blocks x fp16: 64 for Q8_0, 128 for Q4_0), and of block scales
// per stage, after its fragments: each of the 8 waves loads 256 (a dword per
// lane: 4 or 2 weight tiles' scale tiles); the first WGW tiles' are the
// work-group's (waves past them load copies).
__host__ __device__ constexpr int wgemm_sbt(int WT) { return blockq(WT) ? 32 * tile_blocks(WT) : 0; }
__host__ __device__ constexpr int wgemm_scb(int WT) { return blockq(WT) ? 2048 : 0; }
// Fragments (1 KiB each) of one k step of a work-group that owns WGW weight
// tiles and 8 row tiles: the weight tiles, then every row tile's NA fragments.
__host__ __device__ constexpr int wgemm_frags(int WT, int P, int WGW) { return WGW + 8 * wgemm_na(WT, P); }
// Loads per wave per k step: the fragments shared over 8 waves, rounded up
// (with 14 weight tiles the last loads repeat a fragment into a slot nobody
// reads, so that every wave issues the same number and its waits count right).
__host__ __device__ constexpr int wgemm_lpw(int WT, int P, int WGW) { return (wgemm_frags(WT, P, WGW) + 7) / 8; }
// Bytes of one stage of the LDS ring, and the stages: as many k steps as fit
// 128 KiB (Q8_0, whose stages also hold scales: 144 KiB; Q4_0, with four row
// fragments per row tile: 160 KiB), at most 8.
__host__ __device__ constexpr int wgemm_stage_bytes(int WT, int P, int WGW) {
    return 8 * wgemm_lpw(WT, P, WGW) * 1024 + wgemm_scb(WT);
}
__host__ __device__ constexpr int wgemm_budget(int WT) { return (WT == WT_Q4 ? 160 : (WT == WT_Q8 ? 144 : 128)) * 1024; }
__host__ __device__ constexpr int wgemm_stages(int WT, int P, int WGW) {
    return wgemm_budget(WT) / wgemm_stage_bytes(WT, P, WGW) < 8 ? wgemm_budget(WT) / wgemm_stage_bytes(WT, P, WGW) : 8;
}
__host__ __device__ constexpr int wgemm_lds(int WT, int P, int WGW) {
    return wgemm_stages(WT, P, WGW) * wgemm_stage_bytes(WT, P, WGW);
}

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from global memory straight into LDS (lane i's at dst +
// 16*i), and the wait for all but the newest n of this wave's loads and for
// its LDS reads, then the work-group barrier.  Their bodies exist only in the
// device pass (the host compiler has neither the instruction nor the asm).
__device__ __forceinline__ void lds_dma16(const void *src, lds_void *dst) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
#endif
}
// The same with 4 bytes per lane (lane i's at dst + 4*i).
__device__ __forceinline__ void lds_dma4(const void *src, lds_void *dst) {
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(src, dst, 4, 0, 0);
#endif
}
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
#endif
}
__device__ __forceinline__ void wait_vm_all() {
#if defined(__HIP_DEVICE_COMPILE__)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#endif
}

template <int WT, int P, int WGW>
__global__ void __launch_bounds__(512, 1) k_wgemm(WGemmArgs g) {
    constexpr int NA = wgemm_na(WT, P), TK = tile_k(WT);
    constexpr int S = wgemm_stages(WT, P, WGW), FR = wgemm_frags(WT, P, WGW), LPW = wgemm_lpw(WT, P, WGW);
    constexpr int WWT = WGW / 2;  // weight tiles per wave
    constexpr bool BQ = blockq(WT);
    constexpr int NB = BQ ? tile_blocks(WT) : 1;  // blocks per tile (block formats)
    constexpr int SBT = wgemm_sbt(WT);            // bytes of a tile's scales per k step
    constexpr int SB = wgemm_stage_bytes(WT, P, WGW);
    constexpr int LPS = LPW + (BQ ? 1 : 0);  // loads per wave per k step
    static_assert(WGW % 2 == 0 && S >= 3, "two waves share a row tile's weight tiles; three stages at least");
    static_assert(!BQ || WGW * SBT <= wgemm_scb(WT), "the scale area holds the work-group's scale tiles");
    // [S][SB]: W tiles 0..WGW-1, then A [row tile][plane] (1 KiB each), then (Q8_0) the scales
    extern __shared__ __align__(16) uint8_t ring[];
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int id = blockIdx.x, R = g.R;
    long long roff = 0, wofs = 0, sofs = 0;  // grouped: the expert's first row, matrix and scale offsets
    if (g.ecnt) {
        const int ex = id / g.per_e;
        id -= ex * g.per_e;
        R = g.ecnt[ex];
        roff = g.eoff[ex];
        wofs = ex * g.ew;
        sofs = ex * g.es;
    }
    const int zs = id % g.nzs, rest = id / g.nzs;
    const int gxi = rest % g.gx, gyi = rest / g.gx;
    const int z = zs / g.nsplit, s = zs % g.nsplit;
    if (gxi * 128 >= R) return;  // (grouped: a row group past the expert's rows; uniform)
    const int kt0 = (int)((long long)s * g.KT / g.nsplit), kt1 = (int)((long long)(s + 1) * g.KT / g.nsplit);
    const int wt0 = gyi * WGW + WWT * (wv & 1);  // first weight tile the wave computes
    const int rt0 = gxi * 8 + 2 * (wv >> 1);  // first row tile the wave computes
    // The wave loads fragments wv*LPW .. +LPW-1 of every stage: a W tile
    // (clamped to the matrix) or a (row tile, plane) of A (rows clamped to R);
    // a slot past the FR fragments takes a copy of the last one.
    const uint8_t *src[LPW];
    int stride[LPW];  // bytes per k step
#pragma unroll
    for (int q = 0; q < LPW; ++q) {
        const int f = min(wv * LPW + q, FR - 1);
        if (f < WGW) {
            src[q] = g.w[z] + wofs + (long long)min(gyi * WGW + f, g.n_tiles - 1) * g.KT * 1024 + lane * 16;
            stride[q] = 1024;
        } else {
            // bf16: plane p, k 8*(l >> 4) of the step; int8, Q8_0, Q4_0: block p, positions
            // (TK / 4)*(l >> 4) + 8p (the blk_pos order of the tile)
            const int rt = (f - WGW) / NA, p = (f - WGW) % NA;
            const long long r = roff + min((gxi * 8 + rt) * 16 + (lane & 15), R - 1);
            const long long e = (WT == WT_I8 || BQ) ? r * g.lda + (TK / 4) * (lane >> 4) + 8 * p
                                                    : p * g.a_plane + r * g.lda + 8 * (lane >> 4);
            src[q] = reinterpret_cast<const uint8_t *>(g.a + e);
            stride[q] = TK * 2;
        }
    }
    // Block formats: this lane's dword of the stage's scales: byte 256*wv + 4*lane
    // is dword lane % (SBT / 4) of local weight tile ((256 / SBT)*wv + lane / (SBT / 4))
    // mod WGW (clamped to the matrix); the tile's row r holds bytes 2*NB*r .. +2*NB-1
    const uint8_t *ssrc = nullptr;
    if constexpr (BQ) {
        constexpr int DPT = SBT / 4;  // dwords of one tile's scales
        const int t = min(gyi * WGW + ((256 / SBT) * wv + lane / DPT) % WGW, g.n_tiles - 1);
        ssrc = reinterpret_cast<const uint8_t *>(g.sc[z]) + sofs + (long long)t * g.KT * SBT + (lane % DPT) * 4;
    }
    auto issue = [&](int kt, int slot) {  // every call issues LPS loads (k steps past the split re-read the last)
        kt = min(kt, kt1 - 1);
#pragma unroll
        for (int q = 0; q < LPW; ++q)
            lds_dma16(src[q] + (long long)kt * stride[q], (lds_void *)(ring + slot * SB + (wv * LPW + q) * 1024));
        if constexpr (BQ) lds_dma4(ssrc + (long long)kt * SBT, (lds_void *)(ring + slot * SB + 8 * LPW * 1024 + wv * 256));
    };
    f32x4 acc[WWT][2];
#pragma unroll
    for (int i = 0; i < WWT; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // (every split has at least one k step)
#pragma unroll
    for (int st = 0; st < S - 1; ++st) issue(kt0 + st, st);
    for (int kt = kt0; kt < kt1; ++kt) {
        const int slot = (kt - kt0) % S;
        // this wave's loads of step kt have landed (S - 2 later steps may be
        // in flight) and its reads of the previous step are done; then every
        // wave's: the barrier
        wait_vm_barrier<(S - 2) * LPS>();
        u32x4 wf[WWT], af[2][NA];
        const uint8_t *base = ring + slot * SB + lane * 16;
#pragma unroll
        for (int i = 0; i < WWT; ++i) wf[i] = *reinterpret_cast<const u32x4 *>(base + (WWT * (wv & 1) + i) * 1024);
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int p = 0; p < NA; ++p)
                af[j][p] = *reinterpret_cast<const u32x4 *>(base + (WGW + (2 * (wv >> 1) + j) * NA + p) * 1024);
        // the slot of step kt - 1: every wave has read it (it passed the barrier)
        issue(kt + S - 1, (kt - kt0 + S - 1) % S);
        if constexpr (BQ) {
            // the codes widened to f16 (Q8_0 as for int8; Q4_0: the nibbles masked to a
            // byte each, paired into f16 1024 + c, minus 1032); per block h a
            // matrix-core step from zero with the rows as the A operand (so the lane
            // holds weight row l & 15, whose block scales it reads), scaled and added
            // in fp32 in block order
            const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
            const uint8_t *sbase = ring + slot * SB + 8 * LPW * 1024 + (lane & 15) * (2 * NB);
#pragma unroll
            for (int i = 0; i < WWT; ++i) {
                const uint8_t *sp = sbase + (WWT * (wv & 1) + i) * SBT;
                float d[NB];
                u32x4 b[NB];
                if constexpr (WT == WT_Q4) {
                    const u32x2 sw = *reinterpret_cast<const u32x2 *>(sp);
                    const uint32_t w0 = sw[0], w1 = sw[1];
                    d[0] = half_lo(w0);
                    d[1] = half_hi(w0);
                    d[2] = half_lo(w1);
                    d[3] = half_hi(w1);
                    const f16x2 off = {(_Float16)1032.0f, (_Float16)1032.0f};
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        const uint32_t lo = wf[i][h] & 0x0F0F0F0Fu, hi = (wf[i][h] >> 4) & 0x0F0F0F0Fu;
                        const uint32_t pq[4] = {__builtin_amdgcn_perm(0x64646464u, lo, 0x04010400u),
                                                __builtin_amdgcn_perm(0x64646464u, lo, 0x04030402u),
                                                __builtin_amdgcn_perm(0x64646464u, hi, 0x04010400u),
                                                __builtin_amdgcn_perm(0x64646464u, hi, 0x04030402u)};
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            b[h][c] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, pq[c]) - off);
                    }
                } else {
                    const uint32_t sw = *reinterpret_cast<const uint32_t *>(sp);
                    d[0] = half_lo(sw);
                    d[1] = half_hi(sw);
                    const f16x2 off = {(_Float16)1152.0f, (_Float16)1152.0f};
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, wf[i][c], 0x04010400u);
                        const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, wf[i][c], 0x04030402u);
                        b[c >> 1][2 * (c & 1)] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, lo) - off);
                        b[c >> 1][2 * (c & 1) + 1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, hi) - off);
                    }
                }
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    f32x4 t[NB];
#pragma unroll
                    for (int h = 0; h < NB; ++h)
                        t[h] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, af[j][h]),
                                                                      __builtin_bit_cast(f16x8, b[h]), zero, 0, 0, 0);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        float v = acc[i][j][e];
#pragma unroll
                        for (int h = 0; h < NB; ++h) v = fmaf(d[h], t[h][e], v);
                        acc[i][j][e] = v;
                    }
                }
            }
        } else if constexpr (WT == WT_I8) {
            // biased codes u = q + 128 -> f16 (1024 + u) by a byte permute; minus 1152 leaves q
            const f16x2 off = {(_Float16)1152.0f, (_Float16)1152.0f};
#pragma unroll
            for (int i = 0; i < WWT; ++i) {
                u32x4 b[2];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const uint32_t lo = __builtin_amdgcn_perm(0x64646464u, wf[i][c], 0x04010400u);
                    const uint32_t hi = __builtin_amdgcn_perm(0x64646464u, wf[i][c], 0x04030402u);
                    b[c >> 1][2 * (c & 1)] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, lo) - off);
                    b[c >> 1][2 * (c & 1) + 1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, hi) - off);
                }
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, b[h]),
                                                                           __builtin_bit_cast(f16x8, af[j][h]),
                                                                           acc[i][j], 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int i = 0; i < WWT; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int p = 0; p < P; ++p)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wf[i]),
                                                                            __builtin_bit_cast(bf16x8, af[j][p]),
                                                                            acc[i][j], 0, 0, 0);
        }
    }
    wait_vm_all();  // the clamped tail loads land before the work-group ends
    if (wt0 >= g.n_tiles) return;
    float *y = g.y[z] + (long long)s * g.y_split + roff * g.ldy;  // (grouped: the expert's rows)
    if constexpr (BQ) {
        // lane l holds weight row (output n) l & 15 of tile i for A rows 4*(l >> 4) .. +3 of row tile j
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < WWT; ++i) {
                const int n = (wt0 + i) * 16 + (lane & 15);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = (rt0 + j) * 16 + 4 * (lane >> 4) + e;
                    if (r < R && n < g.N) y[(long long)r * g.ldy + n] = acc[i][j][e];
                }
            }
        return;
    }
    // lane l holds rows 4*(l >> 4) .. +3 of weight tile i (outputs n) for A row (l & 15) of row tile j
    const bool vec = (g.ldy & 3) == 0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int r = (rt0 + j) * 16 + (lane & 15);
        if (r >= R) continue;
#pragma unroll
        for (int i = 0; i < WWT; ++i) {
            const int n0 = (wt0 + i) * 16 + 4 * (lane >> 4);
            float *yp = y + (long long)r * g.ldy + n0;
            f32x4 v = acc[i][j];
            if constexpr (WT == WT_I8) {  // the rows' scales (a table padded to whole tiles)
                const float *scz = reinterpret_cast<const float *>(reinterpret_cast<const uint8_t *>(g.sc[z]) + sofs);
                if (wt0 + i < g.n_tiles) v = v * *reinterpret_cast<const f32x4 *>(scz + n0);
            }
            if (vec && n0 + 3 < g.N) {
                *reinterpret_cast<f32x4 *>(yp) = v;
            } else {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    if (n0 + e < g.N) yp[e] = v[e];
            }
        }
    }
}

// The sum over the nsplit partial outputs (in split order) of element idx;
// all loads are issued before the adds (splits past nsplit add +0).
__device__ __forceinline__ float wide_sum(const float *y, long long split, int nsplit, long long idx) {
    float v[kWideSplitMax];
#pragma unroll
    for (int s = 0; s < kWideSplitMax; ++s) v[s] = s < nsplit ? y[(long long)s * split + idx] : 0.f;
    float t = v[0];
#pragma unroll
    for (int s = 1; s < kWideSplitMax; ++s) t += v[s];
    return t;
}

// The same for elements idx .. idx+3 (16-byte aligned), four per load.
__device__ __forceinline__ f32x4 wide_sum4(const float *y, long long split, int nsplit, long long idx) {
    f32x4 v[kWideSplitMax];
#pragma unroll
    for (int s = 0; s < kWideSplitMax; ++s)
        v[s] = s < nsplit ? *reinterpret_cast<const f32x4 *>(y + (long long)s * split + idx) : f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 t = v[0];
#pragma unroll
    for (int s = 1; s < kWideSplitMax; ++s) t += v[s];
    return t;
}

// Sums of squares of x per row and 1024-column block, [row][kWideSsq]: written
// by the kernels that write x, read by the norm in block order.
constexpr int kWideSsq = 8;  // blocks per row (E <= 8192)

// The sum over the work-group (256 threads) of one value per thread, in a
// fixed order: within each wave, then the four waves' sums in wave order.
__device__ __forceinline__ float wide_block_sum(float v) {
    __shared__ float red[4];
    return block_sum<4>(v, red);
}

// x[r] = tok_embd[token[r]] (bf16 table); a bad id uses row 0 and sets a flag.
// Also the row's block sums of squares.  grid: (cdiv(E, 1024), rows); 256
// threads, four columns each.
__global__ void __launch_bounds__(256) k_w_embed(const uint16_t *__restrict__ embd, const int *__restrict__ tokens,
                                                  float *__restrict__ x, int E, int V, int *err,
                                                  float *__restrict__ ssq) {
    const int r = blockIdx.y, c = (blockIdx.x * 256 + threadIdx.x) * 4;
    int tok = tokens[r];
    if (tok < 0 || tok >= V) {
        if (blockIdx.x == 0 && threadIdx.x == 0) atomicOr(err, ERR_TOKEN);
        tok = 0;
    }
    const uint16_t *src = embd + (long long)tok * E;
    float sq = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        if (c + e < E) {
            const float v = __uint_as_float((uint32_t)src[c + e] << 16);
            x[(long long)r * E + c + e] = v;
            sq += v * v;
        }
    }
    sq = wide_block_sum(sq);
    if (threadIdx.x == 0) ssq[r * kWideSsq + blockIdx.x] = sq;
}

// Row kernels: grid (column blocks, rows) with 256 threads and four
// consecutive columns per thread (one pass, every load issued up front),
// except the norm, which reduces its row first.

// Columns c .. c+3 (c a multiple of 4) of row r of A as MFMA planes, in the
// AReady layout: three bf16 pieces of an fp32 value, or its bf16 rounding, or
// f16 for int8 and Q8_0 weights (Q8_0 in blk_pos order, which keeps runs of 8
// in place).  The four land side by side in every plane: one 8-byte store each.
template <int WT, int AT>
__device__ __forceinline__ void wide_put4(uint16_t *a, long long plane, long long idx, const float (&v0)[4]) {
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = AT == AT_BF16 ? bf16_round(v0[e]) : v0[e];
    long long pos = idx;
    if constexpr (blockq(WT)) {
        constexpr int TK = tile_k(WT);
        pos = (idx & ~(long long)(TK - 1)) | blk_pos(tile_blocks(WT), (int)(idx & (TK - 1)));
    }
    if constexpr (f16_a(WT)) {
        *reinterpret_cast<u32x2 *>(a + pos) =
            u32x2{__builtin_bit_cast(uint32_t, f16x2{(_Float16)v[0], (_Float16)v[1]}),
                  __builtin_bit_cast(uint32_t, f16x2{(_Float16)v[2], (_Float16)v[3]})};
    } else if constexpr (AReady<WT, AT>::PIECES == 1) {
        *reinterpret_cast<u32x2 *>(a + pos) = u32x2{bf16_rne_bits(v[0]) | (bf16_rne_bits(v[1]) << 16),
                                                    bf16_rne_bits(v[2]) | (bf16_rne_bits(v[3]) << 16)};
    } else {
        uint32_t b[3][4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float p0 = bf16_round(v[e]);
            const float r1 = v[e] - p0;
            const float p1 = bf16_round(r1);
            const float p2 = bf16_round(r1 - p1);
            b[0][e] = bf16_rne_bits(p0);
            b[1][e] = bf16_rne_bits(p1);
            b[2][e] = bf16_rne_bits(p2);
        }
#pragma unroll
        for (int p = 0; p < 3; ++p)
            *reinterpret_cast<u32x2 *>(a + p * plane + pos) = u32x2{b[p][0] | (b[p][1] << 16), b[p][2] | (b[p][3] << 16)};
    }
}

// The columns of an A row that a product over K reads: K rounded up to whole
// weight tiles.  The row kernels write those (zeros past K) and leave the
// rest of the lda-wide row alone: no product with this K reads it.
__host__ __device__ constexpr int wide_kp(int WT, int K) { return (K + tile_k(WT) - 1) / tile_k(WT) * tile_k(WT); }

// Row r of A = round_act(RMSNorm(x[r]) * gain), zero from K to wide_kp(K),
// the row's sum of squares added from its block sums in block order.  grid:
// (cdiv(wide_kp(K), 1024), rows).  (WT, AT: the layout of AReady - bf16
// pieces or planes, or f16 rows for int8 and Q8_0 weights.)
template <int WT, int AT>
__global__ void __launch_bounds__(256) k_w_norm(const float *__restrict__ x, int K, const float *__restrict__ gain,
                                                 float eps, const float *__restrict__ ssq, uint16_t *__restrict__ a,
                                                 long long a_plane, int lda) {
    const int r = blockIdx.y, c = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (c >= wide_kp(WT, K)) return;
    const int nb = (K + 1023) / 1024;
    // every load first (K is a multiple of 8, so four columns are all in or all out)
    const bool in = c < K;
    const int cc = in ? c : 0;
    const f32x4 xv = *reinterpret_cast<const f32x4 *>(x + (long long)r * K + cc);
    const f32x4 gv = *reinterpret_cast<const f32x4 *>(gain + cc);
    float sv[kWideSsq];
#pragma unroll
    for (int i = 0; i < kWideSsq; ++i) sv[i] = ssq[r * kWideSsq + min(i, nb - 1)];
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < kWideSsq; ++i)
        if (i < nb) ss += sv[i];
    const float ri = 1.0f / sqrtf(ss / (float)K + eps);
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = in ? (xv[e] * ri) * gv[e] : 0.f;
    wide_put4<WT, AT>(a, a_plane, (long long)r * lda + c, v);
}

// Row r of A = round_act(src[r]) (fp32 rows of ld K), zero from K to
// wide_kp(K).  grid: (cdiv(wide_kp(K), 1024), rows).
template <int WT, int AT>
__global__ void __launch_bounds__(256) k_w_conv(const float *__restrict__ src, int K, uint16_t *__restrict__ a,
                                                 long long a_plane, int lda) {
    const int r = blockIdx.y, c = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (c >= wide_kp(WT, K)) return;
    // (K = heads x head_dim, a multiple of 32: four columns are all in or all out)
    const bool in = c < K;
    const f32x4 sv = *reinterpret_cast<const f32x4 *>(src + (long long)r * K + (in ? c : 0));
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = in ? sv[e] : 0.f;
    wide_put4<WT, AT>(a, a_plane, (long long)r * lda + c, v);
}

// h = silu(gate) * up from the split outputs of the gate / up products, as the
// down projection's A planes (zero from F to wide_kp(F)).  grid:
// (cdiv(wide_kp(F), 1024), rows).
template <int WT, int AT>
__global__ void __launch_bounds__(256) k_w_swiglu(const float *__restrict__ yg, const float *__restrict__ yu,
                                                   long long split, int nsplit, int ldy, int F,
                                                   uint16_t *__restrict__ a, long long a_plane, int lda) {
    const int r = blockIdx.y, c = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (c >= wide_kp(WT, F)) return;
    // four columns per load; past F (ldy is F rounded up to 16) the values are not used
    const long long i = (long long)r * ldy + min(c, ldy - 4);
    const f32x4 gt = wide_sum4(yg, split, nsplit, i), up = wide_sum4(yu, split, nsplit, i);
    float h[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = c + e < F ? (gt[e] / (1.0f + expf(-gt[e]))) * up[e] : 0.f;
    wide_put4<WT, AT>(a, a_plane, (long long)r * lda + c, h);
}

// x[r] += y[r] (summed over the splits), and the new row's block sums of
// squares.  grid: (cdiv(E, 1024), rows).
__global__ void __launch_bounds__(256) k_w_resid(float *__restrict__ x, const float *__restrict__ y, long long split,
                                                  int nsplit, int ldy, int E, float *__restrict__ ssq) {
    const int r = blockIdx.y, c = (blockIdx.x * 256 + threadIdx.x) * 4;
    float sq = 0.f;
    if (c < E) {  // (E a multiple of 8: all four columns in; ldy and the split stride multiples of 16)
        const f32x4 v = wide_sum4(y, split, nsplit, (long long)r * ldy + c);
        f32x4 *xp = reinterpret_cast<f32x4 *>(x + (long long)r * E + c);
        const f32x4 xo = *xp;
        f32x4 xn;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            xn[e] = xo[e] + v[e];
            sq += xn[e] * xn[e];
        }
        *xp = xn;
    }
    sq = wide_block_sum(sq);  // (every thread takes part: no early return above)
    if (threadIdx.x == 0) ssq[r * kWideSsq + blockIdx.x] = sq;
}

// The residual add and the RMSNorm that follows it, in one pass over row r:
// x[r] += y[r] (summed over the splits), then row r of A = round_act(
// RMSNorm(x[r]) * gain), zero from E to wide_kp(E).  The sum of squares is
// formed as k_w_resid and k_w_norm form it (per 1024-column block over its
// 256 threads: within each wave, then the four waves in order; then the
// blocks in order), so the result is bitwise that of the two kernels.  grid:
// rows; 1024 threads: thread t takes columns 4*(t & 255) of blocks t >> 8 and
// (t >> 8) + 4 (E <= 8192).
template <int WT, int AT>
__global__ void __launch_bounds__(1024) k_w_resid_norm(float *__restrict__ x, const float *__restrict__ y,
                                                        long long split, int nsplit, int ldy, int E,
                                                        const float *__restrict__ gain, float eps,
                                                        uint16_t *__restrict__ a, long long a_plane, int lda) {
    static_assert(kWideSsq == 8, "two blocks of 1024 columns per thread");
    __shared__ float red[kWideSsq][4];
    const int r = blockIdx.x, t = threadIdx.x;
    const int q = t & 255, bw = t >> 8, wv = (t >> 6) & 3;
    const int nb = (E + 1023) / 1024;
    // every load first (E a multiple of 8: four columns are all in or all out)
    f32x4 xo[2], yv[2], gv[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int c = (bw + 4 * h) * 1024 + q * 4;
        const int cc = c < E ? c : 0;
        yv[h] = wide_sum4(y, split, nsplit, (long long)r * ldy + cc);
        xo[h] = *reinterpret_cast<const f32x4 *>(x + (long long)r * E + cc);
        gv[h] = *reinterpret_cast<const f32x4 *>(gain + cc);
    }
    f32x4 xn[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int b = bw + 4 * h, c = b * 1024 + q * 4;
        float sq = 0.f;
        if (c < E) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xn[h][e] = xo[h][e] + yv[h][e];
                sq += xn[h][e] * xn[h][e];
            }
            *reinterpret_cast<f32x4 *>(x + (long long)r * E + c) = xn[h];
        }
        sq = wave_sum(sq);
        if ((t & 63) == 0) red[b][wv] = sq;
    }
    lds_barrier();
    float ss = 0.f;
    for (int b = 0; b < nb; ++b) {
        float sb = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) sb += red[b][w];
        ss += sb;
    }
    const float ri = 1.0f / sqrtf(ss / (float)E + eps);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int c = (bw + 4 * h) * 1024 + q * 4;
        if (c >= wide_kp(WT, E)) continue;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = c < E ? (xn[h][e] * ri) * gv[h][e] : 0.f;
        wide_put4<WT, AT>(a, a_plane, (long long)r * lda + c, v);
    }
}

// ---- experts on the wide path.  A chunk's R rows each route to n_used
// experts: entry i = r * n_used + k (ids[i], wts[i] from the router).  The
// entries are packed by expert, in entry order within each (so the packing is
// deterministic): expert e's rows are packed rows eoff[e] .. eoff[e] + ecnt[e]
// - 1, entry i sits at packed row pos[i], and packed row p holds entry ent[p].

// The packing, one work-group of 256 threads: wave w counts the entries of
// experts w, w + 4, ... 64 at a time with a ballot (ranks in entry order);
// then the offsets in expert order.  nent <= kWideRows * 8, X <= 64.
__global__ void __launch_bounds__(256) k_w_route_lists(const int *__restrict__ ids, int nent, int X,
                                                        int *__restrict__ ecnt, int *__restrict__ eoff,
                                                        int *__restrict__ ent, int *__restrict__ pos) {
    __shared__ int cnt[64], off[64];
    __shared__ int rank[kWideRows * 8];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    for (int e = w; e < X; e += 4) {
        int base = 0;
        for (int j0 = 0; j0 < nent; j0 += 64) {
            const int j = j0 + lane;
            const bool m = j < nent && ids[j] == e;
            const unsigned long long bal = __ballot(m);
            if (m) rank[j] = base + __popcll(bal & ((1ull << lane) - 1ull));
            base += __popcll(bal);
        }
        if (lane == 0) cnt[e] = base;
    }
    lds_barrier();
    if (threadIdx.x == 0) {
        int o = 0;
        for (int e = 0; e < X; ++e) {
            off[e] = o;
            ecnt[e] = cnt[e];
            eoff[e] = o;
            o += cnt[e];
        }
    }
    lds_barrier();
    for (int j = threadIdx.x; j < nent; j += 256) {
        const int p = off[ids[j]] + rank[j];
        pos[j] = p;
        ent[p] = j;
    }
}

// Packed row p of the experts' A planes = row ent[p] / n_used of the chunk's
// A planes (its first `cols` columns, a multiple of 8).  grid: (cdiv(cols,
// 2048), packed rows, planes); 256 threads, 8 columns each.
__global__ void __launch_bounds__(256) k_w_gather(const uint16_t *__restrict__ a, long long a_plane, int lda,
                                                   const int *__restrict__ ent, int n_used, int cols,
                                                   uint16_t *__restrict__ ap, long long ap_plane) {
    const int p = blockIdx.y, c = (blockIdx.x * 256 + threadIdx.x) * 8;
    if (c >= cols) return;
    const long long src = (long long)blockIdx.z * a_plane + (long long)(ent[p] / n_used) * lda + c;
    const long long dst = (long long)blockIdx.z * ap_plane + (long long)p * lda + c;
    *reinterpret_cast<u32x4 *>(ap + dst) = *reinterpret_cast<const u32x4 *>(a + src);
}

// out[r] = sum over k of wts[r][k] * (expert output of entry (r, k), summed over
// the splits), in k order (as the decode step's combine).  grid: (cdiv(E,
// 1024), rows); 256 threads, four columns each.
__global__ void __launch_bounds__(256) k_w_moe_combine(const float *__restrict__ y, long long split, int nsplit,
                                                        int ldy, const int *__restrict__ pos,
                                                        const float *__restrict__ wts, int n_used, int E,
                                                        float *__restrict__ out) {
    const int r = blockIdx.y, c = (blockIdx.x * 256 + threadIdx.x) * 4;
    if (c >= E) return;  // (E a multiple of 8: four columns all in or all out)
    f32x4 t = {0.f, 0.f, 0.f, 0.f};
    for (int k = 0; k < n_used; ++k) {
        const int i = r * n_used + k;
        const f32x4 v = wide_sum4(y, split, nsplit, (long long)pos[i] * ldy + c);
        const float wk = wts[i];
#pragma unroll
        for (int e = 0; e < 4; ++e) t[e] += wk * v[e];
    }
    *reinterpret_cast<f32x4 *>(out + (long long)r * E + c) = t;
}

struct WQkvArgs {
    const float *y;     // split outputs [r][ldy], rows in packed order (q, k, v)
    long long split;
    int nsplit, ldy;
    int p0;             // position of row 0
    int Hq, Hk, D, kv_es;
    const float *bias;  // packed order, or null
    const double *omega;
    float *q;           // [r][Hq*D]
    char *kvk, *kvv;    // this layer's K, V pages
    const int *pt;
};

// Per row r at position p0 + r and adjacent pair (2i, 2i+1) of the QKV rows:
// bias, RoPE on q and k by the angle (p0 + r) * omega_(pair in head), whose
// sine and cosine are taken in fp64 and rounded to fp32, then q into q[r] and
// k, v into the cache (layouts as kv_k_off / kv_v_off).  grid: (cdiv(pairs,
// 256), rows); 256 threads, a pair each.
__global__ void __launch_bounds__(256) k_w_qkv(WQkvArgs g) {
    const int r = blockIdx.y, pos = g.p0 + r;
    const int hd = g.Hq * g.D, kd = g.Hk * g.D;
    const int page = g.pt[pos / kPage], t = pos % kPage;
    const bool tiled = g.kv_es == 2;
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < (hd + 2 * kd) / 2) {
        const int r0 = 2 * i;
        const long long yi = (long long)r * g.ldy + r0;
        float y0 = wide_sum(g.y, g.split, g.nsplit, yi), y1 = wide_sum(g.y, g.split, g.nsplit, yi + 1);
        if (g.bias) {
            y0 += g.bias[r0];
            y1 += g.bias[r0 + 1];
        }
        const bool isv = r0 >= hd + kd;
        if (!isv) {
            const double phi = (double)pos * g.omega[(r0 % g.D) >> 1];
            double sn, cs;
            sincos(phi, &sn, &cs);
            rope_pair(y0, y1, make_float2((float)cs, (float)sn));
        }
        if (r0 < hd) {
            g.q[(long long)r * hd + r0] = y0;
            g.q[(long long)r * hd + r0 + 1] = y1;
            return;
        }
        const int rr = isv ? r0 - hd - kd : r0 - hd;
        const int j = rr / g.D, dd = rr % g.D;
        const long long hb = ((long long)page * g.Hk + j) * kPage * g.D;
        if (!isv) {
            const long long off = hb + kv_k_off(tiled, t, dd, g.D);  // dd, dd + 1 adjacent
            if (tiled) {
                *reinterpret_cast<uint32_t *>(g.kvk + off * 2) = bf16_rne_bits(y0) | (bf16_rne_bits(y1) << 16);
            } else {
                reinterpret_cast<float *>(g.kvk)[off] = y0;
                reinterpret_cast<float *>(g.kvk)[off + 1] = y1;
            }
        } else {
            const long long o0 = hb + kv_v_off(tiled, t, dd, g.D), o1 = o0 + kv_v_dim_step(tiled);  // dd even
            if (tiled) {
                reinterpret_cast<uint16_t *>(g.kvv)[o0] = (uint16_t)bf16_rne_bits(y0);
                reinterpret_cast<uint16_t *>(g.kvv)[o1] = (uint16_t)bf16_rne_bits(y1);
            } else {
                reinterpret_cast<float *>(g.kvv)[o0] = y0;
                reinterpret_cast<float *>(g.kvv)[o1] = y1;
            }
        }
    }
}

// out[r] = the index of the largest logit of row r (the lowest on ties; NaN
// logits are skipped and set the NaN flag; -1 when every logit is NaN).
// grid: rows; 256 threads.
__global__ void __launch_bounds__(256) k_w_argmax(const float *logits, long long ld, int N, int *out, int *err) {
    __shared__ float sv[256];
    __shared__ int si[256];
    const int r = blockIdx.x, tid = threadIdx.x;
    const float *lr = logits + (long long)r * ld;
    float best = 0.f;
    int bi = -1;
    bool nan = false;
    for (int n = tid; n < N; n += 256) {  // increasing n: a later equal value never wins
        const float v = lr[n];
        if (v != v) {
            nan = true;
            continue;
        }
        if (bi < 0 || v > best) {
            best = v;
            bi = n;
        }
    }
    if (nan) atomicOr(err, ERR_NAN);
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
    if (tid == 0) out[r] = si[0];
}

}  // namespace pn
