// pn_sample.hpp - on-device token sampling ("Engine Architecture", section
// "Sampling": temperature, repetition penalty, top-k, top-p, softmax, draw).
// Included only by pn_lib.hip.
//
// Per row b of logits:
//   z_i = logits_i / temperature (fp32), then each distinct token of the
//   recent window is penalised (z / r if z > 0, else z * r); -0 counts as +0
//   and NaN as -inf.  A temperature <= 0 is greedy: z = the raw logits and
//   top-k = 1.
//   Tokens rank by z, highest first, equal z by lower index.  top-k keeps the
//   first k; their probabilities are exp(z - z_max), summed in fp64; top-p
//   keeps the shortest prefix whose cumulative probability exceeds top_p times
//   the top-k total; the token is the first of that prefix whose cumulative
//   probability exceeds u times the prefix total, u in [0, 1) being the
//   caller's uniform draw for the row.
//
// Three kernels.  k_sample_keys (many work-groups per row) maps each z to a
// 32-bit key that orders like z and adds its top 12 bits into the row's
// histogram.  k_sample_gather (many work-groups per row) finds in that
// histogram the bin holding the k-th key and, when that bin and the bins
// above it fit the candidate buffer, collects those keys.  k_sample_pick (one
// work-group of 1024 threads per row) clears the histogram for the next call;
// when the top bins did not fit it refines on the lower key bits and gathers
// itself.  It then orders the candidates by (key, index) (counting ranks for
// a few, a bitonic network in LDS for many) and applies top-p and the draw
// with an fp64 prefix sum.
#pragma once
#include "pn_host.hpp"
#include "pn_kernels.hpp"

namespace pn {

constexpr int kSampleBlocks = 64;       // key and gather work-groups per row
constexpr int kSampleTab = 2048;        // recent-token hash table slots
constexpr int kSamplePick = 1024;       // threads of k_sample_pick
constexpr int kSampleU = 16;            // key loads a thread of k_sample_pick keeps in flight
constexpr int kSampleRank = 512;        // up to this many candidates are ranked by counting, not sorted

struct SampleArgs {
    const float *logits;  // [n][V]
    int V, n_recent;
    const int *recent;    // [n][n_recent]; entries < 0 or >= V are empty
    const float *u;       // [n] uniform draws in [0, 1)
    int *ids;             // [n] sampled tokens
    unsigned *keys;       // scratch [n][V]
    unsigned *hist;       // scratch [n][kSampleBins], all zero between calls (k_sample_pick clears it)
    unsigned *cnt;        // scratch [n][2] gather counters, zero between calls (k_sample_pick clears them)
    unsigned long long *cand;  // scratch [n][kSampleCap] candidates from k_sample_gather
    float temp[kMaxSlots], rp[kMaxSlots], top_p[kMaxSlots];
    int top_k[kMaxSlots];
};

// A 32-bit key that orders like z (after -0 -> +0 and NaN -> -inf), and back.
__device__ __forceinline__ unsigned sample_key(float z) {
    if (z != z) z = -INFINITY;
    if (z == 0.f) z = 0.f;
    const unsigned u = __float_as_uint(z);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float sample_value(unsigned k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}
__device__ __forceinline__ unsigned sample_hash(int t) { return ((unsigned)t * 2654435761u) >> 21; }  // 11 bits

// grid: (kSampleBlocks, n); 256 threads.  Work-group x covers tokens
// [x*V/B, (x+1)*V/B) of row y (B = kSampleBlocks), like k_sample_gather.
__global__ void __launch_bounds__(256) k_sample_keys(SampleArgs a) {
    __shared__ int tab[kSampleTab];
    __shared__ unsigned h[kSampleBins];
    const int b = blockIdx.y, tid = threadIdx.x;
    const bool greedy = !(a.temp[b] > 0.f);
    const float temp = a.temp[b], rp = a.rp[b];
    for (int i = tid; i < kSampleTab; i += 256) tab[i] = -1;
    for (int i = tid; i < kSampleBins; i += 256) h[i] = 0;
    __syncthreads();
    const bool pen = !greedy && rp != 1.f && a.n_recent > 0;
    if (pen) {
        for (int i = tid; i < a.n_recent; i += 256) {
            const int t = a.recent[(long long)b * a.n_recent + i];
            if (t < 0 || t >= a.V) continue;
            unsigned s = sample_hash(t);
            // at most kSampleMaxRecent tokens in kSampleTab slots: a free slot always remains
            while (true) {
                const int old = atomicCAS(&tab[s], -1, t);
                if (old == -1 || old == t) break;
                s = (s + 1) & (kSampleTab - 1);
            }
        }
        __syncthreads();
    }
    auto recent = [&](int t) -> bool {
        unsigned s = sample_hash(t);
        while (true) {
            const int v = tab[s];
            if (v == t) return true;
            if (v == -1) return false;
            s = (s + 1) & (kSampleTab - 1);
        }
    };
    const int i0 = (int)((long long)blockIdx.x * a.V / kSampleBlocks);
    const int i1 = (int)((long long)(blockIdx.x + 1) * a.V / kSampleBlocks);
    const float *lg = a.logits + (long long)b * a.V;
    unsigned *keys = a.keys + (long long)b * a.V;
    constexpr int U = 8;  // loads in flight per thread
    for (int ib = i0 + tid; ib < i1; ib += 256 * U) {
        float zv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) zv[u] = lg[min(ib + u * 256, i1 - 1)];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = ib + u * 256;
            if (i >= i1) break;
            float z = zv[u];
            if (!greedy) {
                z = z / temp;
                if (pen && recent(i)) z = z > 0.f ? z / rp : z * rp;
            }
            const unsigned k = sample_key(z);
            keys[i] = k;
            atomicAdd(&h[k >> 20], 1u);
        }
    }
    __syncthreads();
    unsigned *ho = a.hist + (long long)b * kSampleBins;
    for (int i = tid; i < kSampleBins; i += 256) {
        const unsigned c = h[i];
        if (c) atomicAdd(&ho[i], c);
    }
}

// Block-wide exclusive prefix sum of one value per thread (NT threads): an
// inclusive scan within each wave by shuffles, then the waves' totals through
// LDS (buf holds at least NT / 64 entries).
template <int NT, typename T>
__device__ __forceinline__ T sample_scan(T v, T *buf, T &total) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    constexpr int NWV = NT / 64;
    T x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const T y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
    }
    if (lane == 63) buf[w] = x;
    __syncthreads();
    T before = T(0), all = T(0);
#pragma unroll
    for (int i = 0; i < NWV; ++i) {
        const T t = buf[i];
        before += i < w ? t : T(0);
        all += t;
    }
    total = all;
    __syncthreads();
    return before + x - v;
}

// The bin of h (nb bins, nb <= kSampleBins) that holds the k-th largest key,
// given `above` keys above the whole range: thread t looks at the bins
// nb-1-E*t, ..., nb-E*t-E (top down).  Returns the bin and sets gt to the keys
// above it.  The bin is always found when h counts every key of the range and
// above < k <= above + the range's keys; the clamp to 0 only keeps a broken
// histogram inside the array.  Every thread of the block gets the result.
template <int NT>
__device__ __forceinline__ int sample_find(const unsigned *h, int nb, unsigned k, unsigned above, unsigned &gt,
                                           unsigned *ubuf, int *s_digit, unsigned *s_gt) {
    constexpr int E = kSampleBins / NT;
    const int tid = threadIdx.x;
    unsigned c[E], loc = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int bin = nb - 1 - (tid * E + e);
        c[e] = bin >= 0 ? h[bin] : 0u;
        loc += c[e];
    }
    unsigned tot;
    const unsigned ex = sample_scan<NT, unsigned>(loc, ubuf, tot);
    if (tid == 0) *s_digit = -1;
    __syncthreads();
    unsigned run = above + ex;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int bin = nb - 1 - (tid * E + e);
        if (bin >= 0 && run < k && run + c[e] >= k) {
            *s_digit = bin;
            *s_gt = run;
        }
        run += c[e];
    }
    __syncthreads();
    const int d = max(*s_digit, 0);
    gt = *s_gt;
    __syncthreads();
    return d;
}

// A slot in a global list for each lane of the wave that has p: one atomic
// per wave on *ctr, slots in lane order.
__device__ __forceinline__ unsigned sample_append(bool p, unsigned *ctr) {
    const unsigned long long m = __ballot(p);
    if (m == 0ull) return 0u;
    const int lane = threadIdx.x & 63;
    const int leader = __ffsll((long long)m) - 1;
    unsigned base = 0;
    if (lane == leader) base = atomicAdd(ctr, (unsigned)__popcll(m));
    base = __shfl(base, leader, 64);
    return base + (unsigned)__popcll(m & ((1ull << lane) - 1ull));
}

__device__ __forceinline__ int sample_k(const SampleArgs &a, int b) {
    return min(a.temp[b] > 0.f ? a.top_k[b] : 1, a.V);
}

// grid: (kSampleBlocks, n); 256 threads.  Every work-group of a row finds the
// same threshold bin d of the row's histogram (gt keys above it).  When the gt
// keys above d and the bin's keys fit kSampleCap, the work-group appends its
// keys above d to the row's list at [0, gt) and those of bin d at [gt, gt +
// bin size), as (key << 32) | ~index; otherwise it does nothing and
// k_sample_pick narrows the bin further.
__global__ void __launch_bounds__(256) k_sample_gather(SampleArgs a) {
    __shared__ unsigned h[kSampleBins];
    __shared__ unsigned ubuf[4];
    __shared__ int s_digit;
    __shared__ unsigned s_gt;
    const int b = blockIdx.y, tid = threadIdx.x;
    const unsigned *hg = a.hist + (long long)b * kSampleBins;
    for (int i = tid; i < kSampleBins; i += 256) h[i] = hg[i];
    __syncthreads();
    unsigned gt;
    const int d = sample_find<256>(h, kSampleBins, (unsigned)sample_k(a, b), 0u, gt, ubuf, &s_digit, &s_gt);
    if (gt + h[d] > (unsigned)kSampleCap) return;  // (the same for every work-group of the row)
    const int i0 = (int)((long long)blockIdx.x * a.V / kSampleBlocks);
    const int i1 = (int)((long long)(blockIdx.x + 1) * a.V / kSampleBlocks);
    const unsigned *keys = a.keys + (long long)b * a.V;
    unsigned *cnt = a.cnt + 2 * b;
    unsigned long long *cand = a.cand + (long long)b * kSampleCap;
    constexpr int U = 8;
    // (the loop bounds are uniform across the block, so every wave runs every round)
    for (int ib0 = i0; ib0 < i1; ib0 += 256 * U) {
        unsigned kv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) kv[u] = keys[min(ib0 + tid + u * 256, i1 - 1)];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int i = ib0 + tid + u * 256;
            const unsigned top = kv[u] >> 20;
            const bool pa = i < i1 && top > (unsigned)d, pb = i < i1 && top == (unsigned)d;
            const unsigned sa = sample_append(pa, &cnt[0]);
            const unsigned sb = gt + sample_append(pb, &cnt[1]);
            const unsigned long long e = ((unsigned long long)kv[u] << 32) | (0xFFFFFFFFu - (unsigned)i);
            if (pa && sa < (unsigned)kSampleCap) cand[sa] = e;
            if (pb && sb < (unsigned)kSampleCap) cand[sb] = e;
        }
    }
}

// grid: n; kSamplePick threads; dynamic LDS: kSampleCap u64 candidates.
__global__ void __launch_bounds__(kSamplePick) k_sample_pick(SampleArgs a) {
    extern __shared__ __align__(16) unsigned long long cand[];  // (key << 32) | ~index
    __shared__ unsigned h[kSampleBins];
    __shared__ double dbuf[kSamplePick];
    __shared__ unsigned ubuf[kSamplePick];
    __shared__ int s_digit;
    __shared__ unsigned s_gt;
    __shared__ int s_first;
    const int b = blockIdx.x, tid = threadIdx.x, V = a.V;
    const bool greedy = !(a.temp[b] > 0.f);
    const int k = sample_k(a, b);
    const unsigned *keys = a.keys + (long long)b * V;

    // level 0: the row's histogram of the top 12 key bits, which is then
    // cleared (with the gather counters) for the next call
    unsigned *hg = a.hist + (long long)b * kSampleBins;
    for (int i = tid; i < kSampleBins; i += kSamplePick) h[i] = hg[i];
    __syncthreads();
    for (int i = tid; i < kSampleBins; i += kSamplePick) hg[i] = 0u;
    if (tid < 2) a.cnt[2 * b + tid] = 0u;

    // Narrow to the bin holding the k-th largest key: `pre` fixes the top
    // `pbits` bits, `above` counts the keys above that prefix's range.
    unsigned pre = 0, above = 0, bucket = 0;
    int pbits = 0;
    for (int level = 0; level < 3; ++level) {
        const int width = level < 2 ? 12 : 8;
        unsigned gt;
        const int d = sample_find<kSamplePick>(h, 1 << width, (unsigned)k, above, gt, ubuf, &s_digit, &s_gt);
        above = gt;
        bucket = h[d];
        pre = (pre << width) | (unsigned)d;
        pbits += width;
        __syncthreads();
        if (above + bucket <= (unsigned)kSampleCap || pbits == 32) break;
        // the next level's histogram over the keys of this bin
        for (int i = tid; i < kSampleBins; i += kSamplePick) h[i] = 0;
        __syncthreads();
        const int nw = level == 0 ? 12 : 8;
        for (int ib = tid; ib < V; ib += kSamplePick * kSampleU) {
            unsigned kv[kSampleU];
#pragma unroll
            for (int u = 0; u < kSampleU; ++u) kv[u] = keys[min(ib + u * kSamplePick, V - 1)];
#pragma unroll
            for (int u = 0; u < kSampleU; ++u) {
                const unsigned key = kv[u];
                if (ib + u * kSamplePick < V && (key >> (32 - pbits)) == pre)
                    atomicAdd(&h[(key >> (32 - pbits - nw)) & ((1u << nw) - 1)], 1u);
            }
        }
        __syncthreads();
    }

    // The candidates: the keys above the prefix range (fewer than k) and the
    // keys of the prefix bin.  At level 0 k_sample_gather has collected them.
    // At a deeper level that fits they are gathered here in any order (the
    // sort orders them); when they do not fit, the bin's keys are all equal
    // (pbits == 32) and the lowest indices among them are taken, which needs
    // index order: thread t then scans tokens [t*C, (t+1)*C).
    __shared__ unsigned s_na, s_nb;
    if (tid == 0) {
        s_na = 0;
        s_nb = 0;
    }
    __syncthreads();
    int nc;
    if (above + bucket <= (unsigned)kSampleCap) {
        nc = (int)(above + bucket);
        if (pbits == 12) {
            const unsigned long long *cg = a.cand + (long long)b * kSampleCap;
            for (int i = tid; i < nc; i += kSamplePick) cand[i] = cg[i];
        } else {
            for (int ib = tid; ib < V; ib += kSamplePick * kSampleU) {
                unsigned kv[kSampleU];
#pragma unroll
                for (int u = 0; u < kSampleU; ++u) kv[u] = keys[min(ib + u * kSamplePick, V - 1)];
#pragma unroll
                for (int u = 0; u < kSampleU; ++u) {
                    const int i = ib + u * kSamplePick;
                    const unsigned key = kv[u];
                    const unsigned top = pbits == 32 ? key : key >> (32 - pbits);
                    if (i < V && top >= pre) {
                        const unsigned slot = top > pre ? atomicAdd(&s_na, 1u) : above + atomicAdd(&s_nb, 1u);
                        if (slot < (unsigned)kSampleCap)
                            cand[slot] = ((unsigned long long)key << 32) | (0xFFFFFFFFu - (unsigned)i);
                    }
                }
            }
        }
    } else {
        const int C = (V + kSamplePick - 1) / kSamplePick;
        const int t0 = min(V, tid * C), t1 = min(V, t0 + C);
        unsigned na = 0, nbk = 0;
        for (int i = t0; i < t1; ++i) {
            const unsigned key = keys[i];
            na += key > pre;
            nbk += key == pre;
        }
        unsigned ta, tb;
        unsigned oa = sample_scan<kSamplePick, unsigned>(na, ubuf, ta);
        unsigned ob = sample_scan<kSamplePick, unsigned>(nbk, ubuf, tb);
        const unsigned room = (unsigned)kSampleCap - ta;
        for (int i = t0; i < t1; ++i) {
            const unsigned key = keys[i];
            const unsigned long long e = ((unsigned long long)key << 32) | (0xFFFFFFFFu - (unsigned)i);
            if (key > pre) cand[oa++] = e;
            else if (key == pre) {
                if (ob < room) cand[ta + ob] = e;
                ++ob;
            }
        }
        nc = (int)(ta + min(tb, room));
    }
    __syncthreads();

    // Order them, largest first (entries are distinct: the index is part of it).
    // A few: each takes its rank, the count of larger entries, and moves to
    // that place in the upper half of the buffer.  Many: a bitonic network.
    const unsigned long long *srt = cand;
    if (nc <= kSampleRank) {
        unsigned long long *dst = cand + kSampleCap / 2;
        if (tid < nc) {
            const unsigned long long e = cand[tid];
            int r = 0;
            for (int i = 0; i < nc; ++i) r += cand[i] > e;
            dst[r] = e;
        }
        srt = dst;
        __syncthreads();
    } else {
        int P = 1;
        while (P < nc) P <<= 1;
        for (int i = nc + tid; i < P; i += kSamplePick) cand[i] = 0ull;  // below every real entry
        __syncthreads();
        for (int size = 2; size <= P; size <<= 1) {
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                for (int i = tid; i < P / 2; i += kSamplePick) {
                    const int lo = 2 * i - (i & (stride - 1));
                    const int hi = lo + stride;
                    const bool desc = (lo & size) == 0;
                    const unsigned long long x = cand[lo], y = cand[hi];
                    if ((x < y) == desc) {
                        cand[lo] = y;
                        cand[hi] = x;
                    }
                }
                __syncthreads();
            }
        }
    }

    // probabilities of the top k (four per thread), fp64 prefix sums
    const float z0 = sample_value((unsigned)(srt[0] >> 32));
    double w[4], lsum = 0.0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int j = tid * 4 + e;
        const float zj = j < k ? sample_value((unsigned)(srt[j] >> 32)) : 0.f;
        w[e] = j < k ? (zj == z0 ? 1.0 : (double)expf(zj - z0)) : 0.0;  // (all -inf: equal weights)
        lsum += w[e];
    }
    double total;
    const double dex = sample_scan<kSamplePick, double>(lsum, dbuf, total);
    double cum[4];
    double run = dex;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        run += w[e];
        cum[e] = run;
    }
    // top-p: the first position whose cumulative probability exceeds top_p * total
    int np = k;
    const float tp = a.top_p[b];
    if (!greedy && tp < 1.f) {
        if (tid == 0) s_first = k - 1;
        __syncthreads();
        const double lim = (double)tp * total;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = tid * 4 + e;
            if (j < k && cum[e] > lim) atomicMin(&s_first, j);
        }
        __syncthreads();
        np = s_first + 1;
    }
    // the draw: the first position of the prefix whose cumulative probability exceeds u * prefix total
    if (tid == 0) s_first = np - 1;
    __syncthreads();
    const int holder = (np - 1) / 4;  // the thread holding the prefix total
    if (tid == holder) dbuf[0] = cum[(np - 1) % 4];
    __syncthreads();
    const double r = greedy ? 0.0 : (double)a.u[b] * dbuf[0];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int j = tid * 4 + e;
        if (j < np && cum[e] > r) atomicMin(&s_first, j);
    }
    __syncthreads();
    if (tid == 0) a.ids[b] = (int)(0xFFFFFFFFu - (unsigned)(srt[s_first] & 0xFFFFFFFFull));
}

}  // namespace pn
