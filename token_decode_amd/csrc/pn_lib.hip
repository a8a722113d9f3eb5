// pn_lib.hip - host engine behind the C ABI in include/pn.h.
//
// The engine validates arguments, lays a model and each state out in the
// caller's device buffers, packs weights once, and enqueues one decode step as
// a fixed sequence of kernels on the caller's stream.  It never allocates
// device memory and never synchronizes except in pn_state_check and
// pn_profile_end.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <string>
#include <tuple>
#include <vector>

#include "pn.h"
#include "pn_host.hpp"
#include "pn_launch.hpp"
#include "pn_small.hpp"
#include "pn_sample.hpp"
#include "pn_wide.hpp"

using namespace pn;

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }
inline int cdiv(long long a, long long b) { return (int)((a + b - 1) / b); }

struct Bump {  // offset assignment inside one caller buffer
    size_t off = 0;
    size_t take(size_t n) {
        size_t at = off;
        off = align256(off + n);
        return at;
    }
};

struct Mat {  // one packed matrix (or a stack of experts' matrices)
    int N = 0, K = 0, n_tiles = 0, KT = 0;
    size_t bytes1 = 0;  // bytes of one packed matrix
    size_t off = 0;     // offset of the packed tiles
    size_t soff = 0;    // offset of the scales: int8 row scales, Q8_0 block-scale tiles
    size_t sbytes1 = 0; // bytes of one matrix's scales (0: none)
};

struct LayerOff {
    size_t attn_norm, ffn_norm, router;
    size_t bqkv;  // q, k, v biases [Nqkv] fp32 in packed row order (0: none)
    Mat qkv, o, gate, up, down;
};

struct Plan {
    int gx = 1, gz = 1, nw = 8, nblk = 1, tpw = 1;
    bool a_lds = false;
    bool wave_rows = true;  // the conversion prologue may run per wave over several slots
    size_t lds = 0;
};

}  // namespace

struct pn_model {
    pn_config cfg;
    char *base = nullptr;
    size_t bytes = 0;
    int E, H, Hk, D, F, V, G, X, n_used, wt, at, kvt, pieces, rows_max;
    int Nqkv;
    std::vector<LayerOff> L;
    size_t embd, out_norm;
    Mat out;
    // scratch
    size_t x, q, o, h, y, route_ids, route_w, am_val, am_idx;
    // routing record (pn_model_route_log): step i writes its experts to
    // route_log[(i % route_log_steps)][layer][slot][k]
    int *route_log = nullptr;
    int route_log_steps = 0;
    long long route_log_step = 0;
    // residual trace (pn_model_trace): x entering each layer and leaving the last,
    // [n_layer + 1][max_batch][n_embd] fp32
    float *trace = nullptr;
    size_t samp_keys = 0, samp_hist = 0, samp_cnt = 0, samp_cand = 0;  // pn_sample scratch
    bool samp_dirty = false;  // a pn_sample call stopped before k_sample_pick cleared its histogram
    size_t attn_part = 0, attn_part_row = 0;  // pn_prefill: per-row attention split scratch
    size_t kv_new = 0;                        // Q4 KV cache: the step's new k, v rows [row][2][Hk][D] fp32
    // wide prefill (prefill_chunk > 0): one chunk's rows.  x [C][E], A planes
    // [pieces][C][wlda] bf16, GEMM split outputs (wy_cap floats), q and the
    // attention output [C][H*D]
    size_t wx = 0, wa = 0, wy = 0, wq = 0, wo = 0, wss = 0;
    long long wa_plane = 0, wy_cap = 0;
    // wide prefill of an MoE model: the chunk's routing (ids, weights [C][n_used]),
    // the entries packed by expert (counts and offsets [64], entry of each packed
    // row, packed row of each entry), the packed rows' A planes [pieces][C *
    // n_used][wlda], and the weighted sum of the experts' outputs [C][E]
    size_t wrid = 0, wrw = 0, wecnt = 0, weoff = 0, went = 0, wpos = 0, wap = 0, wyc = 0;
    long long wap_plane = 0;
    int wlda = 0;
    size_t o_bytes = 0, h_bytes = 0, am_count = 0;
    int a_es = 2;                      // bytes per A-ready element
    long long h_plane = 0;
    int h_ld = 0;
    int attn_kps = 0;   // 0 = automatic
    int attn_kind = 0;  // bf16 cache: 0 = automatic, 1 = vector units, 2 = matrix cores
    int attn_combine = 0;  // split combine: 0 = automatic (O prologue where eligible), 1 = merge launch
    int attn_waves = 0;    // matrix-core attention work-groups: 0 = automatic, 4 or 8 waves
    int prologue = 0;      // O projection's conversion prologue over several slots: 0 = per wave where it fits, 1 = shared
    int nw[GK_COUNT] = {8, 8, 8, 8, 8, 8, 16, 16};  // waves per work-group of each GEMM kind (O_MERGE: O's)
    int nw_down = 16;                       // the down projection (K = n_ff) uses GK_RESID too
    bool nw_set = false;                    // waves chosen by the caller (PN_OPT_WAVES_*): no auto choice
    std::map<std::tuple<int, int, int, size_t>, int> occ;  // resident work-groups per CU of a GEMM variant
    size_t rope = 0, omega = 0, ssp = 0;
    int ssp_ld = 0;
    int prof_kernel = -1;
    std::vector<hipEvent_t> ev;
    size_t ev_used = 0;
    // the launches of each kernel class in the most recent step (one per
    // layer, or one), for pn_profile_replay
    struct Replay {
        int kind = -1;  // GEMM kind, or -1 for attention
        GemmArgs g{};
        Plan p{};
        AttnArgs aa{};
        dim3 grid{};
        bool merge = false;
    };
    std::vector<Replay> last[PN_K_COUNT];
    size_t replay_kv = 0, replay_pt = 0;
};

// A page pool shared by states: K pages then V pages, each [layer][page][Hk][kPage][D].
struct pn_pool {
    pn_model *m;
    char *base;
    size_t bytes;
    int n_pages;
    size_t layer_bytes, kpool, vpool;
    std::vector<int> free_pages;  // a stack of free page ids
    int users = 0;                // states created on the pool and not yet freed
    bool closed = false;          // pn_pool_free called: delete with the last state
};

struct pn_state {
    pn_model *m;
    char *base;
    size_t bytes;
    int max_ctx, n_pages, pos, s_cap;
    // K/V pages: the state's own pools (offsets from base), or a shared pool's
    // (offsets from pool->base)
    size_t kpool, vpool, layer_bytes, pt, part, err;
    pn_pool *pool = nullptr;
    std::vector<int> phys;  // pooled: physical page of each logical page, -1 = none
    bool pt_identity = true;  // private state whose page table is the identity
    int kept_from = 0;      // pooled: logical pages below this were returned to the pool
};

namespace {

int dtype_size(int dt) { return dt == PN_F32 ? 4 : (dt == PN_BF16 ? 2 : 1); }

// bytes of one cached key (or value) of one KV head
size_t kv_key_bytes(const pn_model *m) {
    return m->kvt == PN_Q4_0 ? (size_t)q4kv_key_bytes(m->D) : (size_t)m->D * dtype_size(m->kvt);
}

// LDS of one GEMM launch with nw waves: the A fragments of every k tile and a
// 256-byte zero block (when A is staged in LDS), the waves' partial tiles and
// the summed tile.
size_t lds_of(bool a_in_lds, int KT, int rows, int ntw, int fb, int nw) {
    size_t a = a_in_lds ? (((size_t)KT * 4 * rows * fb + 255) & ~(size_t)255) + 256 : 0;  // + zero block
    return a + (size_t)nw * ntw * 1024 + (size_t)ntw * 1024;
}

// A-ready inputs are copied into LDS when they take at most this much.
constexpr size_t kALdsMax = 96 * 1024;
constexpr int kCUs = 256;

bool norm_kind(int kind) {  // A built in LDS from fp32 rows
    return kind == GK_QKV || kind == GK_SWIGLU || kind == GK_LOGITS || kind == GK_MOE_SWIGLU || kind == GK_O ||
           kind == GK_O_MERGE;
}
int ntw_of(int kind) { return (kind == GK_SWIGLU || kind == GK_LOGITS || kind == GK_MOE_SWIGLU) ? 2 : 1; }

struct OccKey {
    int kind, nw, alds;
    size_t lds;
};

// nblk row blocks per expert, gz experts.  As many work-groups as the
// runtime's occupancy keeps resident at once (but no more than blocks), each
// taking an equal share (+-1) of consecutive blocks, so that every compute
// unit streams.  With auto_nw the wave count is the one of {nw, 16} that puts
// more waves on a compute unit (a large A in LDS may leave room for one
// work-group only).
template <typename OccFn>
// nw_cap: the most waves per work-group (block-quantised kernels keep to 8: with
// 16 waves' 128-register budget their block-scale registers spill)
Plan make_plan(int kind, int nblk, int gz, int KT, int rows, int fb, int nw, OccFn occ_of, bool auto_nw = true,
               int slots_in = 1, int nw_cap = 16, bool a_direct = false) {
    auto plan_for = [&](int want) {
        Plan p;
        p.nw = std::min(want, nw_cap);
        p.gz = gz;
        p.nblk = nblk;
        const bool norm = norm_kind(kind);
        p.a_lds = !norm && !a_direct && (size_t)KT * 4 * rows * fb <= kALdsMax;
        // direct A fragments need the larger register budget (f16 fragments take two or four
        // times the registers)
        if (!norm && !p.a_lds) p.nw = fb >= 32 ? 4 : std::min(want, 8);
        p.lds = lds_of(norm || p.a_lds, KT, rows, ntw_of(kind), fb, p.nw);
        while (p.lds > kMaxLds && p.nw > 4) {  // many A rows: fewer waves leave room for them
            p.nw /= 2;
            p.lds = lds_of(norm || p.a_lds, KT, rows, ntw_of(kind), fb, p.nw);
        }
        const int wpc = std::max(1, occ_of(kind, p.nw, p.a_lds, p.lds));
        const long long slots = (long long)kCUs * wpc;
        // as few work-groups as keep every resident slot busy with whole shares;
        // when that leaves compute units idle, one work-group per resident slot
        p.tpw = std::max(1, (int)cdiv((long long)nblk * gz, slots));
        p.gx = cdiv(nblk, p.tpw);
        if ((long long)p.gx * gz < kCUs) {
            p.gx = (int)std::max(1LL, std::min<long long>(nblk, slots / gz));
            p.tpw = cdiv(nblk, p.gx);
        }
        return std::make_pair(p, p.nw * std::min<long long>(wpc, cdiv((long long)p.gx * gz, kCUs)));
    };
    auto best = plan_for(nw);
    if (auto_nw && nw != 16 && nw_cap >= 16) {
        // 16-wave groups also stage four input rows per prologue batch (against one
        // with 8 waves): with several slots they win ties
        auto alt = plan_for(16);
        if (alt.second > best.second || (alt.second == best.second && norm_kind(kind) && slots_in > 1))
            best = alt;
    }
    return best.first;
}

// n_kv_head 0 stands for n_head (the pages' default for the key)
pn_config normalized(const pn_config &c) {
    pn_config n = c;
    if (n.n_kv_head == 0) n.n_kv_head = n.n_head;
    return n;
}

int check_config_n(const pn_config *c);

int check_config(const pn_config *c) {
    if (!c) return fail(PN_EINVAL, "config is NULL");
    pn_config n = normalized(*c);
    return check_config_n(&n);
}

int check_config_n(const pn_config *c) {
    if (c->n_layer < 1 || c->n_embd < 1 || c->n_head < 1 || c->n_kv_head < 1 || c->n_ff < 1 ||
        c->n_vocab < 1)
        return fail(PN_EINVAL, "dimensions must be positive");
    if (c->n_head % c->n_kv_head != 0) return fail(PN_EINVAL, "n_head must be a multiple of n_kv_head");
    {
        const int G = c->n_head / c->n_kv_head;
        if (G != 1 && G != 2 && G != 3 && G != 4 && G != 6 && G != 8)
            return fail(PN_EUNSUPPORTED, "query heads per kv head must be 1, 2, 3, 4, 6 or 8");
    }
    if (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128)
        return fail(PN_EUNSUPPORTED, "head_dim must be 32, 64 or 128");
    if (c->n_expert < 0 || c->n_expert > 64) return fail(PN_EINVAL, "n_expert must be in [0, 64]");
    if (c->n_expert > 0 && (c->n_expert_used < 1 || c->n_expert_used > std::min(8, c->n_expert)))
        return fail(PN_EINVAL, "n_expert_used must be in [1, min(8, n_expert)]");
    if (c->sliding_window < 0) return fail(PN_EINVAL, "sliding_window must be >= 0");
    if (c->n_embd % 8 != 0 || c->n_embd > 8192)
        return fail(PN_EUNSUPPORTED, "n_embd must be a multiple of 8 and at most 8192");
    if (c->n_ctx < 0) return fail(PN_EINVAL, "n_ctx must be >= 0");
    if (!(c->rope_theta > 0.f) || !std::isfinite(c->rope_theta)) return fail(PN_EINVAL, "rope_theta must be > 0");
    if (!(c->rms_norm_eps >= 0.f) || !std::isfinite(c->rms_norm_eps)) return fail(PN_EINVAL, "rms_norm_eps must be >= 0");
    if (c->w_dtype < PN_F32 || c->w_dtype > PN_Q4_0) return fail(PN_EINVAL, "bad w_dtype");
    const bool bq = c->w_dtype == PN_Q8_0 || c->w_dtype == PN_Q4_0;
    if (bq && c->act_dtype != PN_BF16)
        return fail(PN_EUNSUPPORTED, "block-quantised weights need bf16 activations");
    if (bq && (c->n_embd % 32 != 0 || c->n_ff % 32 != 0))
        return fail(PN_EINVAL, "block-quantised rows are whole 32-weight blocks: n_embd and n_ff must be multiples of 32");
    if (c->kv_dtype != PN_F32 && c->kv_dtype != PN_BF16 && c->kv_dtype != PN_Q4_0)
        return fail(PN_EINVAL, "kv_dtype must be F32, BF16 or Q4_0");
    if (c->act_dtype != PN_F32 && c->act_dtype != PN_BF16) return fail(PN_EINVAL, "act_dtype must be F32 or BF16");
    if (c->w_dtype == PN_I8 && c->act_dtype != PN_BF16)
        return fail(PN_EUNSUPPORTED, "int8 weights need bf16 activations");
    if (c->max_batch < 1 || c->max_batch > kMaxSlots) return fail(PN_EINVAL, "max_batch must be in [1, 16]");
    if ((c->rope_neox & ~1) != 0 || (c->qkv_bias & ~1) != 0) return fail(PN_EINVAL, "rope_neox and qkv_bias must be 0 or 1");
    if (c->rope_neox && c->kv_dtype == PN_Q4_0)
        return fail(PN_EUNSUPPORTED, "a Q4 KV cache quantises k in natural dim order: no NeoX RoPE");
    if (c->prefill_chunk < 0 || c->prefill_chunk > kWideRows)
        return fail(PN_EINVAL, "prefill_chunk must be in [0, %d]", kWideRows);
    if (c->prefill_chunk > 0 && c->n_embd > 1024 * kWideSsq)
        return fail(PN_EUNSUPPORTED, "the wide prefill path takes n_embd up to %d", 1024 * kWideSsq);
    if (c->prefill_chunk > 0 && (c->w_dtype == PN_F32 || c->kv_dtype == PN_Q4_0))
        return fail(PN_EUNSUPPORTED,
                    "the wide prefill path needs bf16, int8, Q8_0 or Q4_0 weights and an fp32 or bf16 cache");
    const int pieces = (c->w_dtype == PN_BF16 && c->act_dtype == PN_F32) ? 3 : 1;
    if (c->max_batch * pieces > kMaxRows)
        return fail(PN_EUNSUPPORTED, "max_batch %d too large for this dtype combination (max %d)",
                    c->max_batch, kMaxRows / pieces);
    const int kt = cdiv(c->n_embd, tile_k(c->w_dtype));
    if (lds_of(true, kt, c->max_batch * pieces, 2, frag_bytes(c->w_dtype), 4) > kMaxLds)
        return fail(PN_EUNSUPPORTED, "n_embd %d too large for max_batch %d", c->n_embd, c->max_batch);
    return PN_OK;
}

Mat make_mat(int N, int K, int wt) {
    Mat m;
    m.N = N;
    m.K = K;
    m.n_tiles = cdiv(N, 16);
    m.KT = cdiv(K, tile_k(wt));
    m.bytes1 = (size_t)m.n_tiles * m.KT * 1024;
    // int8: a row scale per row; block formats: a 2-byte scale per block and row
    m.sbytes1 = wt == PN_I8 ? (size_t)m.n_tiles * 16 * 4
                : blockq(wt) ? (size_t)m.n_tiles * m.KT * 16 * 2 * tile_blocks(wt) : 0;
    return m;
}

// Bytes of one source row of K weights in the caller's format.
size_t src_row_bytes(int wt, int K) {
    return wt == PN_Q8_0 ? (size_t)K / 32 * 34 : wt == PN_Q4_0 ? (size_t)K / 32 * 18 : (size_t)K * dtype_size(wt);
}


// Lay out the model buffer; returns its size. Works on a zero base for sizing.
size_t layout_model(pn_model *m) {
    const pn_config &c = m->cfg;
    m->E = c.n_embd;
    m->H = c.n_head;
    m->Hk = c.n_kv_head;
    m->D = c.head_dim;
    m->F = c.n_ff;
    m->V = c.n_vocab;
    m->G = c.n_head / c.n_kv_head;
    m->X = std::max(1, c.n_expert);
    m->n_used = c.n_expert > 0 ? c.n_expert_used : 1;
    m->wt = c.w_dtype;
    m->at = c.act_dtype;
    m->kvt = c.kv_dtype;
    m->pieces = (c.w_dtype == PN_BF16 && c.act_dtype == PN_F32) ? 3 : 1;
    m->rows_max = c.max_batch * m->pieces;
    m->Nqkv = (m->H + 2 * m->Hk) * m->D;
    const int wt = m->wt, es_aux = (wt == PN_F32) ? 4 : 2;
    const bool i8 = wt == PN_I8;
    Bump bp;
    m->embd = bp.take((size_t)m->V * m->E * es_aux);
    m->out_norm = bp.take((size_t)m->E * 4);
    m->out = make_mat(m->V, m->E, wt);
    m->out.off = bp.take(m->out.bytes1);
    if (m->out.sbytes1) m->out.soff = bp.take(m->out.sbytes1);
    m->L.assign(c.n_layer, LayerOff{});
    for (int l = 0; l < c.n_layer; ++l) {
        LayerOff &L = m->L[l];
        L.attn_norm = bp.take((size_t)m->E * 4);
        L.ffn_norm = bp.take((size_t)m->E * 4);
        L.router = c.n_expert > 0 ? bp.take((size_t)c.n_expert * m->E * es_aux) : 0;
        L.bqkv = c.qkv_bias ? bp.take((size_t)m->Nqkv * 4) : 0;
        L.qkv = make_mat(m->Nqkv, m->E, wt);
        L.o = make_mat(m->E, m->H * m->D, wt);
        L.gate = make_mat(m->F, m->E, wt);
        L.up = make_mat(m->F, m->E, wt);
        L.down = make_mat(m->E, m->F, wt);
        for (Mat *mt : {&L.qkv, &L.o}) {
            mt->off = bp.take(mt->bytes1);
            if (mt->sbytes1) mt->soff = bp.take(mt->sbytes1);
        }
        for (Mat *mt : {&L.gate, &L.up, &L.down}) {
            mt->off = bp.take(mt->bytes1 * m->X);
            if (mt->sbytes1) mt->soff = bp.take(mt->sbytes1 * m->X);
        }
    }
    // scratch
    const int MB = c.max_batch, HD = m->H * m->D;
    m->a_es = wt == PN_F32 ? 4 : 2;
    const int tk = tile_k(wt);
    m->h_ld = cdiv(m->F, tk) * tk;
    m->h_plane = (long long)MB * m->n_used * m->h_ld;
    m->o_bytes = (size_t)MB * HD * 4;
    m->h_bytes = (size_t)m->pieces * m->h_plane * m->a_es;
    m->x = bp.take((size_t)MB * m->E * 4);
    m->q = bp.take((size_t)MB * HD * 4);
    m->o = bp.take(m->o_bytes);
    m->h = bp.take(m->h_bytes);
    m->y = bp.take((size_t)MB * m->n_used * m->E * 4);
    m->route_ids = bp.take((size_t)MB * m->n_used * 4);
    m->route_w = bp.take((size_t)MB * m->n_used * 4);
    m->rope = bp.take((size_t)MB * (m->D / 2) * 8);
    m->omega = bp.take((size_t)(m->D / 2) * 8);
    m->ssp_ld = cdiv(m->E, 16);
    m->ssp = bp.take((size_t)MB * m->ssp_ld * 4);
    m->am_count = (size_t)cdiv(m->out.n_tiles, 2) * MB;
    m->am_val = bp.take(m->am_count * 4);
    m->am_idx = bp.take(m->am_count * 4);
    m->samp_keys = bp.take((size_t)MB * m->V * 4);
    m->attn_part_row = (size_t)m->Hk * kMaxSplits * m->G * (m->D + 4) * 4;
    const int C = c.prefill_chunk;
    // (wide prefill runs its attention 16 rows at a time, each with its own split scratch)
    m->attn_part = bp.take((size_t)std::max(MB, C > 0 ? kMaxSlots : 0) * m->attn_part_row);
    if (C > 0) {
        m->wlda = cdiv(std::max(m->E, std::max(HD, m->F)), tile_k(wt)) * tile_k(wt);
        m->wa_plane = (long long)C * m->wlda;
        m->wx = bp.take((size_t)C * m->E * 4);
        m->wss = bp.take((size_t)C * kWideSsq * 4);
        m->wa = bp.take((size_t)m->pieces * m->wa_plane * 2);
        m->wq = bp.take((size_t)C * HD * 4);
        m->wo = bp.take((size_t)C * HD * 4);
        const long long qo = (long long)cdiv(std::max(m->Nqkv, m->E), 16) * 16;
        m->wy_cap = std::max((long long)kWideSplitMax * C * qo,
                             std::max(2LL * 2 * C * cdiv(m->F, 16) * 16, (long long)C * cdiv(m->V, 16) * 16));
        if (c.n_expert > 0) {
            const long long ne = (long long)C * m->n_used;  // packed rows
            // gate and up of every packed row in the two halves; the down outputs with 2 splits
            m->wy_cap = std::max(m->wy_cap, std::max(2LL * ne * cdiv(m->F, 16) * 16, 2LL * ne * cdiv(m->E, 16) * 16));
            m->wrid = bp.take((size_t)ne * 4);
            m->wrw = bp.take((size_t)ne * 4);
            m->wecnt = bp.take(64 * 4);
            m->weoff = bp.take(64 * 4);
            m->went = bp.take((size_t)ne * 4);
            m->wpos = bp.take((size_t)ne * 4);
            m->wap_plane = ne * m->wlda;
            m->wap = bp.take((size_t)m->pieces * m->wap_plane * 2);
            m->wyc = bp.take((size_t)C * m->E * 4);
        }
        m->wy = bp.take((size_t)m->wy_cap * 4);
    }
    m->kv_new = c.kv_dtype == PN_Q4_0 ? bp.take((size_t)MB * 2 * m->Hk * m->D * 4) : 0;
    m->samp_hist = bp.take((size_t)MB * kSampleBins * 4);
    m->samp_cnt = bp.take((size_t)MB * 2 * 4);
    m->samp_cand = bp.take((size_t)MB * kSampleCap * 8);
    // pn_profile_replay: a QKV replay appends its k, v rows here (page 0 of a
    // one-entry page table) instead of into a state's cache
    m->replay_kv = bp.take((size_t)2 * MB * m->Hk * kPage * kv_key_bytes(m));
    m->replay_pt = bp.take(256);
    return bp.off;
}

// Automatic split size: about one attention work-group per compute unit, or
// two when that still leaves every split 8 pages or more (a short split is
// scored right after its one round trip, so few long ones keep the tail
// short; many pages want both work-groups of a compute unit streaming).
long long attn_target_groups(long long pages) { return pages >= 8LL * 2 * kCUs ? 2 * kCUs : kCUs; }
// The attention addresses a layer's K and V pools with 32-bit buffer offsets.
constexpr size_t kMaxLayerBytes = (size_t)1 << 31;

size_t layout_state(pn_state *s) {
    const pn_model *m = s->m;
    s->n_pages = cdiv(s->max_ctx, kPage);
    s->layer_bytes = s->pool ? s->pool->layer_bytes : (size_t)s->n_pages * m->Hk * kPage * kv_key_bytes(m);
    int keys = s->max_ctx;
    if (m->cfg.sliding_window > 0) keys = std::min(keys, m->cfg.sliding_window);
    // splits start on page boundaries, so a window may touch one more chunk
    s->s_cap = std::min(cdiv(keys + kPage - 1, kAttnChunk), kMaxSplits);
    Bump bp;
    if (s->pool) {
        s->kpool = s->pool->kpool;
        s->vpool = s->pool->vpool;
    } else {
        s->kpool = bp.take(s->layer_bytes * m->cfg.n_layer);
        s->vpool = bp.take(s->layer_bytes * m->cfg.n_layer);
    }
    s->pt = bp.take((size_t)s->n_pages * 4);
    s->part = bp.take((size_t)m->Hk * s->s_cap * m->G * (m->D + 4) * 4);
    s->err = bp.take(4);
    return bp.off;
}

hipStream_t S(void *stream) { return reinterpret_cast<hipStream_t>(stream); }

// One layer's K (or V) pages of a state.
char *kv_layer(const pn_state *s, int layer, bool v) {
    char *b = s->pool ? s->pool->base : s->base;
    return b + (v ? s->vpool : s->kpool) + (size_t)layer * s->layer_bytes;
}

int launched(const char *what, const Plan *p = nullptr);

// Zero the pages of a set (all layers, K and V) and write their page-table
// entries; every page of the set comes from one pool.
void flush_pages(const pn_pool *pool, PageSet &ps, hipStream_t st) {
    if (ps.n > 0) {
        const pn_model *m = pool->m;
        const long long words = (long long)(pool->layer_bytes / pool->n_pages / 16);
        const dim3 grid((unsigned)std::min<long long>(cdiv(words, 256), 64), ps.n, 2 * m->cfg.n_layer);
        hipLaunchKernelGGL(k_zero_pages, grid, dim3(256), 0, st, pool->base + pool->kpool, pool->base + pool->vpool,
                           pool->layer_bytes, words, ps);
        hipLaunchKernelGGL(k_set_pages, dim3(1), dim3(kPageSetMax), 0, st, ps);
    }
    ps.n = 0;
}

// Pooled states: a page of the pool for every logical page of positions [p0[b],
// p1[b]) of each state that has none, all or nothing: on running out, the
// pages this call took go back (their page-table entries are never read: a
// logical page is read only after a call gave it a page).  New pages hold
// zeros, as a private cache does where nothing was written.
int ensure_pages(pn_state *const *st, int n, const int *p0, const int *p1, hipStream_t s) {
    PageSet ps{};
    const pn_pool *cur = nullptr;
    std::vector<std::pair<pn_state *, int>> taken;
    for (int b = 0; b < n; ++b) {
        pn_state *x = st[b];
        if (!x->pool || p1[b] <= p0[b]) continue;
        if (x->pool != cur) flush_pages(cur, ps, s);
        cur = x->pool;
        for (int lp = p0[b] / kPage; lp <= (p1[b] - 1) / kPage; ++lp) {
            if (x->phys[lp] >= 0) continue;
            if (x->pool->free_pages.empty()) {
                flush_pages(cur, ps, s);
                for (auto &t : taken) {
                    t.first->pool->free_pages.push_back(t.first->phys[t.second]);
                    t.first->phys[t.second] = -1;
                }
                return fail(PN_ERANGE, "page pool exhausted (%d pages)", x->pool->n_pages);
            }
            const int pg = x->pool->free_pages.back();
            x->pool->free_pages.pop_back();
            x->phys[lp] = pg;
            taken.push_back({x, lp});
            ps.pt[ps.n] = (int *)(x->base + x->pt);
            ps.idx[ps.n] = lp;
            ps.val[ps.n] = pg;
            if (++ps.n == kPageSetMax) flush_pages(cur, ps, s);
        }
    }
    flush_pages(cur, ps, s);
    return launched("page assignment", nullptr);
}

// First position the window of a step at pos reads (0 without a window).
int window_lo(const pn_model *m, int pos) {
    const int W = m->cfg.sliding_window;
    return W > 0 ? std::max(0, pos - W + 1) : 0;
}

// Pooled states with a window: return the pages wholly before the window of
// the state's next step.
void recycle_pages(pn_state *x) {
    if (!x->pool || x->m->cfg.sliding_window <= 0) return;
    const int lo = window_lo(x->m, x->pos);
    for (int lp = x->kept_from; lp < lo / kPage; ++lp)
        if (x->phys[lp] >= 0) {
            x->pool->free_pages.push_back(x->phys[lp]);
            x->phys[lp] = -1;
        }
    x->kept_from = std::max(x->kept_from, lo / kPage);
}

// Pooled states: every page back to the pool.
void give_back_all(pn_state *x) {
    if (!x->pool) return;
    for (int &pg : x->phys)
        if (pg >= 0) {
            x->pool->free_pages.push_back(pg);
            pg = -1;
        }
    x->kept_from = 0;
}

void fill32(void *p, size_t words, uint32_t v, hipStream_t s) {
    if (!words) return;
    int blocks = (int)std::min<size_t>(cdiv(words, 256), 4096);
    hipLaunchKernelGGL(k_fill32, dim3(blocks), dim3(256), 0, s, (uint32_t *)p, (long long)words, v);
}

void copy_bytes(void *dst, const void *src, size_t n, hipStream_t s) {
    if (!n) return;
    int blocks = (int)std::min<size_t>(cdiv(n, 256), 8192);
    hipLaunchKernelGGL(k_copy_bytes, dim3(blocks), dim3(256), 0, s, (uint8_t *)dst, (const uint8_t *)src,
                       (long long)n);
}

// Pack a row-major [N][K] matrix into tiles (Q8_0: also its block scales into
// the scale tiles at sdst_base); with neox_d > 0 the rows of each head block of
// neox_d rows are reordered into rotation pairs (see neox_src).
void pack(const void *src, int N, int K, int wt, const Mat &mt, int tile_row0, uint8_t *dst_base,
          uint8_t *sdst_base, hipStream_t s, int neox_d = 0) {
    const int nt = cdiv(N, 16);
    uint8_t *dst = dst_base + (size_t)tile_row0 * mt.KT * 1024;
    long long lanes = (long long)nt * mt.KT * 64;
    int blocks = cdiv(lanes, 256);
    const uint8_t *sp = (const uint8_t *)src;
    if (blockq(wt)) {
        uint8_t *sdst = sdst_base + (size_t)tile_row0 * mt.KT * 16 * 2 * tile_blocks(wt);
        if (wt == PN_Q8_0)
            hipLaunchKernelGGL(k_pack_q8, dim3(blocks), dim3(256), 0, s, sp, N, K, mt.KT, nt, dst, sdst, neox_d);
        else
            hipLaunchKernelGGL(k_pack_q4, dim3(blocks), dim3(256), 0, s, sp, N, K, mt.KT, nt, dst, sdst, neox_d);
    } else if (wt == PN_F32)
        hipLaunchKernelGGL(k_pack<4>, dim3(blocks), dim3(256), 0, s, sp, N, K, mt.KT, nt, dst, neox_d);
    else if (wt == PN_BF16)
        hipLaunchKernelGGL(k_pack<2>, dim3(blocks), dim3(256), 0, s, sp, N, K, mt.KT, nt, dst, neox_d);
    else
        hipLaunchKernelGGL(k_pack<1>, dim3(blocks), dim3(256), 0, s, sp, N, K, mt.KT, nt, dst, neox_d);
}

// dst[r] = src[neox_src(r, neox_d)] for n fp32 values (row scales, biases).
void copy_rows_f32(void *dst, const float *src, int n, int neox_d, hipStream_t s) {
    if (n <= 0) return;
    hipLaunchKernelGGL(k_copy_rows_f32, dim3(cdiv(n, 256)), dim3(256), 0, s, (float *)dst, src, n, neox_d);
}

// ---------------------------------------------------------------- launch dispatch

void gemm_entry(int kind, int wt, int at, int nw, int amode, const GemmArgs &g, dim3 grid, size_t lds,
                hipStream_t s, int *occ) {
    if (wt == PN_BF16 && at == PN_F32) launch_gemm_bf16_f32(kind, nw, amode, g, grid, lds, s, occ);
    else if (wt == PN_BF16) launch_gemm_bf16_bf16(kind, nw, amode, g, grid, lds, s, occ);
    else if (wt == PN_F32 && at == PN_F32) launch_gemm_f32_f32(kind, nw, amode, g, grid, lds, s, occ);
    else if (wt == PN_F32) launch_gemm_f32_bf16(kind, nw, amode, g, grid, lds, s, occ);
    else if (wt == PN_I8) launch_gemm_i8_bf16(kind, nw, amode, g, grid, lds, s, occ);
    else if (wt == PN_Q8_0) launch_gemm_q8_bf16(kind, nw, amode, g, grid, lds, s, occ);
    else launch_gemm_q4_bf16(kind, nw, amode, g, grid, lds, s, occ);
}

int pro_of(int kind) {
    if (kind == GK_RESID || kind == GK_MOE_DOWN) return PRO_LOAD;
    if (kind == GK_O_MERGE) return PRO_MERGE;
    return kind == GK_O ? PRO_CONV : PRO_NORM;
}

void launch_gemm(int kind, int wt, int at, GemmArgs g, const Plan &p, hipStream_t s) {
    const dim3 grid(p.gx, 1, p.gz);
    g.nblk = p.nblk;
    g.tpw = p.tpw;
    // the wave-local prologue where one batch of its registers holds a wave's
    // A slice (few slots); MoE kinds gather their rows on the device
    const bool moe = kind == GK_MOE_SWIGLU || kind == GK_MOE_DOWN;
    const int pieces = (wt == PN_BF16 && at == PN_F32) ? 3 : 1;
    const int pro = pro_of(kind);
    int amode = p.a_lds || pro != PRO_LOAD ? A_LDS : A_DIRECT;
    if (!moe && amode == A_LDS && gemm_wave_local_fits(wt, pro, p.nw, g.B, g.B * pieces, g.KT))
        amode = A_LDS_WAVE;
    else if (!moe && amode == A_LDS && p.nw == 16 && p.wave_rows && gemm_wave_rows_fits(wt, pro, p.nw, g.B, g.KT))
        amode = A_LDS_WAVE_ROWS;
    if (kind == GK_O_MERGE) amode = A_LDS_WAVE;  // (eligibility checked by merge_in_o)
    gemm_entry(kind, wt, at, p.nw, amode, g, grid, p.lds, s, nullptr);
}

void record_gemm(pn_model *m, int cls, int kind, const GemmArgs &g, const Plan &p) {
    pn_model::Replay r;
    r.kind = kind;
    r.g = g;
    r.p = p;
    if (kind == GK_QKV) {  // keep a replay away from the states' caches
        const size_t slot = (size_t)m->Hk * kPage * kv_key_bytes(m);
        for (int b = 0; b < g.B; ++b) {
            r.g.kvk[b] = m->base + m->replay_kv + (size_t)(2 * b) * slot;
            r.g.kvv[b] = m->base + m->replay_kv + (size_t)(2 * b + 1) * slot;
            r.g.pt[b] = (const int *)(m->base + m->replay_pt);
            r.g.pos[b] = g.pos[b] % kPage;
        }
    }
    m->last[cls].push_back(r);
}

// the launch just enqueued, checked at once so that a failure names its kernel
int launched(const char *what, const Plan *p) {
    const hipError_t e = hipGetLastError();
    if (e == hipSuccess) return PN_OK;
    if (p)
        return fail(PN_EHIP, "%s launch failed (grid %d x %d, %d waves, %zu B LDS): %s", what, p->gx, p->gz, p->nw,
                    p->lds, hipGetErrorString(e));
    return fail(PN_EHIP, "%s launch failed: %s", what, hipGetErrorString(e));
}

// event timing of one kernel class
struct Timed {
    pn_model *m;
    bool on;
    hipStream_t s;
    Timed(pn_model *mm, int k, hipStream_t ss) : m(mm), on(mm->prof_kernel == k), s(ss) {
        if (!on) return;
        if (m->ev_used + 2 > m->ev.size()) {
            for (int i = 0; i < 256; ++i) {
                hipEvent_t e;
                if (hipEventCreate(&e) != hipSuccess) { on = false; return; }
                m->ev.push_back(e);
            }
        }
        (void)hipEventRecord(m->ev[m->ev_used], s);
    }
    ~Timed() {
        if (!on) return;
        (void)hipEventRecord(m->ev[m->ev_used + 1], s);
        m->ev_used += 2;
    }
};

// One step over n rows.  Row b belongs to st[b] at its pos, or, for a
// prefill (row_pos given), every row to the one state st[0] at row_pos[b]:
// the rows then share the state's cache and page table, and their attention
// splits use the model's per-row scratch.
// Attention geometry of n rows (row b: state st[b] at position pos[b]).
// Splits: a row's window, from its start rounded down to a page, is np pages;
// split s of nsplit takes pages [s*np/nsplit, (s+1)*np/nsplit), so a row's
// splits differ by at most one page.  nsplit comes from the caller's keys per
// split (PN_OPT_ATTN_KEYS_PER_SPLIT), else from sharing about
// attn_target_groups work-groups among the rows in proportion to their pages;
// it is at most the row's pages and its scratch capacity.  With rows, the
// split scratch is the model's per-row buffer (prefill rows share a state);
// otherwise each state's own.  Sets everything but q, o and the K/V pools;
// returns the largest nsplit.
int attn_setup(const pn_model *m, pn_state *const *st, int n, const int *pos, bool rows, AttnArgs &aa,
               int ns_cap = 0) {
    aa.Hq = m->H;
    aa.Hk = m->Hk;
    aa.scale = (float)(1.4426950408889634 / std::sqrt((double)m->D));  // log2(e) / sqrt(D)
    long long np_sum = 0;
    for (int b = 0; b < n; ++b) np_sum += cdiv(pos[b] + 1 - window_lo(m, pos[b]) / kPage * kPage, kPage);
    int nsplit_max = 1;
    for (int b = 0; b < n; ++b) {
        const int lo = window_lo(m, pos[b]);
        aa.pos[b] = pos[b];
        aa.lo[b] = lo;
        aa.origin[b] = lo / kPage * kPage;
        const int np = cdiv(pos[b] + 1 - aa.origin[b], kPage);
        long long ns = m->attn_kps > 0 ? cdiv(np, m->attn_kps / kPage)
                       : ns_cap > 0    ? ns_cap
                                       : attn_target_groups(m->Hk * np_sum) * np / ((long long)m->Hk * np_sum);
        const int cap = rows ? kMaxSplits : st[b]->s_cap;
        ns = std::min<long long>(std::max<long long>(ns, 1), std::min(np, std::min(cap, kMaxSplits)));
        aa.np[b] = np;
        aa.nsplit[b] = (int)ns;
        aa.s_cap[b] = cap;
        nsplit_max = std::max(nsplit_max, aa.nsplit[b]);
        aa.pt[b] = (const int *)(st[b]->base + st[b]->pt);
        aa.part[b] = rows ? (float *)(m->base + m->attn_part + (size_t)b * m->attn_part_row)
                          : (float *)(st[b]->base + st[b]->part);
        aa.kv_bytes[b] = (unsigned)st[b]->layer_bytes;
        aa.pt_ident[b] = (!st[b]->pool && st[b]->pt_identity) ? 1 : 0;
    }
    return nsplit_max;
}

// Whether a decode step combines the attention splits in the O projection's
// prologue instead of a separate merge launch: one slot (not prefill rows), a
// bf16 cache scored on the matrix cores with G <= 4 query heads per KV head
// (8-wave attention work-groups, at most kMergeSplits splits), a window of at
// most kMergePages pages, and an O GEMM whose waves each cover at most 256 k
// (one 4-element piece per lane).  Measured on Llama-3-8B shapes: at 33 pages
// (2048 keys) the step is 0.8% faster this way; at 129 pages (8192 keys) 4.5%
// slower (eight splits of 16 pages take longer than 32 of 4 plus the merge).
constexpr int kMergePages = 48;
bool merge_in_o(const pn_model *m, int n, bool rows, int pos, const Plan &p_o, int KT_o) {
    if (n != 1 || rows || m->kvt != PN_BF16 || m->attn_kind == 1 || m->G > 4 || m->attn_combine == 1) return false;
    const int lo = window_lo(m, pos);
    if (cdiv(pos + 1 - lo / kPage * kPage, kPage) > kMergePages) return false;
    return cdiv(KT_o, p_o.nw) * tile_k(m->wt) <= 256;
}

int forward_impl(pn_model *m, pn_state *const *st, int n, const int32_t *tok, float *logits, int32_t *amax,
                 hipStream_t s, const int *row_pos = nullptr) {
    auto posof = [&](int b) { return row_pos ? row_pos[b] : st[b]->pos; };
    int pos_of_rows[kMaxSlots];
    for (int b = 0; b < n; ++b) pos_of_rows[b] = posof(b);
    const pn_config &c = m->cfg;
    char *mb = m->base;
    for (auto &r : m->last) r.clear();
    const int E = m->E, HD = m->H * m->D, F = m->F;
    const int wt = m->wt, at = m->at;
    const int rows = n * m->pieces;
    const int fb = frag_bytes(wt);
    const int kv_es = dtype_size(m->kvt);
    const bool moe = c.n_expert > 0;

    SlotPtrs sp{};
    GemmArgs base{};
    base.B = n;
    base.eps = c.rms_norm_eps;
    base.Hq = m->H;
    base.Hk = m->Hk;
    base.D = m->D;
    base.kv_es = kv_es;
    base.rope = (const float2 *)(mb + m->rope);
    base.ssp = (float *)(mb + m->ssp);
    base.ssp_ld = m->ssp_ld;
    base.ssp_n = m->ssp_ld;
    for (int b = 0; b < n; ++b) {
        sp.err[b] = (int *)(st[b]->base + st[b]->err);
        sp.pos[b] = posof(b);
        base.err[b] = sp.err[b];
        base.pos[b] = posof(b);
        base.pt[b] = (const int *)(st[b]->base + st[b]->pt);
    }

    float *x = (float *)(mb + m->x);
    {
        Timed tm(m, PN_K_EMBED, s);
        float2 *rope = (float2 *)(mb + m->rope);
        const double *omega = (const double *)(mb + m->omega);
        float *ssp = (float *)(mb + m->ssp);
        if (wt == PN_F32)
            hipLaunchKernelGGL(k_embed<0>, dim3(n), dim3(256), 0, s, (const void *)(mb + m->embd), tok, x, E, m->V, sp,
                               rope, omega, m->D, ssp, m->ssp_ld);
        else
            hipLaunchKernelGGL(k_embed<1>, dim3(n), dim3(256), 0, s, (const void *)(mb + m->embd), tok, x, E, m->V, sp,
                               rope, omega, m->D, ssp, m->ssp_ld);
    }

    // the residual trace: x as it enters layer l (and, at n_layer, as it leaves the last)
    auto trace_x = [&](int l) -> int {
        if (!m->trace || row_pos) return PN_OK;
        const hipError_t e = hipMemcpyAsync(m->trace + (size_t)l * c.max_batch * E, x, (size_t)n * E * 4,
                                            hipMemcpyDeviceToDevice, s);
        return e == hipSuccess ? PN_OK : fail(PN_EHIP, "residual trace copy: %s", hipGetErrorString(e));
    };
    if (int rc = trace_x(0)) return rc;

    const LayerOff &L0 = m->L[0];
    const int gz = moe ? m->X : 1;
    auto occ_of = [&](int kind, int nw, bool alds, size_t lds) -> int {
        const auto key = std::make_tuple(kind, nw, alds ? 1 : 0, lds);
        auto it = m->occ.find(key);
        if (it != m->occ.end()) return it->second;
        int n = 1;
        GemmArgs none{};
        gemm_entry(kind, wt, at, nw, alds ? A_LDS : A_DIRECT, none, dim3(1), lds, s, &n);
        m->occ[key] = n;
        return n;
    };
    const int cap = blockq(wt) ? 8 : 16;
    Plan p_qkv = make_plan(GK_QKV, L0.qkv.n_tiles, 1, L0.qkv.KT, rows, fb, m->nw[GK_QKV], occ_of, !m->nw_set, n,
                           cap);
    Plan p_o = make_plan(GK_O, L0.o.n_tiles, 1, L0.o.KT, rows, fb, m->nw[GK_O], occ_of, !m->nw_set, n, cap);
    Plan p_gu = make_plan(moe ? GK_MOE_SWIGLU : GK_SWIGLU, L0.gate.n_tiles, gz, L0.gate.KT, rows, fb,
                          m->nw[moe ? GK_MOE_SWIGLU : GK_SWIGLU], occ_of, !m->nw_set, n, cap);
    // dense down with bf16 weights: A fragments straight from memory at any
    // batch (Llama-3-8B shape at batch 1: 21.8 -> 19.9 us against A staged in
    // LDS; int8 weights' f16 fragments are slower that way: 13.2 -> 16.1 us)
    Plan p_dn = make_plan(moe ? GK_MOE_DOWN : GK_RESID, L0.down.n_tiles, gz, L0.down.KT, rows, fb,
                          moe ? m->nw[GK_MOE_DOWN] : m->nw_down, occ_of, !m->nw_set, 1, cap, !moe && wt == PN_BF16);
    Plan p_lm = make_plan(GK_LOGITS, cdiv(m->out.n_tiles, 2), 1, m->out.KT, rows, fb, m->nw[GK_LOGITS], occ_of,
                          !m->nw_set, n, cap);
    // (plans for the other kinds take one row block per tile)
    for (Plan *p : {&p_qkv, &p_o, &p_gu, &p_dn, &p_lm}) p->wave_rows = m->prologue == 0;

    // attention geometry per slot; with the split combine in the O prologue, at
    // most kMergeSplits splits per head (unless the caller's keys per split give more)
    bool mio = merge_in_o(m, n, row_pos != nullptr, pos_of_rows[0], p_o, L0.o.KT);
    AttnArgs aa{};
    const int nsplit_max = attn_setup(m, st, n, pos_of_rows, row_pos != nullptr, aa, mio ? kMergeSplits : 0);
    if (nsplit_max > kMergeSplits) mio = false;
    aa.q = (const float *)(mb + m->q);
    aa.o = (float *)(mb + m->o);
    // 8-wave attention work-groups (two pages per chunk) where the split
    // combine runs in the O prologue (few, long splits).  Elsewhere they
    // measured slower (8 slots: 30.8 -> 34.3 us per layer; Llama-3-8B INT8 at
    // 8192 keys: 2.147 -> 2.162 ms per step), so 4 unless the caller asks.
    aa.waves = mio ? 8 : (m->attn_waves && !row_pos ? m->attn_waves : kAttnWaves);

    for (int l = 0; l < c.n_layer; ++l) {
        const LayerOff &L = m->L[l];
        // ---- QKV + RoPE + KV append
        {
            GemmArgs g = base;
            g.w = (const uint8_t *)(mb + L.qkv.off);
            g.sc = (const float *)(mb + L.qkv.soff);
            g.N = L.qkv.N;
            g.n_tiles = L.qkv.n_tiles;
            g.KT = L.qkv.KT;
            g.K = E;
            g.x = x;
            g.gain = (const float *)(mb + L.attn_norm);
            g.q_out = (float *)(mb + m->q);
            g.bias = L.bqkv ? (const float *)(mb + L.bqkv) : nullptr;
            g.kv_new = m->kv_new ? (float *)(mb + m->kv_new) : nullptr;
            for (int b = 0; b < n; ++b) {
                g.kvk[b] = kv_layer(st[b], l, false);
                g.kvv[b] = kv_layer(st[b], l, true);
            }
            Timed tm(m, PN_K_QKV, s);
            launch_gemm(GK_QKV, wt, at, g, p_qkv, s);
            if (int rc = launched("QKV projection", &p_qkv)) return rc;
            record_gemm(m, PN_K_QKV, GK_QKV, g, p_qkv);
            if (m->kv_new) {  // Q4 cache: quantise the new rows into the pages
                KvQ4Args q{};
                q.src = g.kv_new;
                q.Hk = m->Hk;
                q.D = m->D;
                for (int b = 0; b < n; ++b) {
                    q.kvk[b] = g.kvk[b];
                    q.kvv[b] = g.kvv[b];
                    q.pt[b] = g.pt[b];
                    q.pos[b] = g.pos[b];
                }
                hipLaunchKernelGGL(k_kv_q4_append, dim3(n, m->Hk, 2), dim3(64), 0, s, q);
                if (int rc = launched("Q4 KV append")) return rc;
            }
        }
        // ---- attention (+ split combine)
        {
            for (int b = 0; b < n; ++b) {
                aa.kvk[b] = kv_layer(st[b], l, false);
                aa.kvv[b] = kv_layer(st[b], l, true);
            }
            aa.kind = m->attn_kind == 1 ? 0 : 1;
            Timed tm(m, PN_K_ATTN, s);
            launch_attn(m->D, m->kvt, m->G, aa, dim3(nsplit_max, m->Hk, n), nsplit_max > 1 && !mio, s);
            if (int rc = launched("attention")) return rc;
            pn_model::Replay r;
            r.aa = aa;
            r.grid = dim3(nsplit_max, m->Hk, n);
            r.merge = nsplit_max > 1 && !mio;
            m->last[PN_K_ATTN].push_back(r);
        }
        // ---- O projection + residual
        {
            GemmArgs g = base;
            g.w = (const uint8_t *)(mb + L.o.off);
            g.sc = (const float *)(mb + L.o.soff);
            g.N = E;
            g.n_tiles = L.o.n_tiles;
            g.KT = L.o.KT;
            g.K = HD;
            g.x = (const float *)(mb + m->o);
            g.out_f32 = x;
            g.ld_out = E;
            g.part = aa.part[0];
            g.nsplit = aa.nsplit[0];
            g.s_cap = aa.s_cap[0];
            const int ko = mio ? GK_O_MERGE : GK_O;
            Timed tm(m, PN_K_O, s);
            launch_gemm(ko, wt, at, g, p_o, s);
            if (int rc = launched("O projection", &p_o)) return rc;
            record_gemm(m, PN_K_O, ko, g, p_o);
        }
        // ---- FFN
        if (!moe) {
            {
                GemmArgs g = base;
                g.w = (const uint8_t *)(mb + L.gate.off);
                g.w2 = (const uint8_t *)(mb + L.up.off);
                g.sc = (const float *)(mb + L.gate.soff);
                g.sc2 = (const float *)(mb + L.up.soff);
                g.N = F;
                g.n_tiles = L.gate.n_tiles;
                g.KT = L.gate.KT;
                g.K = E;
                g.x = x;
                g.gain = (const float *)(mb + L.ffn_norm);
                g.out_act = mb + m->h;
                g.out_plane = m->h_plane;
                g.ld_out = m->h_ld;
                Timed tm(m, PN_K_GATEUP, s);
                launch_gemm(GK_SWIGLU, wt, at, g, p_gu, s);
                if (int rc = launched("gate/up projection", &p_gu)) return rc;
                record_gemm(m, PN_K_GATEUP, GK_SWIGLU, g, p_gu);
            }
            {
                GemmArgs g = base;
                g.w = (const uint8_t *)(mb + L.down.off);
                g.sc = (const float *)(mb + L.down.soff);
                g.N = E;
                g.n_tiles = L.down.n_tiles;
                g.KT = L.down.KT;
                g.K = F;
                g.a = mb + m->h;
                g.a_plane = m->h_plane;
                g.lda = m->h_ld;
                g.out_f32 = x;
                g.ld_out = E;
                Timed tm(m, PN_K_DOWN, s);
                launch_gemm(GK_RESID, wt, at, g, p_dn, s);
                if (int rc = launched("down projection", &p_dn)) return rc;
                record_gemm(m, PN_K_DOWN, GK_RESID, g, p_dn);
            }
        } else {
            int *rid = (int *)(mb + m->route_ids);
            float *rw = (float *)(mb + m->route_w);
            int *rlog = (m->route_log && !row_pos) ? m->route_log + ((m->route_log_step % m->route_log_steps) * c.n_layer + l) *
                                                           (long long)c.max_batch * m->n_used
                                     : nullptr;
            {
                Timed tm(m, PN_K_ROUTER, s);
                const size_t sh = (size_t)E * 4;
                const void *wr = mb + L.router;
                const float *gn = (const float *)(mb + L.ffn_norm);
                if (wt == PN_F32) {
                    if (at == PN_F32)
                        hipLaunchKernelGGL((k_router<0, AT_F32>), dim3(n), dim3(256), sh, s, (const float *)x, gn, wr, E, c.n_expert, m->n_used, c.rms_norm_eps, (const float *)(mb + m->ssp), m->ssp_ld, m->ssp_ld, rid, rw, rlog);
                    else
                        hipLaunchKernelGGL((k_router<0, AT_BF16>), dim3(n), dim3(256), sh, s, (const float *)x, gn, wr, E, c.n_expert, m->n_used, c.rms_norm_eps, (const float *)(mb + m->ssp), m->ssp_ld, m->ssp_ld, rid, rw, rlog);
                } else {
                    if (at == PN_F32)
                        hipLaunchKernelGGL((k_router<1, AT_F32>), dim3(n), dim3(256), sh, s, (const float *)x, gn, wr, E, c.n_expert, m->n_used, c.rms_norm_eps, (const float *)(mb + m->ssp), m->ssp_ld, m->ssp_ld, rid, rw, rlog);
                    else
                        hipLaunchKernelGGL((k_router<1, AT_BF16>), dim3(n), dim3(256), sh, s, (const float *)x, gn, wr, E, c.n_expert, m->n_used, c.rms_norm_eps, (const float *)(mb + m->ssp), m->ssp_ld, m->ssp_ld, rid, rw, rlog);
                }
            }
            {
                GemmArgs g = base;
                g.w = (const uint8_t *)(mb + L.gate.off);
                g.w2 = (const uint8_t *)(mb + L.up.off);
                g.sc = (const float *)(mb + L.gate.soff);
                g.sc2 = (const float *)(mb + L.up.soff);
                g.ew_stride = (long long)L.gate.bytes1;
                g.es_stride = (long long)(L.gate.sbytes1 / 4);
                g.N = F;
                g.n_tiles = L.gate.n_tiles;
                g.KT = L.gate.KT;
                g.K = E;
                g.x = x;
                g.gain = (const float *)(mb + L.ffn_norm);
                g.route_ids = rid;
                g.n_slots = n;
                g.n_used = m->n_used;
                g.out_act = mb + m->h;
                g.out_plane = m->h_plane;
                g.ld_out = m->h_ld;
                Timed tm(m, PN_K_MOE_GATEUP, s);
                launch_gemm(GK_MOE_SWIGLU, wt, at, g, p_gu, s);
                if (int rc = launched("expert gate/up projection", &p_gu)) return rc;
            }
            {
                GemmArgs g = base;
                g.w = (const uint8_t *)(mb + L.down.off);
                g.sc = (const float *)(mb + L.down.soff);
                g.ew_stride = (long long)L.down.bytes1;
                g.es_stride = (long long)(L.down.sbytes1 / 4);
                g.N = E;
                g.n_tiles = L.down.n_tiles;
                g.KT = L.down.KT;
                g.K = F;
                g.a = mb + m->h;
                g.a_plane = m->h_plane;
                g.lda = m->h_ld;
                g.route_ids = rid;
                g.n_slots = n;
                g.n_used = m->n_used;
                g.out_f32 = (float *)(mb + m->y);
                g.ld_out = E;
                Timed tm(m, PN_K_MOE_DOWN, s);
                launch_gemm(GK_MOE_DOWN, wt, at, g, p_dn, s);
                if (int rc = launched("expert down projection", &p_dn)) return rc;
            }
            {
                Timed tm(m, PN_K_MOE_COMBINE, s);
                hipLaunchKernelGGL(k_moe_combine, dim3(cdiv(E, 256), n), dim3(256), 0, s, x,
                                   (const float *)(mb + m->y), (const float *)rw, E, m->n_used,
                                   (float *)(mb + m->ssp), m->ssp_ld);
            }
        }
        if (int rc = trace_x(l + 1)) return rc;
    }
    // ---- final norm + LM head + argmax
    {
        GemmArgs g = base;
        g.w = (const uint8_t *)(mb + m->out.off);
        g.sc = (const float *)(mb + m->out.soff);
        g.N = m->V;
        g.n_tiles = m->out.n_tiles;
        g.KT = m->out.KT;
        g.K = E;
        g.x = x;
        g.gain = (const float *)(mb + m->out_norm);
        g.out_f32 = logits;
        g.am_val = (float *)(mb + m->am_val);
        g.am_idx = (int *)(mb + m->am_idx);
        Timed tm(m, PN_K_LMHEAD, s);
        launch_gemm(GK_LOGITS, wt, at, g, p_lm, s);
        if (int rc = launched("LM head", &p_lm)) return rc;
        record_gemm(m, PN_K_LMHEAD, GK_LOGITS, g, p_lm);
    }
    {
        Timed tm(m, PN_K_ARGMAX, s);
        hipLaunchKernelGGL(k_argmax, dim3(n), dim3(256), 0, s, (const float *)(mb + m->am_val),
                           (const int *)(mb + m->am_idx), p_lm.nblk, n, (int *)amax);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PN_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
    if (moe && m->route_log && !row_pos) ++m->route_log_step;
    if (row_pos) st[0]->pos += n;
    else for (int b = 0; b < n; ++b) st[b]->pos += 1;
    for (int b = 0; b < n; ++b) recycle_pages(st[b]);
    return PN_OK;
}

// ---- wide prefill: the rows of one chunk through each projection at once

// Attention splits per row on the wide path (the rows already give many work-groups).
constexpr int kWideAttnSplits = 8;
static_assert((long long)kWideRows * kWideAttnSplits <= (long long)kMaxSlots * kMaxSplits,
              "the rows' split scratch fits the per-row attention buffer");

// The weight-group width (8, 14 or 16 tiles) and the splits over K (1 to 8) of
// one wide GEMM, from a model of its time fitted to timings of the kernel
// (8B-model projections at 128 and 256 rows, every width and split count):
// the kernel runs one work-group per compute unit, so the grid runs in rounds
// of kCUs work-groups; a round takes its split's k steps times the measured
// time of one step (by weight type and width) plus about 1 us, and every MB
// of split outputs adds 0.35 us (written here, read back by the row kernel
// that follows); a 14-tile step takes 0.875 of a 16-tile one (its share of
// the matrix-core work; 14 tiles fill whole rounds where 16 leave compute
// units idle, e.g. 896 tiles: 256 work-groups against 224).  The least
// modelled time wins (ties: the narrower width, then fewer splits).  Every split keeps at least 8 k tiles, and the outputs
// fit the split buffer (cap floats).
struct WidePlan {
    int wgw, ks;
};
WidePlan wide_plan(int v, int R, int n_tiles, int KT, int nz, long long per, bool split_ok, long long cap) {
    // us per k step of a 16- and an 8-tile group: bf16 rows, fp32 rows as three
    // bf16 pieces, int8, Q8_0, Q4_0 (the variants of wide_variant; a Q4_0 step is
    // 128 wide)
    static const double step_us[5][2] = {{0.75, 0.43}, {1.185, 0.865}, {1.30, 0.73}, {1.74, 1.03}, {3.96, 2.04}};
    WidePlan best{8, 1};
    double best_t = -1.0;
    for (int w : {8, 14, 16}) {
        const double step = w == 8 ? step_us[v][1] : step_us[v][0] * (w == 14 ? 0.875 : 1.0);
        for (int ks = 1; ks <= (split_ok ? kWideSplitMax : 1); ++ks) {
            if (ks > 1 && (KT / ks < 8 || ks * per * nz > cap)) break;
            const long long groups = (long long)cdiv(R, 128) * cdiv(n_tiles, w) * nz * ks;
            const double rounds = (double)cdiv(groups, (long long)kCUs);
            const double t = rounds * (cdiv(KT, ks) * step + 1.0) + 0.35e-6 * 4.0 * ks * nz * per;
            if (best_t < 0.0 || t < best_t - 1e-9) {
                best_t = t;
                best = {w, ks};
            }
        }
    }
    return best;
}

// Y = A * W^T for R rows of the A planes: nz matrices (1, or 2 for gate and
// up) with outputs y[z] [split][R][ldy]; returns the number of splits used.
// The wide GEMM kernel of the model's weight and activation types: 0 = bf16
// weights with bf16 rows, 1 = bf16 weights with fp32 rows (three pieces), 2 =
// int8 weights, 3 = Q8_0 weights (both with f16 rows).
int wide_variant(const pn_model *m) {
    return m->wt == PN_Q4_0 ? 4 : (m->wt == PN_Q8_0 ? 3 : (m->wt == PN_I8 ? 2 : (m->pieces == 3 ? 1 : 0)));
}
// fn(WT, P, WGW) (as integral constants) for variant v with work-groups of wgw
// weight tiles (8, 14 or 16).
template <typename Fn>
auto with_wide(int v, int wgw, Fn fn) {
    auto go = [&](auto wt, auto p) {
        return wgw == 16   ? fn(wt, p, std::integral_constant<int, 16>{})
               : wgw == 14 ? fn(wt, p, std::integral_constant<int, 14>{})
                           : fn(wt, p, std::integral_constant<int, 8>{});
    };
    using I = std::integral_constant<int, 1>;
    switch (v) {
        case 4: return go(std::integral_constant<int, WT_Q4>{}, I{});
        case 3: return go(std::integral_constant<int, WT_Q8>{}, I{});
        case 2: return go(std::integral_constant<int, WT_I8>{}, I{});
        case 1: return go(std::integral_constant<int, WT_BF16>{}, std::integral_constant<int, 3>{});
        default: return go(std::integral_constant<int, WT_BF16>{}, I{});
    }
}
const void *wide_kernel(int v, int wgw) {
    return with_wide(v, wgw, [](auto wt, auto p, auto w) {
        return reinterpret_cast<const void *>(&k_wgemm<decltype(wt)::value, decltype(p)::value, decltype(w)::value>);
    });
}
int wide_lds(int v, int wgw) {
    return with_wide(v, wgw, [](auto wt, auto p, auto w) {
        return wgemm_lds(decltype(wt)::value, decltype(p)::value, decltype(w)::value);
    });
}

int wide_gemm(const pn_model *m, const Mat &mat, const uint8_t *w0, const uint8_t *w1, const float *s0,
              const float *s1, float *y0, float *y1, int nz, int R, int N, int ldy, bool split_ok, hipStream_t s) {
    const long long per = (long long)R * ldy;
    const WidePlan pl = wide_plan(wide_variant(m), R, mat.n_tiles, mat.KT, nz, per, split_ok, m->wy_cap);
    const int wgw = pl.wgw, ks = pl.ks;
    WGemmArgs g{};
    g.w[0] = w0;
    g.w[1] = w1 ? w1 : w0;
    g.sc[0] = s0;
    g.sc[1] = s1 ? s1 : s0;
    g.y[0] = y0;
    g.y[1] = y1 ? y1 : y0;
    g.y_split = per;
    g.a = (const uint16_t *)(m->base + m->wa);
    g.a_plane = m->wa_plane;
    g.lda = m->wlda;
    g.R = R;
    g.N = N;
    g.n_tiles = mat.n_tiles;
    g.KT = mat.KT;
    g.ldy = ldy;
    g.nsplit = ks;
    g.nzs = nz * ks;
    g.gx = cdiv(R, 128);
    const dim3 grid((unsigned)(g.gx * cdiv(mat.n_tiles, wgw) * g.nzs));
    const int v = wide_variant(m);
    const size_t lds = (size_t)wide_lds(v, wgw);  // (attribute set by wide_lds_attr)
    with_wide(v, wgw, [&](auto wt, auto p, auto w) {
        hipLaunchKernelGGL((k_wgemm<decltype(wt)::value, decltype(p)::value, decltype(w)::value>), grid, dim3(512),
                           lds, s, g);
        return 0;
    });
    return ks;
}

// The experts' products of one wide MoE FFN: Y = A * W_e^T for every expert
// e over its packed rows (counts and offsets on the device, from
// k_w_route_lists; at most R rows each), A the packed planes.  Planned as nz *
// X matrices of the packed rows' average count; returns the splits used.
int wide_gemm_experts(const pn_model *m, const Mat &mat, const uint8_t *w0, const uint8_t *w1, const float *s0,
                      const float *s1, float *y0, float *y1, int nz, int R, int N, int ldy, bool split_ok,
                      hipStream_t s) {
    const int X = m->X;
    const long long ne = (long long)R * m->n_used;
    const long long per = ne * ldy;  // floats of one split's outputs, per matrix
    const WidePlan pl = wide_plan(wide_variant(m), (int)cdiv(ne, (long long)X), mat.n_tiles, mat.KT, nz * X,
                                  cdiv(per, (long long)X), split_ok, m->wy_cap);
    const int wgw = pl.wgw, ks = pl.ks;
    char *mb = m->base;
    WGemmArgs g{};
    g.w[0] = w0;
    g.w[1] = w1 ? w1 : w0;
    g.sc[0] = s0;
    g.sc[1] = s1 ? s1 : s0;
    g.y[0] = y0;
    g.y[1] = y1 ? y1 : y0;
    g.y_split = per;
    g.a = (const uint16_t *)(mb + m->wap);
    g.a_plane = m->wap_plane;
    g.lda = m->wlda;
    g.R = R;
    g.N = N;
    g.n_tiles = mat.n_tiles;
    g.KT = mat.KT;
    g.ldy = ldy;
    g.nsplit = ks;
    g.nzs = nz * ks;
    g.gx = cdiv(R, 128);
    g.ecnt = (const int *)(mb + m->wecnt);
    g.eoff = (const int *)(mb + m->weoff);
    g.ew = (long long)mat.bytes1;
    g.es = (long long)mat.sbytes1;
    g.per_e = g.gx * cdiv(mat.n_tiles, wgw) * g.nzs;
    const dim3 grid((unsigned)((long long)g.per_e * X));
    const int v = wide_variant(m);
    const size_t lds = (size_t)wide_lds(v, wgw);
    with_wide(v, wgw, [&](auto wt, auto p, auto w) {
        hipLaunchKernelGGL((k_wgemm<decltype(wt)::value, decltype(p)::value, decltype(w)::value>), grid, dim3(512),
                           lds, s, g);
        return 0;
    });
    return ks;
}

// The wide GEMMs' LDS ring is dynamic and passes 64 KiB: raise the limit
// once per kernel.
int wide_lds_attr() {
    static bool done = false;
    if (done) return PN_OK;
    for (int v = 0; v < 5; ++v)
        for (int wgw : {8, 14, 16}) {
            const hipError_t e = hipFuncSetAttribute(wide_kernel(v, wgw), hipFuncAttributeMaxDynamicSharedMemorySize,
                                                     wide_lds(v, wgw));
            if (e != hipSuccess) return fail(PN_EHIP, "wide GEMM LDS attribute: %s", hipGetErrorString(e));
        }
    done = true;
    return PN_OK;
}

// One chunk of R rows of state st at positions st->pos .. st->pos + R - 1
// (pages already present).  Same result as R decode steps up to fp32
// summation order.
int prefill_wide(pn_model *m, pn_state *st, const int32_t *tok, int R, float *logits, int32_t *amax, hipStream_t s) {
    const pn_config &c = m->cfg;
    char *mb = m->base;
    const int E = m->E, HD = m->H * m->D, F = m->F, p0 = st->pos;
    float *x = (float *)(mb + m->wx), *y = (float *)(mb + m->wy);
    float *q = (float *)(mb + m->wq), *o = (float *)(mb + m->wo);
    uint16_t *a = (uint16_t *)(mb + m->wa);
    int *err = (int *)(st->base + st->err);
    const float eps = c.rms_norm_eps;
    const int var = wide_variant(m);
    const bool bq = var >= 2;  // f16 rows with per-row (int8) or per-block scales
    float *ssq = (float *)(mb + m->wss);
    // fn(WT, AT) as integral constants: the row kernels' A layout for this model
    auto rows_as = [&](auto fn) {
        using B = std::integral_constant<int, AT_BF16>;
        switch (var) {
            case 4: fn(std::integral_constant<int, WT_Q4>{}, B{}); break;
            case 3: fn(std::integral_constant<int, WT_Q8>{}, B{}); break;
            case 2: fn(std::integral_constant<int, WT_I8>{}, B{}); break;
            case 1: fn(std::integral_constant<int, WT_BF16>{}, std::integral_constant<int, AT_F32>{}); break;
            default: fn(std::integral_constant<int, WT_BF16>{}, B{}); break;
        }
    };
    // the row kernels write the columns a product over K reads (K rounded up to weight tiles)
    const int wtk = var == 4 ? WT_Q4 : (bq ? WT_I8 : WT_BF16);
    auto cols = [&](int K) { return (unsigned)cdiv(wide_kp(wtk, K), 1024); };
    auto norm = [&](const float *gain) {
        rows_as([&](auto wt, auto at) {
            hipLaunchKernelGGL((k_w_norm<decltype(wt)::value, decltype(at)::value>), dim3(cols(E), R), dim3(256), 0, s, x,
                               E, gain, eps, ssq, a, m->wa_plane, m->wlda);
        });
    };
    // x += the split outputs yy (ld columns, ks splits), then the next norm's A planes from the new x
    auto resid_norm_y = [&](const float *yy, int ld, int ks, const float *gain) {
        rows_as([&](auto wt, auto at) {
            hipLaunchKernelGGL((k_w_resid_norm<decltype(wt)::value, decltype(at)::value>), dim3(R), dim3(1024), 0, s, x, yy,
                               (long long)R * ld, ks, ld, E, gain, eps, a, m->wa_plane, m->wlda);
        });
    };
    auto resid_norm = [&](int ld, int ks, const float *gain) { resid_norm_y(y, ld, ks, gain); };
    const bool moe = c.n_expert > 0;
    const bool outputs = logits || amax;
    auto scales = [&](const Mat &mt) { return bq ? (const float *)(mb + mt.soff) : nullptr; };
    if (int rc = wide_lds_attr()) return rc;
    hipLaunchKernelGGL(k_w_embed, dim3(cdiv(E, 1024), R), dim3(256), 0, s, (const uint16_t *)(mb + m->embd), tok, x, E,
                       m->V, err, ssq);
    for (int l = 0; l < c.n_layer; ++l) {
        const LayerOff &L = m->L[l];
        char *kvk = kv_layer(st, l, false), *kvv = kv_layer(st, l, true);
        // ---- QKV, bias, RoPE, K/V append (later layers' attention norm ran with the residual before)
        if (l == 0) norm((const float *)(mb + L.attn_norm));
        {
            const int ld = L.qkv.n_tiles * 16;
            const int ks = wide_gemm(m, L.qkv, (const uint8_t *)(mb + L.qkv.off), nullptr, scales(L.qkv), nullptr, y, nullptr, 1, R, ld, ld,
                                     true, s);
            WQkvArgs w{};
            w.y = y;
            w.split = (long long)R * ld;
            w.nsplit = ks;
            w.ldy = ld;
            w.p0 = p0;
            w.Hq = m->H;
            w.Hk = m->Hk;
            w.D = m->D;
            w.kv_es = dtype_size(m->kvt);
            w.bias = L.bqkv ? (const float *)(mb + L.bqkv) : nullptr;
            w.omega = (const double *)(mb + m->omega);
            w.q = q;
            w.kvk = kvk;
            w.kvv = kvv;
            w.pt = (const int *)(st->base + st->pt);
            hipLaunchKernelGGL(k_w_qkv, dim3(cdiv(m->Nqkv / 2, 256), R), dim3(256), 0, s, w);
            if (int rc = launched("wide QKV")) return rc;
        }
        // ---- attention: one launch over the chunk's rows (each row sees keys up to its own position)
        {
            AttnArgs aa{};
            attn_setup(m, &st, 1, &p0, true, aa);  // scale, and slot 0's pages, table and scratch
            aa.q = q;
            aa.o = o;
            aa.kvk[0] = kvk;
            aa.kvv[0] = kvv;
            aa.rows = R;
            aa.p0 = p0;
            aa.window = c.sliding_window;
            aa.ns_rows = (int)std::max(1LL, std::min((long long)kWideAttnSplits, 1024LL / ((long long)R * m->Hk)));
            aa.s_cap[0] = kWideAttnSplits;
            aa.part_row = (long long)m->Hk * kWideAttnSplits * m->G * (m->D + 4);
            aa.kind = m->attn_kind == 1 ? 0 : 1;
            // a bf16 cache on the matrix cores takes 16 / G rows per work-group (sharing their K/V
            // loads, one split) when that still gives 64 work-groups; else a row each, with splits
            const int G = m->G, tr = 16 / std::max(G, 1);
            const bool tiled = m->kvt == PN_BF16 && aa.kind == 1 && tr > 1 &&
                               (G == 1 || G == 2 || G == 3 || G == 4 || G == 6 || G == 8) &&
                               (long long)cdiv(R, tr) * m->Hk >= 64;
            if (tiled) {
                aa.tile = tr;
                aa.ns_rows = 1;
                launch_attn(m->D, m->kvt, G, aa, dim3(1, m->Hk, cdiv(R, tr)), false, s);
            } else {
                launch_attn(m->D, m->kvt, G, aa, dim3(aa.ns_rows, m->Hk, R), aa.ns_rows > 1, s);
            }
            if (int rc = launched("wide attention")) return rc;
        }
        // ---- O + residual
        {
            rows_as([&](auto wt, auto at) {
                hipLaunchKernelGGL((k_w_conv<decltype(wt)::value, decltype(at)::value>), dim3(cols(HD), R), dim3(256), 0, s,
                                   o, HD, a, m->wa_plane, m->wlda);
            });
        }
        {
            const int ld = L.o.n_tiles * 16;
            const int ks = wide_gemm(m, L.o, (const uint8_t *)(mb + L.o.off), nullptr, scales(L.o), nullptr, y, nullptr, 1, R, ld, ld, true, s);
            if (!moe) {
                resid_norm(ld, ks, (const float *)(mb + L.ffn_norm));
            } else {
                // the residual with its block sums of squares (the router's norm reads them), the FFN norm
                hipLaunchKernelGGL(k_w_resid, dim3(cdiv(E, 1024), R), dim3(256), 0, s, x, y, (long long)R * ld, ks, ld, E,
                                   ssq);
                norm((const float *)(mb + L.ffn_norm));
            }
            if (int rc = launched("wide O")) return rc;
        }
        // the residual after the FFN (outputs yy: ld columns, ks splits), and the next norm
        auto finish_layer = [&](const float *yy, int ld, int ks) {
            if (l + 1 < c.n_layer)
                resid_norm_y(yy, ld, ks, (const float *)(mb + m->L[l + 1].attn_norm));
            else if (outputs)
                resid_norm_y(yy, ld, ks, (const float *)(mb + m->out_norm));
            else
                hipLaunchKernelGGL(k_w_resid, dim3(cdiv(E, 1024), R), dim3(256), 0, s, x, yy, (long long)R * ld, ks, ld, E,
                                   ssq);
        };
        if (moe) {
            // ---- experts: route every row, pack the entries by expert, gather their rows' A
            // planes, each expert's gate/up and down over its rows, the weighted sum per row
            const int nu = m->n_used, ne = R * nu;
            int *rid = (int *)(mb + m->wrid);
            float *rw = (float *)(mb + m->wrw);
            {
                const size_t sh = (size_t)E * 4;
                const void *wr = mb + L.router;
                const float *gn = (const float *)(mb + L.ffn_norm);
                const int nbk = cdiv(E, 1024);
                if (m->at == PN_F32)
                    hipLaunchKernelGGL((k_router<1, AT_F32>), dim3(R), dim3(256), sh, s, (const float *)x, gn, wr, E,
                                       c.n_expert, nu, eps, (const float *)ssq, kWideSsq, nbk, rid, rw, (int *)nullptr);
                else
                    hipLaunchKernelGGL((k_router<1, AT_BF16>), dim3(R), dim3(256), sh, s, (const float *)x, gn, wr, E,
                                       c.n_expert, nu, eps, (const float *)ssq, kWideSsq, nbk, rid, rw, (int *)nullptr);
                hipLaunchKernelGGL(k_w_route_lists, dim3(1), dim3(256), 0, s, (const int *)rid, ne, c.n_expert,
                                   (int *)(mb + m->wecnt), (int *)(mb + m->weoff), (int *)(mb + m->went),
                                   (int *)(mb + m->wpos));
                const int kp = wide_kp(wtk, E);
                hipLaunchKernelGGL(k_w_gather, dim3(cdiv(kp, 2048), ne, m->pieces), dim3(256), 0, s, (const uint16_t *)a,
                                   m->wa_plane, m->wlda, (const int *)(mb + m->went), nu, kp, (uint16_t *)(mb + m->wap),
                                   m->wap_plane);
                if (int rc = launched("wide routing")) return rc;
            }
            uint16_t *ap = (uint16_t *)(mb + m->wap);
            {
                const int ld = L.gate.n_tiles * 16;
                float *yu = y + m->wy_cap / 2;
                const int ks = wide_gemm_experts(m, L.gate, (const uint8_t *)(mb + L.gate.off),
                                                 (const uint8_t *)(mb + L.up.off), scales(L.gate), scales(L.up), y, yu, 2,
                                                 R, ld, ld, true, s);
                const long long sp = (long long)ne * ld;
                rows_as([&](auto wt, auto at) {  // (the gathered planes are free again: the down product's input)
                    hipLaunchKernelGGL((k_w_swiglu<decltype(wt)::value, decltype(at)::value>), dim3(cols(F), ne), dim3(256), 0,
                                       s, y, yu, sp, ks, ld, F, ap, m->wap_plane, m->wlda);
                });
                if (int rc = launched("wide expert gate/up")) return rc;
            }
            {
                const int ld = L.down.n_tiles * 16;
                const int ks = wide_gemm_experts(m, L.down, (const uint8_t *)(mb + L.down.off), nullptr, scales(L.down),
                                                 nullptr, y, nullptr, 1, R, E, ld, true, s);
                float *yc = (float *)(mb + m->wyc);
                hipLaunchKernelGGL(k_w_moe_combine, dim3(cdiv(E, 1024), R), dim3(256), 0, s, (const float *)y,
                                   (long long)ne * ld, ks, ld, (const int *)(mb + m->wpos), (const float *)rw, nu, E, yc);
                finish_layer(yc, E, 1);
                if (int rc = launched("wide expert down")) return rc;
            }
            continue;
        }
        // ---- gate/up, SwiGLU, down + residual (and the next norm)
        {
            const int ld = L.gate.n_tiles * 16;
            float *yu = y + m->wy_cap / 2;  // (2 matrices x at most 2 splits of R x ld fit each half)
            const bool fits = 2LL * 2 * R * ld <= m->wy_cap;
            const int ks = wide_gemm(m, L.gate, (const uint8_t *)(mb + L.gate.off), (const uint8_t *)(mb + L.up.off),
                                     scales(L.gate), scales(L.up), y, yu, 2, R, ld, ld, fits, s);
            const long long sp = (long long)R * ld;
            rows_as([&](auto wt, auto at) {
                hipLaunchKernelGGL((k_w_swiglu<decltype(wt)::value, decltype(at)::value>), dim3(cols(F), R), dim3(256), 0, s,
                                   y, yu, sp, ks, ld, F, a, m->wa_plane, m->wlda);
            });
            if (int rc = launched("wide gate/up")) return rc;
        }
        {
            const int ld = L.down.n_tiles * 16;
            const int ks = wide_gemm(m, L.down, (const uint8_t *)(mb + L.down.off), nullptr, scales(L.down), nullptr, y, nullptr, 1, R, ld, ld,
                                     true, s);
            finish_layer(y, ld, ks);
            if (int rc = launched("wide down")) return rc;
        }
    }
    // ---- LM head, argmax (only when an output is asked for; its norm ran with the last residual)
    if (outputs) {
        float *lg = logits ? logits : y;
        const int ld = logits ? m->V : m->out.n_tiles * 16;
        wide_gemm(m, m->out, (const uint8_t *)(mb + m->out.off), nullptr, scales(m->out), nullptr, lg, nullptr, 1, R, m->V, ld, false, s);
        if (amax) hipLaunchKernelGGL(k_w_argmax, dim3(R), dim3(256), 0, s, lg, (long long)ld, m->V, amax, err);
        if (int rc = launched("wide LM head")) return rc;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PN_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
    st->pos += R;
    recycle_pages(st);
    return PN_OK;
}

}  // namespace

// ==================================================================== C ABI

extern "C" {

void pn_config_default(pn_config *cfg) {
    if (!cfg) return;
    std::memset(cfg, 0, sizeof *cfg);
    cfg->n_ctx = 2048;
    cfg->rope_theta = 10000.0f;
    cfg->rms_norm_eps = 1e-5f;
    cfg->sliding_window = 0;
    cfg->max_batch = 1;
    cfg->w_dtype = PN_BF16;
    cfg->kv_dtype = PN_BF16;
    cfg->act_dtype = PN_F32;
}

int pn_config_check(const pn_config *cfg) {
    g_err.clear();
    return check_config(cfg);
}

size_t pn_model_bytes(const pn_config *cfg) {
    if (check_config(cfg) != PN_OK) return 0;
    pn_model m;
    m.cfg = normalized(*cfg);
    return layout_model(&m);
}

int pn_model_init(const pn_config *cfg, void *dev_buf, size_t bytes, pn_model **out) {
    g_err.clear();
    if (!out) return fail(PN_EINVAL, "out is NULL");
    *out = nullptr;
    int rc = check_config(cfg);
    if (rc) return rc;
    if (!dev_buf) return fail(PN_EINVAL, "device buffer is NULL");
    if (((uintptr_t)dev_buf & 255) != 0) return fail(PN_EINVAL, "device buffer must be 256-byte aligned");
    pn_model *m = new pn_model();
    m->cfg = normalized(*cfg);
    size_t need = layout_model(m);
    if (bytes < need) {
        delete m;
        return fail(PN_ERANGE, "model buffer too small: %zu < %zu", bytes, need);
    }
    m->base = (char *)dev_buf;
    m->bytes = bytes;
    *out = m;
    return PN_OK;
}

}  // extern "C"

namespace pn {

// The sampler's host side, shared by pn_sample (scratch in the model buffer)
// and pn_sample_noalloc (scratch in a file-scope device array).
// Host checks of the sampling parameters of n rows over a vocabulary of V, into a.
namespace {

int sample_args(int n, int V, const pn_sampling_params *params, const int32_t *recent_dev, int n_recent,
                const float *logits_dev, const float *u_dev, int32_t *ids_dev, SampleArgs &a) {
    if (n_recent < 0 || n_recent > kSampleMaxRecent)
        return fail(PN_EINVAL, "n_recent = %d outside [0, %d]", n_recent, kSampleMaxRecent);
    if (n_recent > 0 && !recent_dev) return fail(PN_EINVAL, "recent_dev is NULL");
    a.logits = logits_dev;
    a.V = V;
    a.n_recent = n_recent;
    a.recent = recent_dev;
    a.u = u_dev;
    a.ids = ids_dev;
    for (int b = 0; b < n; ++b) {
        const pn_sampling_params &p = params[b];
        if (std::isnan(p.temperature)) return fail(PN_EINVAL, "row %d: temperature is NaN", b);
        if (p.temperature > 0.f) {
            if (!std::isfinite(p.temperature)) return fail(PN_EINVAL, "row %d: temperature must be finite", b);
            if (p.top_k < 1 || p.top_k > kSampleMaxK)
                return fail(PN_EUNSUPPORTED, "row %d: top_k = %d outside [1, %d]", b, p.top_k, kSampleMaxK);
            if (!(p.repeat_penalty > 0.f) || !std::isfinite(p.repeat_penalty))
                return fail(PN_EINVAL, "row %d: repeat_penalty must be finite and > 0", b);
            if (std::isnan(p.top_p)) return fail(PN_EINVAL, "row %d: top_p is NaN", b);
        }
        a.temp[b] = p.temperature;
        a.rp[b] = p.repeat_penalty;
        a.top_p[b] = p.top_p;
        a.top_k[b] = p.top_k;
    }
    return PN_OK;
}

// The sampler's three kernels over n rows.  The histogram and the gather
// counters (rows_cap rows of them) start each call at zero: the previous call's
// k_sample_pick cleared them, unless that call stopped early (`dirty`), and
// then a fill kernel clears them first (a kernel, not a memset, so that the
// call may be captured in a graph).
int sample_run(const SampleArgs &a, int n, int rows_cap, bool &dirty, hipStream_t st) {
    if (dirty) {
        fill32(a.hist, (size_t)rows_cap * kSampleBins, 0u, st);
        fill32(a.cnt, (size_t)rows_cap * 2, 0u, st);
        if (int rc = launched("sampling scratch clear")) return rc;
        dirty = false;
    }
    // the candidate buffer is dynamic LDS; with the kernel's static LDS the
    // total passes 64 KiB, which needs the attribute (the two within 160 KiB)
    static bool lds_set = false;
    const size_t lds = (size_t)kSampleCap * 8;
    if (!lds_set) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_sample_pick),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return fail(PN_EHIP, "sampling LDS attribute: %s", hipGetErrorString(e));
        lds_set = true;
    }
    dirty = true;
    hipLaunchKernelGGL(k_sample_keys, dim3(kSampleBlocks, n), dim3(256), 0, st, a);
    if (int rc = launched("sampling keys")) return rc;
    hipLaunchKernelGGL(k_sample_gather, dim3(kSampleBlocks, n), dim3(256), 0, st, a);
    if (int rc = launched("sampling gather")) return rc;
    hipLaunchKernelGGL(k_sample_pick, dim3(n), dim3(kSamplePick), lds, st, a);
    if (int rc = launched("sampling pick")) return rc;
    dirty = false;
    return PN_OK;
}

}  // namespace

int host_sample(const float *logits_dev, int n, int V, const pn_sampling_params *params, const int32_t *recent_dev,
                int n_recent, const float *u_dev, int32_t *ids_dev, const SampleScratchPtrs &sp, int rows_cap,
                bool &dirty, hipStream_t st) {
    SampleArgs a{};
    if (int rc = sample_args(n, V, params, recent_dev, n_recent, logits_dev, u_dev, ids_dev, a)) return rc;
    a.keys = sp.keys;
    a.hist = sp.hist;
    a.cnt = sp.cnt;
    a.cand = sp.cand;
    return sample_run(a, n, rows_cap, dirty, st);
}

int host_fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

void host_clear_error() { g_err.clear(); }

}  // namespace pn

namespace {

// the pointer checks of the load calls, shared with pn_model_create, which
// runs them over every layer before it enqueues anything
int check_globals(const pn_config *cfg, const void *tok_embd, const float *out_norm, const void *w_out,
                  const float *s_out) {
    const bool i8 = cfg->w_dtype == PN_I8;
    if (!tok_embd || !out_norm || !w_out || (i8 && !s_out)) return fail(PN_EINVAL, "missing global weight pointer");
    return PN_OK;
}

int check_layer(const pn_config *cfg, int32_t layer, const pn_layer_weights *W) {
    if (!W) return fail(PN_EINVAL, "NULL argument");
    if (layer < 0 || layer >= cfg->n_layer) return fail(PN_EINVAL, "layer %d out of range", layer);
    const bool i8 = cfg->w_dtype == PN_I8;
    if (!W->attn_norm || !W->ffn_norm || !W->wq || !W->wk || !W->wv || !W->wo || !W->w_gate || !W->w_up || !W->w_down)
        return fail(PN_EINVAL, "missing weight pointer in layer %d", layer);
    if (cfg->n_expert > 0 && !W->w_router) return fail(PN_EINVAL, "missing router in layer %d", layer);
    if (i8 && (!W->s_q || !W->s_k || !W->s_v || !W->s_o || !W->s_gate || !W->s_up || !W->s_down))
        return fail(PN_EINVAL, "missing int8 scales in layer %d", layer);
    if (cfg->qkv_bias && (!W->b_q || !W->b_k || !W->b_v)) return fail(PN_EINVAL, "missing q/k/v bias in layer %d", layer);
    return PN_OK;
}

}  // namespace

extern "C" {

int pn_model_load_globals(pn_model *m, const void *tok_embd, const float *out_norm, const void *w_out,
                          const float *s_out, void *stream) {
    g_err.clear();
    if (!m) return fail(PN_EINVAL, "model is NULL");
    const bool i8 = m->wt == PN_I8;
    if (int rc = check_globals(&m->cfg, tok_embd, out_norm, w_out, s_out)) return rc;
    hipStream_t s = S(stream);
    char *mb = m->base;
    const int es_aux = m->wt == PN_F32 ? 4 : 2;
    copy_bytes(mb + m->embd, tok_embd, (size_t)m->V * m->E * es_aux, s);
    copy_bytes(mb + m->out_norm, out_norm, (size_t)m->E * 4, s);
    pack(w_out, m->V, m->E, m->wt, m->out, 0, (uint8_t *)(mb + m->out.off), (uint8_t *)(mb + m->out.soff), s);
    if (i8) {
        fill32(mb + m->out.soff, (size_t)m->out.n_tiles * 16, 0u, s);
        copy_bytes(mb + m->out.soff, s_out, (size_t)m->V * 4, s);
    }
    hipLaunchKernelGGL(k_omega, dim3(1), dim3(64), 0, s, (double *)(mb + m->omega), m->D, (double)m->cfg.rope_theta);
    fill32(mb + m->o, m->o_bytes / 4, 0u, s);
    fill32(mb + m->h, m->h_bytes / 4, 0u, s);
    fill32(mb + m->replay_pt, 64, 0u, s);
    fill32(mb + m->samp_hist, (size_t)m->cfg.max_batch * kSampleBins, 0u, s);
    fill32(mb + m->samp_cnt, (size_t)m->cfg.max_batch * 2, 0u, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PN_EHIP, "weight packing failed: %s", hipGetErrorString(e));
    return PN_OK;
}

int pn_model_load_layer(pn_model *m, int32_t layer, const pn_layer_weights *W, void *stream) {
    g_err.clear();
    if (!m || !W) return fail(PN_EINVAL, "NULL argument");
    const pn_config *cfg = &m->cfg;
    if (int rc = check_layer(cfg, layer, W)) return rc;
    const bool i8 = m->wt == PN_I8;
    hipStream_t s = S(stream);
    char *mb = m->base;
    const int wt = m->wt, es_aux = wt == PN_F32 ? 4 : 2;
    const int E = m->E, HD = m->H * m->D, F = m->F, X = m->X;
    const LayerOff &L = m->L[layer];
    copy_bytes(mb + L.attn_norm, W->attn_norm, (size_t)E * 4, s);
    copy_bytes(mb + L.ffn_norm, W->ffn_norm, (size_t)E * 4, s);
    if (cfg->n_expert > 0) copy_bytes(mb + L.router, W->w_router, (size_t)cfg->n_expert * E * es_aux, s);
    // q, k and v blocks are tile aligned because head_dim is a multiple of 16
    uint8_t *qkv = (uint8_t *)(mb + L.qkv.off);
    // NeoX RoPE: q and k rows are packed in rotation-pair order, so the
    // epilogue's adjacent-pair rotation is the half-split one
    const int nx = cfg->rope_neox ? m->D : 0;
    uint8_t *qkv_s = (uint8_t *)(mb + L.qkv.soff);
    pack(W->wq, m->H * m->D, E, wt, L.qkv, 0, qkv, qkv_s, s, nx);
    pack(W->wk, m->Hk * m->D, E, wt, L.qkv, m->H * m->D / 16, qkv, qkv_s, s, nx);
    pack(W->wv, m->Hk * m->D, E, wt, L.qkv, (m->H + m->Hk) * m->D / 16, qkv, qkv_s, s);
    if (cfg->qkv_bias) {
        char *bq = mb + L.bqkv;
        copy_rows_f32(bq, W->b_q, m->H * m->D, nx, s);
        copy_rows_f32(bq + (size_t)m->H * m->D * 4, W->b_k, m->Hk * m->D, nx, s);
        copy_rows_f32(bq + (size_t)(m->H + m->Hk) * m->D * 4, W->b_v, m->Hk * m->D, 0, s);
    }
    pack(W->wo, E, HD, wt, L.o, 0, (uint8_t *)(mb + L.o.off), (uint8_t *)(mb + L.o.soff), s);
    if (i8) {
        char *sq = mb + L.qkv.soff;
        fill32(sq, (size_t)L.qkv.n_tiles * 16, 0u, s);
        copy_rows_f32(sq, W->s_q, m->H * m->D, nx, s);
        copy_rows_f32(sq + (size_t)m->H * m->D * 4, W->s_k, m->Hk * m->D, nx, s);
        copy_bytes(sq + (size_t)(m->H + m->Hk) * m->D * 4, W->s_v, (size_t)m->Hk * m->D * 4, s);
        fill32(mb + L.o.soff, (size_t)L.o.n_tiles * 16, 0u, s);
        copy_bytes(mb + L.o.soff, W->s_o, (size_t)E * 4, s);
    }
    for (int e = 0; e < X; ++e) {
        const char *g = (const char *)W->w_gate + (size_t)e * F * src_row_bytes(wt, E);
        const char *u = (const char *)W->w_up + (size_t)e * F * src_row_bytes(wt, E);
        const char *d = (const char *)W->w_down + (size_t)e * E * src_row_bytes(wt, F);
        pack(g, F, E, wt, L.gate, 0, (uint8_t *)(mb + L.gate.off + e * L.gate.bytes1),
             (uint8_t *)(mb + L.gate.soff + e * L.gate.sbytes1), s);
        pack(u, F, E, wt, L.up, 0, (uint8_t *)(mb + L.up.off + e * L.up.bytes1),
             (uint8_t *)(mb + L.up.soff + e * L.up.sbytes1), s);
        pack(d, E, F, wt, L.down, 0, (uint8_t *)(mb + L.down.off + e * L.down.bytes1),
             (uint8_t *)(mb + L.down.soff + e * L.down.sbytes1), s);
        if (i8) {
            const size_t gs = (size_t)L.gate.n_tiles * 16 * 4, ds = (size_t)L.down.n_tiles * 16 * 4;
            fill32(mb + L.gate.soff + e * gs, gs / 4, 0u, s);
            fill32(mb + L.up.soff + e * gs, gs / 4, 0u, s);
            fill32(mb + L.down.soff + e * ds, ds / 4, 0u, s);
            copy_bytes(mb + L.gate.soff + e * gs, W->s_gate + (size_t)e * F, (size_t)F * 4, s);
            copy_bytes(mb + L.up.soff + e * gs, W->s_up + (size_t)e * F, (size_t)F * 4, s);
            copy_bytes(mb + L.down.soff + e * ds, W->s_down + (size_t)e * E, (size_t)E * 4, s);
        }
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PN_EHIP, "weight packing failed: %s", hipGetErrorString(e));
    return PN_OK;
}

int pn_model_create(const pn_config *cfg, const pn_weights *w, void *dev_buf, size_t bytes, void *stream,
                    pn_model **out) {
    g_err.clear();
    if (!out) return fail(PN_EINVAL, "out is NULL");
    *out = nullptr;
    int rc = check_config(cfg);
    if (rc) return rc;
    if (!w || !w->layers) return fail(PN_EINVAL, "weights are NULL");
    // every pointer of every layer is checked before anything is enqueued
    const pn_config n = normalized(*cfg);
    if ((rc = check_globals(&n, w->tok_embd, w->out_norm, w->w_out, w->s_out))) return rc;
    for (int l = 0; l < n.n_layer; ++l)
        if ((rc = check_layer(&n, l, &w->layers[l]))) return rc;
    pn_model *m = nullptr;
    rc = pn_model_init(cfg, dev_buf, bytes, &m);
    if (rc) return rc;
    rc = pn_model_load_globals(m, w->tok_embd, w->out_norm, w->w_out, w->s_out, stream);
    for (int l = 0; rc == PN_OK && l < cfg->n_layer; ++l) rc = pn_model_load_layer(m, l, &w->layers[l], stream);
    if (rc) {
        std::string msg = g_err;
        delete m;
        g_err = msg;
        return rc;
    }
    *out = m;
    return PN_OK;
}

void pn_model_free(pn_model *m) {
    if (!m) return;
    for (hipEvent_t e : m->ev) (void)hipEventDestroy(e);
    delete m;
}

size_t pn_state_bytes(const pn_model *m, int32_t max_ctx) {
    if (!m) return 0;
    if (max_ctx == 0) max_ctx = m->cfg.n_ctx;
    if (max_ctx < 1) return 0;
    pn_state s{};
    s.m = const_cast<pn_model *>(m);
    s.max_ctx = max_ctx;
    const size_t need = layout_state(&s);
    return s.layer_bytes < kMaxLayerBytes ? need : 0;
}

int pn_state_reset(pn_state *s, void *stream) {
    g_err.clear();
    if (!s) return fail(PN_EINVAL, "state is NULL");
    hipStream_t st = S(stream);
    if (s->pool) {
        give_back_all(s);  // new pages are zeroed when taken
    } else {
        fill32(s->base + s->kpool, s->layer_bytes * s->m->cfg.n_layer / 4, 0u, st);
        fill32(s->base + s->vpool, s->layer_bytes * s->m->cfg.n_layer / 4, 0u, st);
    }
    fill32(s->base + s->err, 1, 0u, st);
    s->pos = 0;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PN_EHIP, "reset failed: %s", hipGetErrorString(e));
    return PN_OK;
}

int pn_state_new(pn_model *m, int32_t max_ctx, void *dev_buf, size_t bytes, void *stream, pn_state **out) {
    g_err.clear();
    if (!out) return fail(PN_EINVAL, "out is NULL");
    *out = nullptr;
    if (!m || !dev_buf) return fail(PN_EINVAL, "model or device buffer is NULL");
    if (((uintptr_t)dev_buf & 255) != 0) return fail(PN_EINVAL, "device buffer must be 256-byte aligned");
    if (max_ctx == 0) max_ctx = m->cfg.n_ctx;
    if (max_ctx < 1) return fail(PN_EINVAL, "max_ctx must be >= 1");
    pn_state *s = new pn_state{};
    s->m = m;
    s->max_ctx = max_ctx;
    size_t need = layout_state(s);
    if (s->layer_bytes >= kMaxLayerBytes) {
        delete s;
        return fail(PN_ERANGE, "max_ctx %d too large: one layer's K pool would reach 2 GiB", max_ctx);
    }
    if (bytes < need) {
        delete s;
        return fail(PN_ERANGE, "state buffer too small: %zu < %zu", bytes, need);
    }
    s->base = (char *)dev_buf;
    s->bytes = bytes;
    hipLaunchKernelGGL(k_iota, dim3(cdiv(s->n_pages, 256)), dim3(256), 0, S(stream), (int *)(s->base + s->pt),
                       s->n_pages);
    int rc = pn_state_reset(s, stream);
    if (rc) {
        delete s;
        return rc;
    }
    *out = s;
    return PN_OK;
}

// Bytes of one page (all positions and KV heads of one layer's K or V pool).
size_t pool_page_bytes(const pn_model *m) { return (size_t)m->Hk * kPage * kv_key_bytes(m); }

size_t pn_pool_bytes(const pn_model *m, int32_t n_pages) {
    if (!m || n_pages < 1) return 0;
    const size_t layer = pool_page_bytes(m) * n_pages;
    if (layer >= kMaxLayerBytes) return 0;
    return 2 * layer * m->cfg.n_layer;
}

int pn_pool_new(pn_model *m, int32_t n_pages, void *dev_buf, size_t bytes, pn_pool **out) {
    g_err.clear();
    if (!out) return fail(PN_EINVAL, "out is NULL");
    *out = nullptr;
    if (!m || !dev_buf) return fail(PN_EINVAL, "model or device buffer is NULL");
    if (((uintptr_t)dev_buf & 255) != 0) return fail(PN_EINVAL, "device buffer must be 256-byte aligned");
    if (n_pages < 1) return fail(PN_EINVAL, "n_pages must be >= 1");
    const size_t need = pn_pool_bytes(m, n_pages);
    if (need == 0) return fail(PN_ERANGE, "%d pages: one layer's K pool would reach 2 GiB", n_pages);
    if (bytes < need) return fail(PN_ERANGE, "pool buffer too small: %zu < %zu", bytes, need);
    pn_pool *p = new pn_pool{};
    p->m = m;
    p->base = (char *)dev_buf;
    p->bytes = bytes;
    p->n_pages = n_pages;
    p->layer_bytes = pool_page_bytes(m) * n_pages;
    p->kpool = 0;
    p->vpool = p->layer_bytes * m->cfg.n_layer;
    p->free_pages.resize(n_pages);
    for (int i = 0; i < n_pages; ++i) p->free_pages[i] = n_pages - 1 - i;  // page 0 is taken first
    *out = p;
    return PN_OK;
}

void pn_pool_free(pn_pool *p) {
    if (!p) return;
    p->closed = true;
    if (p->users == 0) delete p;
}

int32_t pn_pool_free_pages(const pn_pool *p) { return p ? (int32_t)p->free_pages.size() : -1; }

size_t pn_state_bytes_pooled(const pn_model *m, int32_t max_ctx) {
    if (!m) return 0;
    if (max_ctx == 0) max_ctx = m->cfg.n_ctx;
    if (max_ctx < 1) return 0;
    pn_pool dummy{};
    pn_state s{};
    s.m = const_cast<pn_model *>(m);
    s.max_ctx = max_ctx;
    s.pool = &dummy;
    return layout_state(&s);
}

int pn_state_new_pooled(pn_model *m, pn_pool *pool, int32_t max_ctx, void *dev_buf, size_t bytes, void *stream,
                        pn_state **out) {
    g_err.clear();
    if (!out) return fail(PN_EINVAL, "out is NULL");
    *out = nullptr;
    if (!m || !pool || !dev_buf) return fail(PN_EINVAL, "model, pool or device buffer is NULL");
    if (pool->m != m) return fail(PN_EINVAL, "pool belongs to another model");
    if (pool->closed) return fail(PN_EINVAL, "pool was freed");
    if (((uintptr_t)dev_buf & 255) != 0) return fail(PN_EINVAL, "device buffer must be 256-byte aligned");
    if (max_ctx == 0) max_ctx = m->cfg.n_ctx;
    if (max_ctx < 1) return fail(PN_EINVAL, "max_ctx must be >= 1");
    pn_state *s = new pn_state{};
    s->m = m;
    s->max_ctx = max_ctx;
    s->pool = pool;
    const size_t need = layout_state(s);
    if (bytes < need) {
        delete s;
        return fail(PN_ERANGE, "state buffer too small: %zu < %zu", bytes, need);
    }
    s->base = (char *)dev_buf;
    s->bytes = bytes;
    s->phys.assign(s->n_pages, -1);
    // entries without a page are never read; 0 keeps every entry inside the pool
    fill32(s->base + s->pt, s->n_pages, 0u, S(stream));
    pool->users += 1;
    int rc = pn_state_reset(s, stream);
    if (rc) {
        pn_state_free(s);
        return rc;
    }
    *out = s;
    return PN_OK;
}

int pn_state_set_kv(pn_state *s, int32_t layer, int32_t pos0, int32_t n, const void *k, const void *v,
                    void *stream) {
    g_err.clear();
    if (!s || !k || !v) return fail(PN_EINVAL, "NULL argument");
    const pn_model *m = s->m;
    if (layer < 0 || layer >= m->cfg.n_layer) return fail(PN_EINVAL, "layer %d out of range", layer);
    if (n < 0 || pos0 < 0 || (long long)pos0 + n > s->max_ctx) return fail(PN_ERANGE, "positions out of range");
    if (n == 0) return PN_OK;
    if (s->pool) {
        if (pos0 < s->kept_from * kPage)
            return fail(PN_ERANGE, "positions below %d went back to the page pool", s->kept_from * kPage);
        const int p1 = pos0 + n;
        if (int rc = ensure_pages(&s, 1, &pos0, &p1, S(stream))) return rc;
    }
    char *kp = kv_layer(s, layer, false);
    char *vp = kv_layer(s, layer, true);
    long long total = (long long)n * m->Hk * m->D;
    dim3 grid(cdiv(total, 256));
    const int nx = m->cfg.rope_neox ? m->D : 0;  // k is cached in rotation-pair order
    if (m->kvt == PN_Q4_0)
        hipLaunchKernelGGL(k_kv_q4_set, dim3(n, m->Hk, 2), dim3(64), 0, S(stream), kp, vp, (const int *)(s->base + s->pt),
                           (const float *)k, (const float *)v, pos0, m->Hk, m->D);
    else if (m->kvt == PN_BF16)
        hipLaunchKernelGGL(k_set_kv<2>, grid, dim3(256), 0, S(stream), kp, vp, (const int *)(s->base + s->pt),
                           (const char *)k, (const char *)v, pos0, n, m->Hk, m->D, nx);
    else
        hipLaunchKernelGGL(k_set_kv<4>, grid, dim3(256), 0, S(stream), kp, vp, (const int *)(s->base + s->pt),
                           (const char *)k, (const char *)v, pos0, n, m->Hk, m->D, nx);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PN_EHIP, "set_kv failed: %s", hipGetErrorString(e));
    return PN_OK;
}

int pn_state_set_page_table(pn_state *s, const int32_t *pages, int32_t n, void *stream) {
    g_err.clear();
    if (!s || !pages) return fail(PN_EINVAL, "NULL argument");
    if (s->pool) return fail(PN_EUNSUPPORTED, "a pooled state's pages come from its pool");
    if (n != s->n_pages) return fail(PN_EINVAL, "page table must have %d entries", s->n_pages);
    std::vector<char> seen(n, 0);
    for (int i = 0; i < n; ++i) {
        if (pages[i] < 0 || pages[i] >= n || seen[pages[i]]) return fail(PN_EINVAL, "page table is not a permutation");
        seen[pages[i]] = 1;
    }
    hipError_t e = hipMemcpyAsync(s->base + s->pt, pages, (size_t)n * 4, hipMemcpyHostToDevice, S(stream));
    if (e == hipSuccess) e = hipStreamSynchronize(S(stream));
    if (e != hipSuccess) return fail(PN_EHIP, "page table copy failed: %s", hipGetErrorString(e));
    bool ident = true;
    for (int i = 0; i < n && ident; ++i) ident = pages[i] == i;
    s->pt_identity = ident;  // attention computes page ids for an identity table instead of loading them
    return PN_OK;
}

int32_t pn_state_pages(const pn_state *s) { return s ? s->n_pages : 0; }
int32_t pn_page_size(void) { return kPage; }

int pn_state_set_pos(pn_state *s, int32_t pos, void *stream) {
    g_err.clear();
    if (!s) return fail(PN_EINVAL, "state is NULL");
    if (pos < 0 || pos > s->max_ctx) return fail(PN_ERANGE, "pos %d out of range", pos);
    if (s->pool) {
        // the next step reads the window [lo, pos]: its pages below pos must exist
        const int lo = window_lo(s->m, pos);
        if (lo / kPage < s->kept_from)
            return fail(PN_ERANGE, "pos %d reads positions below %d, which went back to the page pool", pos,
                        s->kept_from * kPage);
        if (int rc = ensure_pages(&s, 1, &lo, &pos, S(stream))) return rc;
    }
    s->pos = pos;
    return PN_OK;
}

int32_t pn_state_pos(const pn_state *s) { return s ? s->pos : -1; }
int32_t pn_state_max_ctx(const pn_state *s) { return s ? s->max_ctx : 0; }

int pn_state_check(pn_state *s, void *stream, int32_t *flags_out) {
    g_err.clear();
    if (!s || !flags_out) return fail(PN_EINVAL, "NULL argument");
    int32_t f = 0;
    hipError_t e = hipMemcpyAsync(&f, s->base + s->err, 4, hipMemcpyDeviceToHost, S(stream));
    if (e == hipSuccess) e = hipStreamSynchronize(S(stream));
    if (e != hipSuccess) return fail(PN_EHIP, "flag read failed: %s", hipGetErrorString(e));
    fill32(s->base + s->err, 1, 0u, S(stream));
    *flags_out = f;
    return PN_OK;
}

void pn_state_free(pn_state *s) {
    if (!s) return;
    for (auto &r : s->m->last) r.clear();  // recorded launches may point into this state
    if (pn_pool *p = s->pool) {
        give_back_all(s);
        if (--p->users == 0 && p->closed) delete p;
    }
    delete s;
}

int pn_forward_batch(pn_model *m, pn_state *const *states, int32_t n, const int32_t *tokens_dev,
                     float *logits_dev, int32_t *argmax_dev, void *stream) {
    g_err.clear();
    if (!m || !states || !tokens_dev) return fail(PN_EINVAL, "NULL argument");
    if (n < 1 || n > m->cfg.max_batch) return fail(PN_EINVAL, "n = %d outside [1, max_batch = %d]", n, m->cfg.max_batch);
    for (int i = 0; i < n; ++i) {
        if (!states[i]) return fail(PN_EINVAL, "state %d is NULL", i);
        if (states[i]->m != m) return fail(PN_EINVAL, "state %d belongs to another model", i);
        if (states[i]->pos < 0 || states[i]->pos >= states[i]->max_ctx)
            return fail(PN_ERANGE, "state %d: pos %d leaves no room (max_ctx %d)", i, states[i]->pos, states[i]->max_ctx);
        for (int j = 0; j < i; ++j)
            if (states[j] == states[i]) return fail(PN_EINVAL, "state %d appears twice", i);
    }
    int p0[kMaxSlots], p1[kMaxSlots];
    for (int i = 0; i < n; ++i) {
        p0[i] = states[i]->pos;
        p1[i] = states[i]->pos + 1;
    }
    if (int rc = ensure_pages(states, n, p0, p1, S(stream))) return rc;
    return forward_impl(m, states, n, tokens_dev, logits_dev, argmax_dev, S(stream));
}

int pn_prefill(pn_model *m, pn_state *s, const int32_t *tokens_dev, int32_t n, float *logits_dev,
               int32_t *argmax_dev, void *stream) {
    g_err.clear();
    if (!m || !s || !tokens_dev) return fail(PN_EINVAL, "NULL argument");
    if (s->m != m) return fail(PN_EINVAL, "state belongs to another model");
    if (n < 1) return fail(PN_EINVAL, "n = %d must be >= 1", n);
    if (s->pos < 0 || (long long)s->pos + n > s->max_ctx)
        return fail(PN_ERANGE, "positions %d..%lld exceed max_ctx %d", s->pos, (long long)s->pos + n - 1, s->max_ctx);
    if (m->cfg.prefill_chunk > 0) {  // the wide path
        for (int t0 = 0; t0 < n; t0 += m->cfg.prefill_chunk) {
            const int c = std::min(m->cfg.prefill_chunk, n - t0);
            const int p1 = s->pos + c;
            if (int rc = ensure_pages(&s, 1, &s->pos, &p1, S(stream))) return rc;
            if (int rc = prefill_wide(m, s, tokens_dev + t0, c, logits_dev ? logits_dev + (size_t)t0 * m->V : nullptr,
                                      argmax_dev ? argmax_dev + t0 : nullptr, S(stream)))
                return rc;
        }
        return PN_OK;
    }
    // chunks of max_batch tokens, each one batched step over consecutive positions
    const int chunk = m->cfg.max_batch;
    std::vector<pn_state *> rows(chunk, s);
    int rp[kMaxSlots];
    for (int t0 = 0; t0 < n; t0 += chunk) {
        const int c = std::min(chunk, n - t0);
        const int p1 = s->pos + c;
        if (int rc = ensure_pages(&s, 1, &s->pos, &p1, S(stream))) return rc;
        for (int b = 0; b < c; ++b) rp[b] = s->pos + b;
        if (int rc = forward_impl(m, rows.data(), c, tokens_dev + t0, logits_dev ? logits_dev + (size_t)t0 * m->V : nullptr,
                                  argmax_dev ? argmax_dev + t0 : nullptr, S(stream), rp))
            return rc;
    }
    return PN_OK;
}

int pn_sample(pn_model *m, const float *logits_dev, int32_t n, const pn_sampling_params *params,
              const int32_t *recent_dev, int32_t n_recent, const float *u_dev, int32_t *ids_dev, void *stream) {
    g_err.clear();
    if (!m || !logits_dev || !params || !u_dev || !ids_dev) return fail(PN_EINVAL, "NULL argument");
    if (n < 1 || n > m->cfg.max_batch) return fail(PN_EINVAL, "n = %d outside [1, max_batch = %d]", n, m->cfg.max_batch);
    SampleScratchPtrs sp{(unsigned *)(m->base + m->samp_keys), (unsigned *)(m->base + m->samp_hist),
                         (unsigned *)(m->base + m->samp_cnt), (unsigned long long *)(m->base + m->samp_cand)};
    return host_sample(logits_dev, n, m->V, params, recent_dev, n_recent, u_dev, ids_dev, sp, m->cfg.max_batch,
                       m->samp_dirty, S(stream));
}

int pn_forward_step(pn_model *m, pn_state *s, const int32_t *token_dev, float *logits_dev, int32_t *argmax_dev,
                    void *stream) {
    pn_state *one[1] = {s};
    return pn_forward_batch(m, one, 1, token_dev, logits_dev, argmax_dev, stream);
}

int pn_model_set_option(pn_model *m, int32_t option, int64_t value) {
    g_err.clear();
    if (!m) return fail(PN_EINVAL, "model is NULL");
    if (option >= PN_OPT_WAVES_QKV && option <= PN_OPT_WAVES_LMHEAD) {
        if (value != 4 && value != 8 && value != 16) return fail(PN_EINVAL, "waves must be 4, 8 or 16");
        switch (option) {
            case PN_OPT_WAVES_QKV: m->nw[GK_QKV] = (int)value; break;
            case PN_OPT_WAVES_O: m->nw[GK_O] = (int)value; break;
            case PN_OPT_WAVES_GATEUP: m->nw[GK_SWIGLU] = (int)value; m->nw[GK_MOE_SWIGLU] = (int)value; break;
            case PN_OPT_WAVES_DOWN: m->nw_down = (int)value; m->nw[GK_MOE_DOWN] = (int)value; break;
            default: m->nw[GK_LOGITS] = (int)value; break;
        }
        m->nw_set = true;
        return PN_OK;
    }
    if (option == PN_OPT_ATTN_KERNEL) {
        if (value < 0 || value > 2) return fail(PN_EINVAL, "attention kernel must be 0, 1 or 2");
        m->attn_kind = (int)value;
        return PN_OK;
    }
    if (option == PN_OPT_ATTN_WAVES) {
        if (value != 0 && value != 4 && value != 8) return fail(PN_EINVAL, "attention waves must be 0, 4 or 8");
        m->attn_waves = (int)value;
        return PN_OK;
    }
    if (option == PN_OPT_GEMM_PROLOGUE) {
        if (value < 0 || value > 1) return fail(PN_EINVAL, "GEMM prologue must be 0 or 1");
        m->prologue = (int)value;
        return PN_OK;
    }
    if (option == PN_OPT_ATTN_COMBINE) {
        if (value < 0 || value > 1) return fail(PN_EINVAL, "split combine must be 0 or 1");
        m->attn_combine = (int)value;
        return PN_OK;
    }
    if (option == PN_OPT_ATTN_KEYS_PER_SPLIT) {
        if (value < 0 || value % kAttnChunk != 0 || value > (1 << 24))
            return fail(PN_EINVAL, "keys per split must be 0 or a multiple of %d", kAttnChunk);
        m->attn_kps = (int)value;
        return PN_OK;
    }
    return fail(PN_EINVAL, "unknown option %d", option);
}

int pn_profile_begin(pn_model *m, int32_t kernel) {
    g_err.clear();
    if (!m) return fail(PN_EINVAL, "model is NULL");
    if (kernel < 0 || kernel >= PN_K_COUNT) return fail(PN_EINVAL, "unknown kernel class %d", kernel);
    m->prof_kernel = kernel;
    m->ev_used = 0;
    return PN_OK;
}

int pn_profile_replay(pn_model *m, int32_t kernel, int32_t reps, void *stream) {
    g_err.clear();
    if (!m) return fail(PN_EINVAL, "model is NULL");
    if (kernel < 0 || kernel >= PN_K_COUNT) return fail(PN_EINVAL, "unknown kernel class %d", kernel);
    if (reps < 1) return fail(PN_EINVAL, "reps must be positive");
    const std::vector<pn_model::Replay> &rs = m->last[kernel];
    if (rs.empty() || (kernel != PN_K_ATTN && rs[0].kind < 0))
        return fail(PN_EINVAL, "no recorded launch of kernel class %d", kernel);
    hipStream_t s = S(stream);
    for (int i = 0; i < reps; ++i) {
        const pn_model::Replay &r = rs[i % rs.size()];
        if (kernel == PN_K_ATTN) launch_attn(m->D, m->kvt, m->G, r.aa, r.grid, r.merge, s);
        else launch_gemm(r.kind, m->wt, m->at, r.g, r.p, s);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PN_EHIP, "replay launch failed: %s", hipGetErrorString(e));
    return PN_OK;
}

int pn_profile_end(pn_model *m, void *stream, double *total_ms, int64_t *launches) {
    g_err.clear();
    if (!m || !total_ms || !launches) return fail(PN_EINVAL, "NULL argument");
    m->prof_kernel = -1;
    hipError_t e = hipStreamSynchronize(S(stream));
    if (e != hipSuccess) return fail(PN_EHIP, "synchronize failed: %s", hipGetErrorString(e));
    double tot = 0.0;
    for (size_t i = 0; i + 1 < m->ev_used; i += 2) {
        float ms = 0.f;
        e = hipEventElapsedTime(&ms, m->ev[i], m->ev[i + 1]);
        if (e != hipSuccess) return fail(PN_EHIP, "event timing failed: %s", hipGetErrorString(e));
        tot += ms;
    }
    *total_ms = tot;
    *launches = (int64_t)(m->ev_used / 2);
    m->ev_used = 0;
    return PN_OK;
}

int pn_model_route_log(pn_model *m, int32_t *log_dev, int32_t n_steps) {
    g_err.clear();
    if (!m) return fail(PN_EINVAL, "model is NULL");
    if (m->cfg.n_expert == 0) return fail(PN_EINVAL, "a dense model has no routing to record");
    if (log_dev && n_steps < 1) return fail(PN_EINVAL, "n_steps must be >= 1");
    m->route_log = log_dev;
    m->route_log_steps = log_dev ? n_steps : 0;
    m->route_log_step = 0;
    return PN_OK;
}

int pn_model_trace(pn_model *m, float *trace_dev) {
    g_err.clear();
    if (!m) return fail(PN_EINVAL, "model is NULL");
    m->trace = trace_dev;
    return PN_OK;
}

int pn_stream_read(const void *src_dev, size_t bytes, uint32_t *sink_dev, void *stream) {
    g_err.clear();
    if (!src_dev || !sink_dev) return fail(PN_EINVAL, "NULL argument");
    if (bytes == 0 || bytes % 16 != 0) return fail(PN_EINVAL, "bytes must be a positive multiple of 16");
    if (((uintptr_t)src_dev & 15) != 0) return fail(PN_EINVAL, "src_dev must be 16-byte aligned");
    // eight work-groups of 256 threads per compute unit, eight loads in flight per thread
    const long long n16 = (long long)(bytes / 16);
    const int groups = (int)std::min<long long>(kCUs * 8, cdiv(n16, 256LL * 8));
    hipLaunchKernelGGL(k_stream_read, dim3(groups), dim3(256), 0, S(stream), (const u32x4 *)src_dev, n16,
                       (unsigned *)sink_dev);
    return launched("stream read");
}

const char *pn_last_error(void) { return g_err.c_str(); }

}  // extern "C"
