// pn_launch.hpp - launch entry points of the kernel translation units.
#pragma once
#include <hip/hip_runtime.h>

#include "pn_attn.hpp"

namespace pn {

// The GEMM variants of one decode step.
enum GemmKind {
    GK_QKV = 0,        // norm prologue, RoPE + KV-append epilogue
    GK_RESID = 1,      // A-ready input, residual epilogue (O, down)
    GK_SWIGLU = 2,     // norm prologue, gate/up pair, SwiGLU epilogue
    GK_LOGITS = 3,     // norm prologue, two tiles per block, logits + argmax partials
    GK_MOE_SWIGLU = 4, // gathered rows, per-expert gate/up pair
    GK_MOE_DOWN = 5,   // gathered A-ready rows, per-expert down
    GK_O = 6,          // fp32 rows rounded to the activation type, residual epilogue
    GK_O_MERGE = 7,    // GK_O for one slot whose attention splits are combined in the prologue
    GK_COUNT = 8
};

// Dynamic LDS a launch may use, in bytes: a work-group's 160 KiB less 1 KiB
// for the kernels' static LDS (the two together may not exceed the limit).
constexpr size_t kMaxLds = 159 * 1024;

// Defined once per (weight type, activation type) in pn_gemm.hip; nw = waves
// per work-group (4, 8 or 16); amode: A_DIRECT reads an A-ready input straight
// from memory, A_LDS stages A in LDS, A_LDS_WAVE stages it per wave (the
// wave-local prologue; not for MoE kinds), A_LDS_WAVE_ROWS per wave over
// several slots (the conversion prologue, up to kWaveRowsMax slots).
// With occ non-null nothing is launched: *occ receives the resident
// work-groups per CU.
enum AMode { A_DIRECT = 0, A_LDS = 1, A_LDS_WAVE = 2, A_LDS_WAVE_ROWS = 3 };
void launch_gemm_f32_f32(int kind, int nw, int amode, const GemmArgs &g, dim3 grid, size_t lds, hipStream_t s,
                         int *occ);
void launch_gemm_f32_bf16(int kind, int nw, int amode, const GemmArgs &g, dim3 grid, size_t lds, hipStream_t s,
                         int *occ);
void launch_gemm_bf16_f32(int kind, int nw, int amode, const GemmArgs &g, dim3 grid, size_t lds, hipStream_t s,
                         int *occ);
void launch_gemm_bf16_bf16(int kind, int nw, int amode, const GemmArgs &g, dim3 grid, size_t lds, hipStream_t s,
                         int *occ);
void launch_gemm_i8_bf16(int kind, int nw, int amode, const GemmArgs &g, dim3 grid, size_t lds, hipStream_t s,
                         int *occ);
void launch_gemm_q8_bf16(int kind, int nw, int amode, const GemmArgs &g, dim3 grid, size_t lds, hipStream_t s,
                         int *occ);
void launch_gemm_q4_bf16(int kind, int nw, int amode, const GemmArgs &g, dim3 grid, size_t lds, hipStream_t s,
                         int *occ);

// Defined once per (head_dim, KV type) in pn_attn.hip: attention with G query
// heads per KV head, and the split combine when `combine`.
#define PN_ATTN_DECL(name) \
    void name(int G, const AttnArgs &a, dim3 grid, bool merge, hipStream_t s);
PN_ATTN_DECL(launch_attn_32_0)
PN_ATTN_DECL(launch_attn_32_1)
PN_ATTN_DECL(launch_attn_64_0)
PN_ATTN_DECL(launch_attn_64_1)
PN_ATTN_DECL(launch_attn_128_0)
PN_ATTN_DECL(launch_attn_128_1)
PN_ATTN_DECL(launch_attn_32_2)
PN_ATTN_DECL(launch_attn_64_2)
PN_ATTN_DECL(launch_attn_128_2)
#undef PN_ATTN_DECL

// kvt: the pn_dtype of the cache (PN_F32 0, PN_BF16 1, PN_Q4_0 4 -> instantiation 2)
inline void launch_attn(int D, int kvt, int G, const AttnArgs &a, dim3 grid, bool merge, hipStream_t s) {
    if (kvt == 4) {
        if (D == 32) launch_attn_32_2(G, a, grid, merge, s);
        else if (D == 64) launch_attn_64_2(G, a, grid, merge, s);
        else launch_attn_128_2(G, a, grid, merge, s);
    } else if (kvt == 1) {
        if (D == 32) launch_attn_32_1(G, a, grid, merge, s);
        else if (D == 64) launch_attn_64_1(G, a, grid, merge, s);
        else launch_attn_128_1(G, a, grid, merge, s);
    } else {
        if (D == 32) launch_attn_32_0(G, a, grid, merge, s);
        else if (D == 64) launch_attn_64_0(G, a, grid, merge, s);
        else launch_attn_128_0(G, a, grid, merge, s);
    }
}

}  // namespace pn
