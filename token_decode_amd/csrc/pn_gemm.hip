// pn_gemm.hip - the GEMM kernels of one (weight type, activation type) pair.
// Compiled once per pair with -DPN_WT=<0|1|2> -DPN_AT=<0|1> -DPN_NAME=<entry>.
#include "pn_launch.hpp"

namespace pn {
namespace {

// Dynamic LDS above 64 KiB has to be enabled per kernel; done once for each
// kernel (one flag per instantiation: the kernels all share one signature).
template <auto *KERNEL>
void allow_lds(size_t lds) {
    static bool done = false;
    if (lds > 64 * 1024 && !done) {
        (void)hipFuncSetAttribute(reinterpret_cast<const void *>(KERNEL),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds);
        done = true;
    }
}

// occ >= 0: report resident work-groups per CU in *occ instead of launching
template <int PRO, int EPI, int NTW, bool PAIR, int NW, bool ALDS, int WL>
void go_k(const GemmArgs &g, dim3 grid, size_t lds, hipStream_t s, int *occ) {
    auto *k = &k_gemm<PN_WT, PN_AT, PRO, EPI, NTW, PAIR, NW, ALDS, WL>;
    allow_lds<&k_gemm<PN_WT, PN_AT, PRO, EPI, NTW, PAIR, NW, ALDS, WL>>(lds);
    if (occ) {
        int n = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k, NW * 64, lds) != hipSuccess) n = 1;
        *occ = n;
        return;
    }
    hipLaunchKernelGGL(k, grid, dim3(NW * 64), lds, s, g);
}

template <int PRO, int EPI, int NTW, bool PAIR, int NW>
void go_nw(int amode, const GemmArgs &g, dim3 grid, size_t lds, hipStream_t s, int *occ) {
    constexpr bool MOE = EPI == EPI_MOE_SWIGLU || EPI == EPI_MOE_DOWN;
    if constexpr (PRO == PRO_MERGE) {  // (wave-local only)
        go_k<PRO, EPI, NTW, PAIR, NW, true, 1>(g, grid, lds, s, occ);
    } else {
        if constexpr (!MOE) {
            if (amode == A_LDS_WAVE) {
                go_k<PRO, EPI, NTW, PAIR, NW, true, 1>(g, grid, lds, s, occ);
                return;
            }
        }
        // several slots per wave: the conversion prologue of 16-wave groups
        if constexpr (PRO == PRO_CONV && NW == 16) {
            if (amode == A_LDS_WAVE_ROWS) {
                go_k<PRO, EPI, NTW, PAIR, NW, true, 2>(g, grid, lds, s, occ);
                return;
            }
        }
        if constexpr (PRO != PRO_LOAD) {
            go_k<PRO, EPI, NTW, PAIR, NW, true, 0>(g, grid, lds, s, occ);
        } else {
            if (amode != A_DIRECT) go_k<PRO, EPI, NTW, PAIR, NW, true, 0>(g, grid, lds, s, occ);
            else go_k<PRO, EPI, NTW, PAIR, NW, false, 0>(g, grid, lds, s, occ);
        }
    }
}

template <int PRO, int EPI, int NTW, bool PAIR>
void go(int nw, int amode, const GemmArgs &g, dim3 grid, size_t lds, hipStream_t s, int *occ) {
    if (nw == 4) go_nw<PRO, EPI, NTW, PAIR, 4>(amode, g, grid, lds, s, occ);
    else if (nw == 8) go_nw<PRO, EPI, NTW, PAIR, 8>(amode, g, grid, lds, s, occ);
    else go_nw<PRO, EPI, NTW, PAIR, 16>(amode, g, grid, lds, s, occ);
}

}  // namespace

void PN_NAME(int kind, int nw, int amode, const GemmArgs &g, dim3 grid, size_t lds, hipStream_t s, int *occ) {
    switch (kind) {
        case GK_QKV: go<PRO_NORM, EPI_QKV, 1, false>(nw, amode, g, grid, lds, s, occ); break;
        case GK_RESID: go<PRO_LOAD, EPI_RESID, 1, false>(nw, amode, g, grid, lds, s, occ); break;
        case GK_SWIGLU: go<PRO_NORM, EPI_SWIGLU, 2, true>(nw, amode, g, grid, lds, s, occ); break;
        case GK_LOGITS: go<PRO_NORM, EPI_LOGITS, 2, false>(nw, amode, g, grid, lds, s, occ); break;
        case GK_MOE_SWIGLU: go<PRO_NORM, EPI_MOE_SWIGLU, 2, true>(nw, amode, g, grid, lds, s, occ); break;
        case GK_MOE_DOWN: go<PRO_LOAD, EPI_MOE_DOWN, 1, false>(nw, amode, g, grid, lds, s, occ); break;
        case GK_O: go<PRO_CONV, EPI_RESID, 1, false>(nw, amode, g, grid, lds, s, occ); break;
        case GK_O_MERGE: go<PRO_MERGE, EPI_RESID, 1, false>(nw, amode, g, grid, lds, s, occ); break;
        default: break;
    }
}

}  // namespace pn
