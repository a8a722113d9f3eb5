// pn_attn.hip - split-K flash-decode attention and its split merge for one
// (head_dim, KV type) pair.  Compiled once per pair with -DPN_D=<32|64|128>
// -DPN_KV=<0|1|2> (fp32, bf16, Q4) -DPN_NAME=<entry>.
#include "pn_launch.hpp"

namespace pn {
namespace {

template <int G>
void go(const AttnArgs &a, dim3 grid, bool merge, hipStream_t s) {
    // fp32 and Q4 caches go to the vector units; a bf16 one where a.kind says
    // (prefill rows in tiles of 16 / G when a.tile is set)
    // (8-wave work-groups for decode with G <= 4, where a.waves asks for them)
    if (PN_KV == 1 && a.kind == 1 && a.tile > 1) hipLaunchKernelGGL((k_attn_mfma<PN_D, G, 16 / G>), grid, dim3(256), 0, s, a);
    else if (PN_KV == 1 && a.kind == 1 && G <= 4 && a.waves == 8)
        hipLaunchKernelGGL((k_attn_mfma<PN_D, G, 1, (G <= 4 ? 8 : kAttnWaves)>), grid, dim3(512), 0, s, a);
    else if (PN_KV == 1 && a.kind == 1) hipLaunchKernelGGL((k_attn_mfma<PN_D, G>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((k_attn<PN_D, PN_KV, G>), grid, dim3(256), 0, s, a);
    if (merge) hipLaunchKernelGGL((k_attn_merge<PN_D, G>), dim3(a.Hq, grid.z), dim3(256), 0, s, a);
}

}  // namespace

void PN_NAME(int G, const AttnArgs &a, dim3 grid, bool merge, hipStream_t s) {
    switch (G) {
        case 1: go<1>(a, grid, merge, s); break;
        case 2: go<2>(a, grid, merge, s); break;
        case 3: go<3>(a, grid, merge, s); break;
        case 4: go<4>(a, grid, merge, s); break;
        case 6: go<6>(a, grid, merge, s); break;
        default: go<8>(a, grid, merge, s); break;
    }
}

}  // namespace pn
