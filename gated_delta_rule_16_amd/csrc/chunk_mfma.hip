// Launches of the bf16 chunk kernel (chunk_kernel.h) for gdr_chunk_fwd and
// its _ex, split and backward-state uses: every head dim pair, row block,
// output dtype and the fused q, k normalisation.
#include "chunk_kernel.h"

namespace gdr {

namespace {

template <int DK, int DV, int RB, typename TOut, bool NORM, bool NOO = false>
hipError_t launch_bf16_n(const ChunkArgs& a) {
    Bf16Params p{};   // bh0 = 0: all heads in one launch
    p.T = a.T;
    p.H = a.H;
    p.BH = a.B * a.H;
    p.q = (const bf16_t*)a.q;
    p.k = (const bf16_t*)a.k;
    p.v = (const bf16_t*)a.v;
    p.alpha = (const float*)a.alpha;
    p.beta = (const float*)a.beta;
    p.s0 = a.s0;
    p.o = a.o;
    p.s_final = a.s_final;
    const size_t lds = Lay<DK, RB, NORM>::TOTAL;
    auto fn = chunk_bf16_kernel<DK, DV, RB, TOut, NORM, false, NOO>;
    hipError_t e =
        hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    // 8 * ceil(B*H / 8) heads' worth of row blocks; surplus workgroups exit
    const unsigned grid = (unsigned)(((a.B * a.H + 7) / 8) * 8 * (DV / RB));
    hipLaunchKernelGGL(fn, dim3(grid), dim3(64 * (RB / 16 + NB)), lds, a.stream, p);
    return hipGetLastError();
}

template <int DK, int DV, int RB, typename TOut>
hipError_t launch_bf16_t(const ChunkArgs& a) {
    if (!a.o)   // only the final state wanted (the sequence split's state passes)
        return a.l2norm ? launch_bf16_n<DK, DV, RB, float, true, true>(a)
                        : launch_bf16_n<DK, DV, RB, float, false, true>(a);
    return a.l2norm ? launch_bf16_n<DK, DV, RB, TOut, true>(a)
                    : launch_bf16_n<DK, DV, RB, TOut, false>(a);
}

template <int DK, int DV>
hipError_t launch_bf16_d(const ChunkArgs& a) {
    if (narrow_row_blocks(a.B * a.H, DV)) {
        return a.out_bf16 ? launch_bf16_t<DK, DV, 16, bf16_t>(a) : launch_bf16_t<DK, DV, 16, float>(a);
    }
    return a.out_bf16 ? launch_bf16_t<DK, DV, 64, bf16_t>(a) : launch_bf16_t<DK, DV, 64, float>(a);
}

}  // namespace

hipError_t launch_chunk_bf16(const ChunkArgs& a) {
    if (a.Dk == 128 && a.Dv == 128) return launch_bf16_d<128, 128>(a);
    if (a.Dk == 128 && a.Dv == 64) return launch_bf16_d<128, 64>(a);
    if (a.Dk == 64 && a.Dv == 128) return launch_bf16_d<64, 128>(a);
    return launch_bf16_d<64, 64>(a);
}

}  // namespace gdr
