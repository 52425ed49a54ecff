// Launches of the bf16 chunk kernel (chunk_kernel.h) with the block's output
// gate fused on its stores, for gdr_chunk_fwd_gate: each workgroup writes
// y = o / sqrt(mean o^2 + eps) w SiLU(gate) instead of o ("Gated DeltaNet-2"
// on agihunt.info, the block paragraph: the recurrent output passes an
// RMSNorm and a SiLU output gate; GDN review on meaningful96.github.io,
// section 3.8).
//
// A token's mean square runs over all Dv rows, which the row blocks of a
// head share out over workgroups; they exchange per-token sums of squares
// through the caller's workspace, each waiting (boundedly) for the others'
// sums.  So every row block of a head must be resident at once: heads go out
// in cooperative launches of at most as many workgroups as the GPU holds.
#include "chunk_kernel.h"

namespace gdr {

namespace {

template <int DK, int DV, int RB, typename TOut, bool NORM>
hipError_t launch_gate_n(const ChunkArgs& a) {
    constexpr int NRB = DV / RB;
    Bf16Params p{};
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
    p.gate = a.gate;
    p.gate_bf16 = a.gate_bf16;
    p.w = a.w;
    p.eps = a.eps;
    p.xch = reinterpret_cast<unsigned long long*>(a.xch);
    const size_t lds = Lay<DK, RB, NORM, true>::TOTAL;
    const int block = 64 * (RB / 16 + NB);
    auto fn = chunk_bf16_kernel<DK, DV, RB, TOut, NORM, true>;
    hipError_t e =
        hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    // exchange words start at zero (no chunk tag); a fill kernel, so the
    // call stays free of memset nodes
    if ((e = launch_zero(a.xch, (int64_t)chunk_gate_xch_bytes(a.B, a.H, a.Dv), a.stream)) !=
        hipSuccess)
        return e;
    int dev = 0, ncu = 0, per_cu = 0;
    if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
    if ((e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev)) !=
        hipSuccess)
        return e;
    if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void*)fn, block, lds)) !=
        hipSuccess)
        return e;
    // heads per launch: whole groups of 8 (the workgroup-to-XCD order),
    // every row block of each resident at once
    const int64_t heads = ((int64_t)ncu * per_cu / NRB) / 8 * 8;
    if (heads < 8) return hipErrorNotSupported;
    for (int64_t bh0 = 0; bh0 < p.BH; bh0 += heads) {
        const int64_t nb = p.BH - bh0 < heads ? p.BH - bh0 : heads;
        p.bh0 = bh0;
        void* args[] = {&p};
        e = hipLaunchCooperativeKernel((const void*)fn, dim3((unsigned)(((nb + 7) / 8) * 8 * NRB)),
                                       dim3(block), args, (unsigned)lds, a.stream);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

template <int DK, int DV, int RB, typename TOut>
hipError_t launch_gate_t(const ChunkArgs& a) {
    return a.l2norm ? launch_gate_n<DK, DV, RB, TOut, true>(a)
                    : launch_gate_n<DK, DV, RB, TOut, false>(a);
}

template <int DK, int DV>
hipError_t launch_gate_d(const ChunkArgs& a) {
    if (narrow_row_blocks(a.B * a.H, DV))
        return a.out_bf16 ? launch_gate_t<DK, DV, 16, bf16_t>(a) : launch_gate_t<DK, DV, 16, float>(a);
    return a.out_bf16 ? launch_gate_t<DK, DV, 64, bf16_t>(a) : launch_gate_t<DK, DV, 64, float>(a);
}

}  // namespace

size_t chunk_gate_xch_bytes(int64_t B, int64_t H, int64_t Dv) {
    // [B H][row blocks][4 chunks][32 tokens] 8-byte words (sum, chunk tag)
    const int64_t nrb = narrow_row_blocks(B * H, Dv) ? Dv / 16 : Dv / 64;
    return (size_t)(B * H * nrb * 4 * 32 * 8);
}

hipError_t launch_chunk_bf16_gate(const ChunkArgs& a) {
    if (a.Dk == 128 && a.Dv == 128) return launch_gate_d<128, 128>(a);
    if (a.Dk == 128 && a.Dv == 64) return launch_gate_d<128, 64>(a);
    if (a.Dk == 64 && a.Dv == 128) return launch_gate_d<64, 128>(a);
    return launch_gate_d<64, 64>(a);
}

}  // namespace gdr
