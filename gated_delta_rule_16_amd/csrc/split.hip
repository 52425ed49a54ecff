// Kernels of the sequence-split calls (gdr_chunk_fwd_split,
// gdr_chunk_bwd_split): identity and zero fills, the scans over segment
// transitions (forward for the start states, reverse for the backward's
// carry), and the gather of one segment's state per sequence.
//
// The state map of a segment is affine in its start state: running the rule
// over tokens t0 .. t1 from S gives S P + R, where R is the result from a
// zero start and P = prod_t alpha_t (I - beta_t k_t k_t^T) is the result of
// the same run with v = 0 from the identity (the chunked form of the rule,
// "Gated Delta Networks", agihunt.info, "Method"; GDN review on
// meaningful96.github.io, section 3.4, written for a whole segment).  The
// start states of consecutive segments follow S_in(p) = S_in(p - 1) P_{p-1}
// + R_{p-1}.
#include "gdr_device.h"
#include "launch.h"

namespace gdr {

namespace {

constexpr int SROWS = 16;   // state rows per scan workgroup

// x[n][i][j] = (i == j) for n matrices of d x d
__global__ __launch_bounds__(256) void identity_kernel(float* __restrict__ x, int64_t n, int d) {
    const int64_t dd = (int64_t)d * d;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n * dd;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t e = i % dd;
        x[i] = (e / d == e % d) ? 1.f : 0.f;
    }
}

// n16 16-byte words of zeros
__global__ __launch_bounds__(256) void zero_kernel(u32x4* __restrict__ x, int64_t n16) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
         i += (int64_t)gridDim.x * blockDim.x)
        x[i] = u32x4{0u, 0u, 0u, 0u};
}

// For each (b, h) and rows row0 .. row0 + 15, a chain over the segments on
// the fp32 matrix cores (v_mfma_f32_16x16x4_f32: the same fp32 products and
// sums as the recurrence, in blocks of four):
// - forward (REV false): S = s0 (or 0); for p = 0 .. nseg - 1,
//   Sin[b nseg + p] = S, then S = S P[b nseg + p] + R[b nseg + p];
// - reverse (REV true), the backward's carry dL/dS_in(p) = G_end(p) P_p^T +
//   N_p with N_p the segment's own contribution (its backward from
//   G_end = 0): G = dsf (or 0); for p = nseg - 1 .. 0, Gend[b nseg + p] = G,
//   then G = G P[b nseg + p]^T + N[b nseg + p].
// (init, X, out) are (s0, R, Sin) forward and (dsf, N, Gend) in reverse.
// Wave w owns column tiles TW w .. TW w + TW - 1 of the state as
// accumulators (register r: row 4 (l / 16) + r, column l mod 16 of the
// tile); P is staged row-major in LDS once per step and read as the B
// operand (P, or P^T by swapped indices), the state as the A operand from a
// row copy in LDS.  The next step's P and X are loaded into registers while
// the current step computes.
template <int DK, int DV, bool REV>
__global__ __launch_bounds__(256) void split_scan_kernel(int64_t H, int nseg,
                                                         const float* __restrict__ init,
                                                         const float* __restrict__ X,
                                                         const float* __restrict__ P,
                                                         float* __restrict__ out) {
    // P rows DK + 16 apart forward (a B read spans four rows: four disjoint
    // 16-bank groups) and DK + 4 in reverse (a B read spans 16 rows at four
    // columns: rows four banks apart); state rows DK + 4 (the 16 rows of one
    // A read on distinct banks)
    constexpr int PP = REV ? DK + 4 : DK + 16;
    constexpr int PS = DK + 4;
    constexpr int TW = DK / 16 / 4;          // column tiles per wave
    constexpr int NP = DK * DK / 4 / 256;    // 16-byte pieces of P per thread
    static_assert(TW >= 1 && NP >= 1, "shape");
    __shared__ __align__(16) float Ps[DK * PP];
    __shared__ __align__(16) float Sr[SROWS * PS];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    const int64_t unit = blockIdx.x / (DV / SROWS);
    const int row0 = (int)(blockIdx.x % (DV / SROWS)) * SROWS;
    const int64_t h = unit % H, b = unit / H;
    auto seg_of = [&](int p) { return (b * nseg + p) * H + h; };
    // element (4 lg + r, column of tile t) of this lane within a d_v x d_k
    // state of the workgroup's rows
    auto at = [&](int t, int r) {
        return (int64_t)(row0 + 4 * lg + r) * DK + 16 * (TW * wv + t) + l16;
    };
    f32x4 pr[NP];
    f32x4 xr[TW];
    auto fetch = [&](int p) {
        const int64_t seg = seg_of(p);
#pragma unroll
        for (int it = 0; it < NP; ++it) {
            const int e = tid + 256 * it;
            const int m = e / (DK / 4), c = 4 * (e % (DK / 4));
            pr[it] = *reinterpret_cast<const f32x4*>(P + (seg * DK + m) * DK + c);
        }
#pragma unroll
        for (int t = 0; t < TW; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) xr[t][r] = X[seg * DV * DK + at(t, r)];
    };
    f32x4 s[TW];
#pragma unroll
    for (int t = 0; t < TW; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) s[t][r] = init ? init[(b * H + h) * DV * DK + at(t, r)] : 0.f;
    if (nseg > 1) fetch(REV ? nseg - 1 : 0);
    for (int q = 0; q < nseg; ++q) {
        const int p = REV ? nseg - 1 - q : q;
        const int64_t seg = seg_of(p);
#pragma unroll
        for (int t = 0; t < TW; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) out[seg * DV * DK + at(t, r)] = s[t][r];
        if (q == nseg - 1) break;
        __syncthreads();   // the previous step's reads of Ps and Sr are done
#pragma unroll
        for (int it = 0; it < NP; ++it) {
            const int e = tid + 256 * it;
            const int m = e / (DK / 4), c = 4 * (e % (DK / 4));
            *reinterpret_cast<f32x4*>(Ps + m * PP + c) = pr[it];
        }
#pragma unroll
        for (int t = 0; t < TW; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) Sr[(4 * lg + r) * PS + 16 * (TW * wv + t) + l16] = s[t][r];
        f32x4 acc[TW];
#pragma unroll
        for (int t = 0; t < TW; ++t) acc[t] = xr[t];
        if (q + 1 < nseg - 1) fetch(REV ? p - 1 : p + 1);
        __syncthreads();
#pragma unroll
        for (int kb = 0; kb < DK / 4; ++kb) {
            const float av = Sr[l16 * PS + 4 * kb + lg];
#pragma unroll
            for (int t = 0; t < TW; ++t) {
                const int k = 4 * kb + lg, n = 16 * (TW * wv + t) + l16;
                const float bv = REV ? Ps[n * PP + k] : Ps[k * PP + n];
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv, acc[t], 0, 0, 0);
            }
        }
#pragma unroll
        for (int t = 0; t < TW; ++t) s[t] = acc[t];
    }
}

// sf[b] = F[b nseg + seg] (each `per` floats): one segment's state per
// sequence (the last segment's final state, the first segment's dS_0)
__global__ __launch_bounds__(256) void seg_state_kernel(const float* __restrict__ F,
                                                        float* __restrict__ sf, int64_t B,
                                                        int nseg, int seg, int64_t per) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < B * per;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t b = i / per, e = i % per;
        sf[i] = F[(b * nseg + seg) * per + e];
    }
}

template <int DK, int DV>
hipError_t rscan_t(const SplitScanArgs& a) {
    const int64_t blocks = a.B * a.H * (DV / SROWS);
    hipLaunchKernelGGL((split_scan_kernel<DK, DV, true>), dim3((unsigned)blocks), dim3(256), 0,
                       a.stream, a.H, a.nseg, a.s0, a.R, a.P, a.Sin);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t scan_t(const SplitScanArgs& a) {
    const int64_t blocks = a.B * a.H * (DV / SROWS);
    hipLaunchKernelGGL((split_scan_kernel<DK, DV, false>), dim3((unsigned)blocks), dim3(256), 0,
                       a.stream, a.H, a.nseg, a.s0, a.R, a.P, a.Sin);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_identity(float* x, int64_t n, int d, hipStream_t st) {
    const int64_t total = n * d * d;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(identity_kernel, dim3(stride_blocks(total)), dim3(256), 0, st, x, n, d);
    return hipGetLastError();
}

hipError_t launch_zero(void* x, int64_t bytes, hipStream_t st) {
    const int64_t n16 = bytes / 16;
    if (n16 == 0) return hipSuccess;
    hipLaunchKernelGGL(zero_kernel, dim3(stride_blocks(n16)), dim3(256), 0, st,
                       reinterpret_cast<u32x4*>(x), n16);
    return hipGetLastError();
}

hipError_t launch_split_scan(const SplitScanArgs& a) {
    if (a.Dk == 128 && a.Dv == 128) return scan_t<128, 128>(a);
    if (a.Dk == 128 && a.Dv == 64) return scan_t<128, 64>(a);
    if (a.Dk == 64 && a.Dv == 128) return scan_t<64, 128>(a);
    return scan_t<64, 64>(a);
}

// the same arguments, read as: s0 = dL/dS_T or NULL, R = N, P = P, Sin = Gend
hipError_t launch_split_rscan(const SplitScanArgs& a) {
    if (a.Dk == 128 && a.Dv == 128) return rscan_t<128, 128>(a);
    if (a.Dk == 128 && a.Dv == 64) return rscan_t<128, 64>(a);
    if (a.Dk == 64 && a.Dv == 128) return rscan_t<64, 128>(a);
    return rscan_t<64, 64>(a);
}

hipError_t launch_seg_state(const float* F, float* sf, int64_t B, int nseg, int seg,
                            int64_t per, hipStream_t st) {
    const int64_t total = B * per;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(seg_state_kernel, dim3(stride_blocks(total)), dim3(256), 0, st, F, sf, B,
                       nseg, seg, per);
    return hipGetLastError();
}

}  // namespace gdr
