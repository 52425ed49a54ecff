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
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n * d * d) return;
    const int64_t e = i % ((int64_t)d * d);
    x[i] = (e / d == e % d) ? 1.f : 0.f;
}

// n16 16-byte words of zeros
__global__ __launch_bounds__(256) void zero_kernel(u32x4* __restrict__ x, int64_t n16) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n16) x[i] = u32x4{0u, 0u, 0u, 0u};
}

// For each (b, h) and rows row0 .. row0 + 15: S = s0 (or 0); for p < nseg,
// Sin[b nseg + p] = S, then S = S P[b nseg + p] + R[b nseg + p].  P goes
// through LDS; each thread keeps DK / 16 entries of its row.  The next
// step's P and R are loaded into registers while the current step computes.
template <int DK, int DV>
__global__ __launch_bounds__(256) void split_scan_kernel(int64_t H, int nseg,
                                                         const float* __restrict__ s0,
                                                         const float* __restrict__ R,
                                                         const float* __restrict__ P,
                                                         float* __restrict__ Sin) {
    constexpr int PK = DK + 4;
    constexpr int NCOL = DK / 16;
    constexpr int NP = DK * DK / 4 / 256;   // 16-byte pieces of P per thread
    __shared__ __align__(16) float Ps[DK * PK];
    __shared__ __align__(16) float Sr[SROWS * PK];
    const int tid = threadIdx.x;
    const int64_t unit = blockIdx.x / (DV / SROWS);
    const int row0 = (int)(blockIdx.x % (DV / SROWS)) * SROWS;
    const int64_t h = unit % H, b = unit / H;
    const int i = tid >> 4, j0 = NCOL * (tid & 15);
    auto seg_of = [&](int p) { return (b * nseg + p) * H + h; };
    f32x4 pr[NP];
    float rr[NCOL];
    auto fetch = [&](int p) {
        const int64_t seg = seg_of(p);
#pragma unroll
        for (int it = 0; it < NP; ++it) {
            const int e = tid + 256 * it;
            const int m = e / (DK / 4), c = 4 * (e % (DK / 4));
            pr[it] = *reinterpret_cast<const f32x4*>(P + (seg * DK + m) * DK + c);
        }
#pragma unroll
        for (int j = 0; j < NCOL; ++j) rr[j] = R[(seg * DV + row0 + i) * DK + j0 + j];
    };
    float s[NCOL];
#pragma unroll
    for (int j = 0; j < NCOL; ++j)
        s[j] = s0 ? s0[((b * H + h) * DV + row0 + i) * DK + j0 + j] : 0.f;
    if (nseg > 1) fetch(0);
    for (int p = 0; p < nseg; ++p) {
        const int64_t seg = seg_of(p);
#pragma unroll
        for (int j = 0; j < NCOL; ++j) Sin[(seg * DV + row0 + i) * DK + j0 + j] = s[j];
        if (p == nseg - 1) break;
        __syncthreads();   // the previous step's reads of Ps and Sr are done
#pragma unroll
        for (int it = 0; it < NP; ++it) {
            const int e = tid + 256 * it;
            const int m = e / (DK / 4), c = 4 * (e % (DK / 4));
            *reinterpret_cast<f32x4*>(Ps + m * PK + c) = pr[it];
        }
#pragma unroll
        for (int j = 0; j < NCOL; ++j) Sr[i * PK + j0 + j] = s[j];
        float acc[NCOL];
#pragma unroll
        for (int j = 0; j < NCOL; ++j) acc[j] = rr[j];
        if (p + 1 < nseg - 1) fetch(p + 1);
        __syncthreads();
#pragma unroll 4
        for (int m = 0; m < DK; ++m) {
            const float sm = Sr[i * PK + m];
#pragma unroll
            for (int j = 0; j < NCOL; ++j) acc[j] += sm * Ps[m * PK + j0 + j];
        }
#pragma unroll
        for (int j = 0; j < NCOL; ++j) s[j] = acc[j];
    }
}

// The backward's carry composes the same way in reverse: dL/dS_in(p) =
// G_end(p) P_p^T + N_p, with N_p the segment's own contribution (its
// backward from G_end = 0).  For each (b, h) and rows row0 .. row0 + 15:
// G = dsf (or 0) for the last segment; for p = nseg - 1 .. 1,
// Gend[b nseg + p] = G, then G = G P[b nseg + p]^T + N[b nseg + p];
// Gend[b nseg] = G.  P_p^T staged in LDS, as in split_scan_kernel.
template <int DK, int DV>
__global__ __launch_bounds__(256) void split_rscan_kernel(int64_t H, int nseg,
                                                          const float* __restrict__ dsf,
                                                          const float* __restrict__ N,
                                                          const float* __restrict__ P,
                                                          float* __restrict__ Gend) {
    constexpr int PK = DK + 4;
    constexpr int NCOL = DK / 16;
    constexpr int NP = DK * DK / 4 / 256;
    __shared__ __align__(16) float Pt[DK * PK];   // Pt[m][j] = P[j][m]
    __shared__ __align__(16) float Gr[SROWS * PK];
    const int tid = threadIdx.x;
    const int64_t unit = blockIdx.x / (DV / SROWS);
    const int row0 = (int)(blockIdx.x % (DV / SROWS)) * SROWS;
    const int64_t h = unit % H, b = unit / H;
    const int i = tid >> 4, j0 = NCOL * (tid & 15);
    auto seg_of = [&](int p) { return (b * nseg + p) * H + h; };
    f32x4 pr[NP];
    float nr[NCOL];
    auto fetch = [&](int p) {
        const int64_t seg = seg_of(p);
#pragma unroll
        for (int it = 0; it < NP; ++it) {
            const int e = tid + 256 * it;
            const int m = e / (DK / 4), c = 4 * (e % (DK / 4));
            pr[it] = *reinterpret_cast<const f32x4*>(P + (seg * DK + m) * DK + c);
        }
#pragma unroll
        for (int j = 0; j < NCOL; ++j) nr[j] = N[(seg * DV + row0 + i) * DK + j0 + j];
    };
    float gv[NCOL];
#pragma unroll
    for (int j = 0; j < NCOL; ++j)
        gv[j] = dsf ? dsf[((b * H + h) * DV + row0 + i) * DK + j0 + j] : 0.f;
    if (nseg > 1) fetch(nseg - 1);
    for (int p = nseg - 1; p >= 0; --p) {
        const int64_t seg = seg_of(p);
#pragma unroll
        for (int j = 0; j < NCOL; ++j) Gend[(seg * DV + row0 + i) * DK + j0 + j] = gv[j];
        if (p == 0) break;
        __syncthreads();   // the previous step's reads of Pt and Gr are done
#pragma unroll
        for (int it = 0; it < NP; ++it) {   // transposed into LDS
            const int e = tid + 256 * it;
            const int m = e / (DK / 4), c = 4 * (e % (DK / 4));
#pragma unroll
            for (int z = 0; z < 4; ++z) Pt[(c + z) * PK + m] = pr[it][z];
        }
#pragma unroll
        for (int j = 0; j < NCOL; ++j) Gr[i * PK + j0 + j] = gv[j];
        float acc[NCOL];
#pragma unroll
        for (int j = 0; j < NCOL; ++j) acc[j] = nr[j];
        if (p - 1 > 0) fetch(p - 1);
        __syncthreads();
#pragma unroll 4
        for (int m = 0; m < DK; ++m) {
            const float gm = Gr[i * PK + m];
#pragma unroll
            for (int j = 0; j < NCOL; ++j) acc[j] += gm * Pt[m * PK + j0 + j];
        }
#pragma unroll
        for (int j = 0; j < NCOL; ++j) gv[j] = acc[j];
    }
}

// sf[b] = F[b nseg + seg] (each `per` floats): one segment's state per
// sequence (the last segment's final state, the first segment's dS_0)
__global__ __launch_bounds__(256) void seg_state_kernel(const float* __restrict__ F,
                                                        float* __restrict__ sf, int64_t B,
                                                        int nseg, int seg, int64_t per) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= B * per) return;
    const int64_t b = i / per, e = i % per;
    sf[i] = F[(b * nseg + seg) * per + e];
}

template <int DK, int DV>
hipError_t rscan_t(const SplitScanArgs& a) {
    const int64_t blocks = a.B * a.H * (DV / SROWS);
    hipLaunchKernelGGL((split_rscan_kernel<DK, DV>), dim3((unsigned)blocks), dim3(256), 0,
                       a.stream, a.H, a.nseg, a.s0, a.R, a.P, a.Sin);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t scan_t(const SplitScanArgs& a) {
    const int64_t blocks = a.B * a.H * (DV / SROWS);
    hipLaunchKernelGGL((split_scan_kernel<DK, DV>), dim3((unsigned)blocks), dim3(256), 0, a.stream,
                       a.H, a.nseg, a.s0, a.R, a.P, a.Sin);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_identity(float* x, int64_t n, int d, hipStream_t st) {
    const int64_t total = n * d * d;
    if (total == 0) return hipSuccess;
    hipLaunchKernelGGL(identity_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, x,
                       n, d);
    return hipGetLastError();
}

hipError_t launch_zero(void* x, int64_t bytes, hipStream_t st) {
    const int64_t n16 = bytes / 16;
    if (n16 == 0) return hipSuccess;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, st,
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
    hipLaunchKernelGGL(seg_state_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st,
                       F, sf, B, nseg, seg, per);
    return hipGetLastError();
}

}  // namespace gdr
