// gdr_recurrent_step: one decode token of the gated delta rule, state in place.
//
// The rule S_t = S_{t-1} alpha (I - beta k k^T) + beta v k^T with o = S_t q
// ("Gated Delta Networks", agihunt.info, "Method"; GDN review on
// meaningful96.github.io, sections 1 and 3.4) touches row i of S (value
// channel i) only through that row, v_i and the shared k, q, alpha, beta.
// So one pass over each row suffices:
//   a_i = s_i . k,  c_i = s_i . q            (both from the old row)
//   d_i = beta (v_i - alpha a_i)
//   s_i <- alpha s_i + d_i k
//   o_i = s_new . q = alpha c_i + d_i (k . q)
//
// The op is bound by HBM: each (n, h) streams Dv x Dk fp32 in and out once
// (128 KiB at d = 128) against ~7 d^2 flops.  Layout of the work:
//   * one 256-thread workgroup per (n, h), four waves, Dv/4 rows per wave;
//   * a row of Dk floats is read by Dk/4 lanes with one 16-byte load each,
//     so a wave covers 2 rows (d = 128) or 4 rows (d = 64) per access and
//     every access is a fully coalesced 1 KiB;
//   * a wave issues all of its row loads before any arithmetic, so each
//     wave keeps Dv/4 x Dk x 4 bytes (8 KiB at d = 128) in flight;
//   * the two row dot products are reduced across the Dk/4 lanes of a row
//     with xor shuffles that never leave the row's lane group;
//   * state traffic uses non-temporal loads and stores: every byte is
//     touched exactly once per call;
//   * with GDR_L2NORM_QK, q and k are scaled by 1 / norm after the load;
//     their sums of squares take the same in-row reduction as the dots.
#include "gdr_device.h"
#include "launch.h"

namespace gdr {

template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
    return x;
}

template <int DK, int DV, typename TIn, typename TOut>
__global__ __launch_bounds__(256) void step_kernel(
    const TIn* __restrict__ q, const TIn* __restrict__ k,
    const TIn* __restrict__ v, const float* __restrict__ alpha,
    const float* __restrict__ beta, float* __restrict__ state,
    TOut* __restrict__ o, bool l2norm) {
    constexpr int LPR = DK / 4;               // lanes per row
    constexpr int RPP = 64 / LPR;             // rows per wave access
    constexpr int ROWS_W = DV / 4;            // rows per wave
    constexpr int PASSES = ROWS_W / RPP;
    static_assert(PASSES * RPP == ROWS_W, "row split");

    const int64_t head = blockIdx.x;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int cg = lane % LPR;                // 4 columns 4cg .. 4cg+3
    const int rsub = lane / LPR;

    float* S = state + head * (int64_t)(DV * DK);
    const int row0 = wave * ROWS_W + rsub;

    f32x4 s[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
        s[p] = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4*>(S + (row0 + p * RPP) * DK) + cg);

    float kk[4], qq[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        kk[j] = io<TIn>::ld(k + head * DK + 4 * cg + j);
        qq[j] = io<TIn>::ld(q + head * DK + 4 * cg + j);
    }
    const float a = alpha[head];
    const float b = beta[head];
    float vv[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
        vv[p] = io<TIn>::ld(v + head * DV + row0 + p * RPP);

    if (l2norm) {
        const float rk = l2_inv(row_sum<LPR>(kk[0] * kk[0] + kk[1] * kk[1] +
                                             kk[2] * kk[2] + kk[3] * kk[3]));
        const float rq = l2_inv(row_sum<LPR>(qq[0] * qq[0] + qq[1] * qq[1] +
                                             qq[2] * qq[2] + qq[3] * qq[3]));
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            kk[j] *= rk;
            qq[j] *= rq;
        }
    }
    const float kq = row_sum<LPR>(kk[0] * qq[0] + kk[1] * qq[1] +
                                  kk[2] * qq[2] + kk[3] * qq[3]);

#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        float sk = s[p].x * kk[0] + s[p].y * kk[1] + s[p].z * kk[2] + s[p].w * kk[3];
        float sq = s[p].x * qq[0] + s[p].y * qq[1] + s[p].z * qq[2] + s[p].w * qq[3];
        sk = row_sum<LPR>(sk);
        sq = row_sum<LPR>(sq);
        const float d = b * (vv[p] - a * sk);
        f32x4 n;
        n.x = a * s[p].x + d * kk[0];
        n.y = a * s[p].y + d * kk[1];
        n.z = a * s[p].z + d * kk[2];
        n.w = a * s[p].w + d * kk[3];
        __builtin_nontemporal_store(
            n, reinterpret_cast<f32x4*>(S + (row0 + p * RPP) * DK) + cg);
        if (cg == 0) io<TOut>::st(o + head * DV + row0 + p * RPP, a * sq + d * kq);
    }
}

template <int DK, int DV, typename TIn, typename TOut>
static hipError_t launch_step_t(const StepArgs& a) {
    hipLaunchKernelGGL((step_kernel<DK, DV, TIn, TOut>), dim3((unsigned)(a.N * a.H)),
                       dim3(256), 0, a.stream, (const TIn*)a.q, (const TIn*)a.k,
                       (const TIn*)a.v, a.alpha, a.beta, a.state, (TOut*)a.o, a.l2norm);
    return hipGetLastError();
}

template <int DK, int DV>
static hipError_t launch_step_d(const StepArgs& a) {
    if (a.in_bf16) {
        return a.out_bf16 ? launch_step_t<DK, DV, bf16_t, bf16_t>(a)
                          : launch_step_t<DK, DV, bf16_t, float>(a);
    }
    return a.out_bf16 ? launch_step_t<DK, DV, float, bf16_t>(a)
                      : launch_step_t<DK, DV, float, float>(a);
}

hipError_t launch_step(const StepArgs& a) {
    if (a.Dk == 128 && a.Dv == 128) return launch_step_d<128, 128>(a);
    if (a.Dk == 128 && a.Dv == 64) return launch_step_d<128, 64>(a);
    if (a.Dk == 64 && a.Dv == 128) return launch_step_d<64, 128>(a);
    return launch_step_d<64, 64>(a);
}

}  // namespace gdr
