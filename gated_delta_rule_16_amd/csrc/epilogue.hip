// gdr_output_gate: the block's output gate on the recurrent output,
//
//   y = o / sqrt(mean(o^2) + eps) * w * g * sigmoid(g)
//
// per token and head over the Dv channels: an RMS normalisation (per-channel
// weight w) and a SiLU output gate ("Gated DeltaNet-2" on agihunt.info, the
// block paragraph; GDN review on meaningful96.github.io, section 3.8).  It
// cannot be folded into the chunk kernels' stores: there a head's Dv rows
// are split over workgroups, so the row's mean square would need a
// cross-workgroup reduction.  It is one pass over HBM instead.
//
// Layout: each lane owns 4 consecutive channels of one row (one 16-byte
// fp32 or 8-byte bf16 load per tensor), Dv / 4 lanes per row, 64 / (Dv / 4)
// rows per wave; the row's sum of squares is reduced by DPP inside the 16
// lanes of a DPP row and by one bpermute across rows when Dv = 128.  Each
// lane keeps UNROLL rows in flight, all loads issued before any arithmetic.
// y may be o itself: every element is read and written by the same lane,
// its loads before its stores.
#include "launch.h"
#include "mfma_common.h"

namespace gdr {

namespace {

constexpr int UNROLL = 4;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <typename T> struct v4;
template <> struct v4<float> {
    __device__ __forceinline__ static f32x4 ld(const float* p) {
        return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    }
};
template <> struct v4<bf16_t> {
    __device__ __forceinline__ static f32x4 ld(const bf16_t* p) {
        const u32x2 u = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
        return f32x4{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
    }
};

__device__ __forceinline__ void st4(float* p, const f32x4& x) {
    __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(p));
}
__device__ __forceinline__ void st4(bf16_t* p, const f32x4& x) {
    __builtin_nontemporal_store(u32x2{cvt_pk(x[0], x[1]), cvt_pk(x[2], x[3])},
                                reinterpret_cast<u32x2*>(p));
}

__device__ __forceinline__ float silu(float x) {
    return x * __builtin_amdgcn_rcpf(1.f + __expf(-x));
}

template <int DV, typename TO, typename TG, typename TY>
__global__ __launch_bounds__(256) void output_gate_kernel(int64_t rows, const TO* o,
                                                          const TG* __restrict__ g,
                                                          const float* __restrict__ w, float eps,
                                                          TY* y) {
    constexpr int LPR = DV / 4;          // lanes per row
    constexpr int RPW = 64 / LPR;        // rows per wave
    constexpr int RPB = 4 * RPW;         // rows per workgroup and step
    const int lane = threadIdx.x & 63;
    const int c0 = 4 * (lane % LPR);
    const int64_t rsub = (threadIdx.x >> 6) * RPW + lane / LPR;
    f32x4 wv = {1.f, 1.f, 1.f, 1.f};
    if (w) wv = *reinterpret_cast<const f32x4*>(w + c0);
    const int64_t stride = (int64_t)gridDim.x * RPB;
    for (int64_t r0 = (int64_t)blockIdx.x * RPB + rsub; r0 < rows; r0 += UNROLL * stride) {
        f32x4 ov[UNROLL], gv[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int64_t r = r0 + u * stride;
            ov[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            gv[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (r < rows) {
                ov[u] = v4<TO>::ld(o + r * DV + c0);
                gv[u] = v4<TG>::ld(g + r * DV + c0);
            }
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int64_t r = r0 + u * stride;
            // all lanes of a row share r, and every lane runs the reduction
            // (inactive rows contribute to no live row's sum)
            float ss = ov[u][0] * ov[u][0] + ov[u][1] * ov[u][1] + ov[u][2] * ov[u][2] +
                       ov[u][3] * ov[u][3];
            ss += dpp_mov<0xB1>(ss);    // quad_perm [1, 0, 3, 2]
            ss += dpp_mov<0x4E>(ss);    // quad_perm [2, 3, 0, 1]
            ss += dpp_mov<0x141>(ss);   // row_half_mirror
            ss += dpp_mov<0x140>(ss);   // row_mirror
            if constexpr (LPR == 32) ss += __shfl_xor(ss, 16, 64);
            const float inv = rsqrtf(ss * (1.f / DV) + eps);
            if (r < rows) {
                f32x4 out;
#pragma unroll
                for (int e = 0; e < 4; ++e) out[e] = ov[u][e] * inv * wv[e] * silu(gv[u][e]);
                st4(y + r * DV + c0, out);
            }
        }
    }
}

template <int DV, typename TO, typename TG, typename TY>
hipError_t launch_gate_t(const GateArgs& a) {
    constexpr int RPB = 4 * (64 / (DV / 4));
    const int64_t rows = a.N * a.H;
    int64_t blocks = (rows + RPB * UNROLL - 1) / (RPB * UNROLL);
    blocks = blocks < 8192 ? blocks : 8192;   // 32 workgroups per CU, grid-stride beyond
    hipLaunchKernelGGL((output_gate_kernel<DV, TO, TG, TY>), dim3((unsigned)blocks), dim3(256), 0,
                       a.stream, rows, (const TO*)a.o, (const TG*)a.g, a.w, a.eps, (TY*)a.y);
    return hipGetLastError();
}

template <int DV, typename TO, typename TG>
hipError_t launch_gate_y(const GateArgs& a) {
    return a.out_bf16 ? launch_gate_t<DV, TO, TG, bf16_t>(a) : launch_gate_t<DV, TO, TG, float>(a);
}

template <int DV, typename TO>
hipError_t launch_gate_g(const GateArgs& a) {
    return a.g_bf16 ? launch_gate_y<DV, TO, bf16_t>(a) : launch_gate_y<DV, TO, float>(a);
}

template <int DV>
hipError_t launch_gate_d(const GateArgs& a) {
    return a.o_bf16 ? launch_gate_g<DV, bf16_t>(a) : launch_gate_g<DV, float>(a);
}

}  // namespace

hipError_t launch_output_gate(const GateArgs& a) {
    return a.Dv == 128 ? launch_gate_d<128>(a) : launch_gate_d<64>(a);
}

}  // namespace gdr
