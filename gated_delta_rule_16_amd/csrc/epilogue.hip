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
#include <mutex>

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

// Reverse mode of the gate, per row with r = 1 / sqrt(mean o^2 + eps),
// n = r o, s(g) = g sigmoid(g):
//
//   dn = dy w s(g),  do = r (dn - n mean(n dn)),
//   dg = dy n w sigmoid(g) (1 + g (1 - sigmoid(g))),
//   dw = sum over rows of dy n s(g).
//
// Same lane layout and UNROLL-row steps as the forward (all loads of a step
// before its arithmetic).  dw: each lane sums its 4 channels over the rows
// it visits; lanes of a wave that share channels, then the four waves, are
// added in the workgroup, which writes its partial sums channel-major
// (dwp[c][workgroup]); gate_dw_reduce adds them, one workgroup per channel.
template <int DV, typename TO, typename TG, typename TD>
__global__ __launch_bounds__(256) void output_gate_bwd_kernel(int64_t rows, const TO* o,
                                                              const TG* __restrict__ g,
                                                              const float* __restrict__ w,
                                                              float eps, const TD* dy,
                                                              float* __restrict__ dout,
                                                              float* __restrict__ dg,
                                                              float* __restrict__ dwp) {
    constexpr int LPR = DV / 4;
    constexpr int RPW = 64 / LPR;
    constexpr int RPB = 4 * RPW;
    __shared__ f32x4 red[4][LPR];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int c0 = 4 * (lane % LPR);
    const int64_t rsub = wv * RPW + lane / LPR;
    f32x4 wv4 = {1.f, 1.f, 1.f, 1.f};
    if (w) wv4 = *reinterpret_cast<const f32x4*>(w + c0);
    f32x4 dwacc = {0.f, 0.f, 0.f, 0.f};
    const int64_t stride = (int64_t)gridDim.x * RPB;
    // every lane runs every step's row reductions (the step base is uniform
    // over the workgroup); rows past the end load zeros and store nothing
    for (int64_t base = (int64_t)blockIdx.x * RPB; base < rows; base += UNROLL * stride) {
        f32x4 ov[UNROLL], gv[UNROLL], yv[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int64_t r = base + u * stride + rsub;
            ov[u] = gv[u] = yv[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (r < rows) {
                ov[u] = v4<TO>::ld(o + r * DV + c0);
                gv[u] = v4<TG>::ld(g + r * DV + c0);
                yv[u] = v4<TD>::ld(dy + r * DV + c0);
            }
        }
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const int64_t r = base + u * stride + rsub;
            float ss = ov[u][0] * ov[u][0] + ov[u][1] * ov[u][1] + ov[u][2] * ov[u][2] +
                       ov[u][3] * ov[u][3];
            ss += dpp_mov<0xB1>(ss);
            ss += dpp_mov<0x4E>(ss);
            ss += dpp_mov<0x141>(ss);
            ss += dpp_mov<0x140>(ss);
            if constexpr (LPR == 32) ss += __shfl_xor(ss, 16, 64);
            const float rr = rsqrtf(ss * (1.f / DV) + eps);
            f32x4 nv, dn, sgm;
            float t = 0.f;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sgm[e] = __builtin_amdgcn_rcpf(1.f + __expf(-gv[u][e]));
                nv[e] = ov[u][e] * rr;
                dn[e] = yv[u][e] * wv4[e] * gv[u][e] * sgm[e];
                t += nv[e] * dn[e];
            }
            t += dpp_mov<0xB1>(t);
            t += dpp_mov<0x4E>(t);
            t += dpp_mov<0x141>(t);
            t += dpp_mov<0x140>(t);
            if constexpr (LPR == 32) t += __shfl_xor(t, 16, 64);
            const float tm = t * (1.f / DV);
            if (r < rows) {
                f32x4 dov, dgv;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    dov[e] = rr * (dn[e] - nv[e] * tm);
                    dgv[e] = yv[u][e] * nv[e] * wv4[e] * sgm[e] * (1.f + gv[u][e] * (1.f - sgm[e]));
                    dwacc[e] += yv[u][e] * nv[e] * gv[u][e] * sgm[e];
                }
                st4(dout + r * DV + c0, dov);
                st4(dg + r * DV + c0, dgv);
            }
        }
    }
    if (!dwp) return;
    // lanes of this wave with the same channels: lane % LPR
#pragma unroll
    for (int m = LPR; m < 64; m <<= 1)
#pragma unroll
        for (int e = 0; e < 4; ++e) dwacc[e] += __shfl_xor(dwacc[e], m, 64);
    if (lane < LPR) red[wv][lane] = dwacc;
    __syncthreads();
    if (threadIdx.x < LPR) {
        f32x4 sacc = red[0][threadIdx.x];
#pragma unroll
        for (int k = 1; k < 4; ++k) sacc += red[k][threadIdx.x];
#pragma unroll
        for (int e = 0; e < 4; ++e)
            dwp[(int64_t)(4 * threadIdx.x + e) * gridDim.x + blockIdx.x] = sacc[e];
    }
}

// dw[c] = sum over the workgroups' partial sums dwp[c][0 .. nblk), one
// 256-thread workgroup per channel
__global__ __launch_bounds__(256) void gate_dw_reduce(const float* __restrict__ dwp, int nblk,
                                                     float* __restrict__ dw) {
    __shared__ float red[256];
    const int c = blockIdx.x;
    float sacc = 0.f;
    for (int b = threadIdx.x; b < nblk; b += 256) sacc += dwp[(int64_t)c * nblk + b];
    red[threadIdx.x] = sacc;
    __syncthreads();
    for (int m = 128; m >= 1; m >>= 1) {
        if (threadIdx.x < m) red[threadIdx.x] += red[threadIdx.x + m];
        __syncthreads();
    }
    if (threadIdx.x == 0) dw[c] = red[0];
}

constexpr int GATE_BWD_MAX_BLOCKS = 2048;

template <int DV>
int64_t gate_bwd_blocks(int64_t rows) {
    constexpr int RPB = 4 * (64 / (DV / 4));
    int64_t blocks = (rows + RPB * UNROLL - 1) / (RPB * UNROLL);
    return blocks < GATE_BWD_MAX_BLOCKS ? blocks : GATE_BWD_MAX_BLOCKS;
}

template <int DV, typename TO, typename TG, typename TD>
hipError_t launch_gate_bwd_t(const GateBwdArgs& a) {
    const int64_t rows = a.N * a.H;
    const int64_t blocks = gate_bwd_blocks<DV>(rows);
    float* dwp = a.dw ? reinterpret_cast<float*>(a.workspace) : nullptr;
    hipLaunchKernelGGL((output_gate_bwd_kernel<DV, TO, TG, TD>), dim3((unsigned)blocks), dim3(256),
                       0, a.stream, rows, (const TO*)a.o, (const TG*)a.g, a.w, a.eps,
                       (const TD*)a.dy, a.dout, a.dg, dwp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !a.dw) return e;
    hipLaunchKernelGGL(gate_dw_reduce, dim3(DV), dim3(256), 0, a.stream, dwp, (int)blocks, a.dw);
    return hipGetLastError();
}

template <int DV, typename TO, typename TG>
hipError_t launch_gate_bwd_y(const GateBwdArgs& a) {
    return a.dy_bf16 ? launch_gate_bwd_t<DV, TO, TG, bf16_t>(a)
                     : launch_gate_bwd_t<DV, TO, TG, float>(a);
}

template <int DV, typename TO>
hipError_t launch_gate_bwd_g(const GateBwdArgs& a) {
    return a.g_bf16 ? launch_gate_bwd_y<DV, TO, bf16_t>(a) : launch_gate_bwd_y<DV, TO, float>(a);
}

template <int DV>
hipError_t launch_gate_bwd_d(const GateBwdArgs& a) {
    return a.o_bf16 ? launch_gate_bwd_g<DV, bf16_t>(a) : launch_gate_bwd_g<DV, float>(a);
}

// Scratch of the allocation-free gate backward (gdr_output_gate_bwd_noalloc):
// the workgroups' dw partials, at most GATE_BWD_MAX_BLOCKS x 128 floats
// (1 MiB).  Each GPU the library runs on holds its own copy until the process
// ends.  Host code never passes the array's name to a kernel: on the host it
// is only a stand-in for the symbol, whose device address is looked up once
// per device below.
static __device__ __align__(256) float scratch[GATE_BWD_MAX_BLOCKS * 128];
static_assert(sizeof(scratch) == GDR_GATE_BWD_SCRATCH_BYTES, "scratch size as declared");

constexpr int kMaxDevices = 256;

}  // namespace

size_t gate_bwd_scratch_bytes() { return sizeof(scratch); }

// Device address of `scratch` on the current device: hipGetSymbolAddress is
// called once per device, with that device current, and its result kept.
hipError_t gate_bwd_scratch(float** out) {
    static std::mutex mu;
    static float* addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        addr[dev] = static_cast<float*>(p);
    }
    *out = addr[dev];
    return hipSuccess;
}

size_t gate_bwd_workspace_bytes(int64_t rows, int64_t Dv) {
    const int64_t blocks = Dv == 128 ? gate_bwd_blocks<128>(rows) : gate_bwd_blocks<64>(rows);
    return sizeof(float) * (size_t)(blocks * Dv);
}

hipError_t launch_output_gate_bwd(const GateBwdArgs& a) {
    return a.Dv == 128 ? launch_gate_bwd_d<128>(a) : launch_gate_bwd_d<64>(a);
}

hipError_t launch_output_gate(const GateArgs& a) {
    return a.Dv == 128 ? launch_gate_d<128>(a) : launch_gate_d<64>(a);
}

}  // namespace gdr
