// Helpers of the backward kernels: 16-byte LDS reads, element loads of either
// input type, raw vector loads of global rows, 16 x 16 tiles on the fp32
// matrix cores, DPP row sums, and the reduce kernel of the fused L2 norm.
#pragma once

#include "gdr_device.h"

namespace gdr {

__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

template <typename T>
__device__ __forceinline__ float ldf(const void* p, int64_t i) {
    return io<T>::ld(reinterpret_cast<const T*>(p) + i);
}

typedef uint32_t u32x2w __attribute__((ext_vector_type(2)));

// Buffer resource over [base, base + bytes): loads past the end read 0,
// stores and atomics past it are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// W 32-bit words from global memory in one or a few vector loads; the
// address is aligned to min(16, 4 W) bytes.  Loads kept as raw words so that
// they can be issued a chunk ahead and converted when they are used.
template <int W>
__device__ __forceinline__ void ldw(uint32_t (&w)[W], const void* p) {
    if constexpr (W % 4 == 0) {
#pragma unroll
        for (int h = 0; h < W / 4; ++h) {
            const u32x4 x = reinterpret_cast<const u32x4*>(p)[h];
            w[4 * h] = x[0];
            w[4 * h + 1] = x[1];
            w[4 * h + 2] = x[2];
            w[4 * h + 3] = x[3];
        }
    } else if constexpr (W == 2) {
        const u32x2w x = *reinterpret_cast<const u32x2w*>(p);
        w[0] = x[0];
        w[1] = x[1];
    } else {
        static_assert(W == 1, "1, 2 or a multiple of 4 words");
        w[0] = *reinterpret_cast<const uint32_t*>(p);
    }
}

// Element y of a vector of T held as packed 32-bit words, as fp32.
template <typename T> struct packed;
template <> struct packed<float> {
    static constexpr int PER_WORD = 1;
    __device__ __forceinline__ static float at(const uint32_t* w, int y) {
        return __uint_as_float(w[y]);
    }
};
template <> struct packed<bf16_t> {
    static constexpr int PER_WORD = 2;
    __device__ __forceinline__ static float at(const uint32_t* w, int y) {
        const uint32_t u = w[y >> 1];
        return __uint_as_float((y & 1) ? (u & 0xffff0000u) : (u << 16));
    }
};

// acc += A B for one 16 x 16 tile over K = 16 NQ on the fp32 matrix cores.
// Lane l holds D[4 (l / 16) + i][l % 16] in acc[i].  Operands from LDS:
// A(m, k) = AR ? A[m pa + k] : A[k pa + m], B(k, n) = BR ? B[n pb + k] : B[k pb + n]
// (NEG negates A).  Inside each 16-deep block, lane group g = l / 16 takes
// k = 16 q + 4 g + e on the e-th instruction, so a row operand is one 16-byte
// read per block and a column operand reads rows 4 apart across the groups.
// `lane` is the caller's lane index (a caller may pass a copy that the
// compiler cannot hoist out of its loop, so that the operand addresses are
// formed where they are used instead of being held in registers).
template <int NQ, bool AR, bool BR, bool NEG = false>
__device__ __forceinline__ f32x4 mma16(f32x4 acc, const float* A, int pa, const float* B, int pb,
                                       int lane = threadIdx.x & 63) {
    const int l16 = lane & 15, g = lane >> 4;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        const int kb = 16 * q + 4 * g;
        f32x4 av, bv;
        if constexpr (AR) {
            av = ld4(A + l16 * pa + kb);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) av[e] = A[(kb + e) * pa + l16];
        }
        if constexpr (BR) {
            bv = ld4(B + l16 * pb + kb);
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) bv[e] = B[(kb + e) * pb + l16];
        }
        if constexpr (NEG) av = -av;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            acc = __builtin_amdgcn_mfma_f32_16x16x4f32(av[e], bv[e], acc, 0, 0, 0);
    }
    return acc;
}

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

// log2 of a decay gate, clamped as safe_log: 0 (or a denormal) maps to -126
__device__ __forceinline__ float safe_log2(float a) {
    return fmaxf(__builtin_amdgcn_logf(fmaxf(a, 1.17549435e-38f)), -126.f);
}

// sum over the 4 lanes of each aligned quad (DPP quad_perm xor 1, then xor 2)
__device__ __forceinline__ float qsum(float x) {
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                0xB1, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                0x4E, 0xF, 0xF, false));
    return x;
}

__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
}

// sum over the 16 lanes of each DPP row; every lane gets the sum
__device__ __forceinline__ float rsum16(float x) {
    x = qsum(x);
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                0x141, 0xF, 0xF, false));
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                0x140, 0xF, 0xF, false));
    return x;
}

namespace {

// GDR_L2NORM_QK: the kernel's dq, dk are gradients with respect to q_hat,
// k_hat; one wave per (token, head) row adds the row blocks' partials and
// applies the norm's reverse mode, dx = (dx_hat - x_hat (x_hat . dx_hat)) / n
// with n = sqrt(|x|^2 + eps).  G2: derase and dalpha too (elementwise).
template <int NRB, int DK, typename TIn, bool G2>
__global__ __launch_bounds__(256) void bwd_reduce_rows_norm(
    int64_t rows, const float* __restrict__ pq, const float* __restrict__ pk,
    const float* __restrict__ pb, const float* __restrict__ pg, const void* q, const void* k,
    const void* alpha, float* __restrict__ dq, float* __restrict__ dk, float* __restrict__ db,
    float* __restrict__ da) {
    constexpr int E = DK / 64;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;   // whole waves
    const int lane = threadIdx.x & 63;
    const int64_t n = rows * DK;
    float dqh[E], dkh[E], qv[E], kv[E];
    float sq = 0.f, sk = 0.f, tq = 0.f, tk = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int64_t i = row * DK + lane + 64 * e;
        float a = 0.f, b = 0.f;
#pragma unroll
        for (int r = 0; r < NRB; ++r) {
            a += pq[r * n + i];
            b += pk[r * n + i];
        }
        dqh[e] = a;
        dkh[e] = b;
        qv[e] = ldf<TIn>(q, i);
        kv[e] = ldf<TIn>(k, i);
        sq += qv[e] * qv[e];
        sk += kv[e] * kv[e];
        tq += qv[e] * a;
        tk += kv[e] * b;
        if constexpr (G2) {
            float c = 0.f, d = 0.f;
#pragma unroll
            for (int r = 0; r < NRB; ++r) {
                c += pb[r * n + i];
                d += pg[r * n + i];
            }
            db[i] = c;
            da[i] = d / fmaxf(ldf<TIn>(alpha, i), 1.17549435e-38f);
        }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        sq += __shfl_xor(sq, m, 64);
        sk += __shfl_xor(sk, m, 64);
        tq += __shfl_xor(tq, m, 64);
        tk += __shfl_xor(tk, m, 64);
    }
    const float iq = l2_inv(sq), ik = l2_inv(sk);
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int64_t i = row * DK + lane + 64 * e;
        dq[i] = iq * (dqh[e] - qv[e] * iq * (tq * iq));
        dk[i] = ik * (dkh[e] - kv[e] * ik * (tk * ik));
    }
}

}  // namespace

}  // namespace gdr
