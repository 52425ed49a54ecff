// Register-tiled fp32 products on LDS operands for the vector-ALU kernels
// (the backward passes): 16-byte LDS reads, small register tiles.
#pragma once

#include "gdr_device.h"

namespace gdr {

__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

// c[x][y] = sum_k A[r0 + x][k] B[c0 + y][k] over N (a multiple of 4) for row-
// major A, B with 16-byte-aligned rows: a 2 x 2 register tile, 16-byte reads
// along the contraction.
template <int N>
__device__ __forceinline__ void dot22(const float* A, int pa, int r0, const float* B, int pb,
                                      int c0, float (&c)[2][2]) {
    c[0][0] = c[0][1] = c[1][0] = c[1][1] = 0.f;
#pragma unroll 4
    for (int k = 0; k < N; k += 4) {
        const f32x4 a0 = ld4(A + r0 * pa + k), a1 = ld4(A + (r0 + 1) * pa + k);
        const f32x4 b0 = ld4(B + c0 * pb + k), b1 = ld4(B + (c0 + 1) * pb + k);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            c[0][0] += a0[e] * b0[e];
            c[0][1] += a0[e] * b1[e];
            c[1][0] += a1[e] * b0[e];
            c[1][1] += a1[e] * b1[e];
        }
    }
}

// acc[x][y] += sum_k a(x, k) B[k][c0 + y], k < KN, y < NC (4 or 8): a 2 x NC
// register tile, the right operand read as 16-byte vectors.
template <int KN, int NC, typename FA>
__device__ __forceinline__ void mm2n(float (&acc)[2][NC], FA a, const float* B, int pb, int c0) {
#pragma unroll 4
    for (int k = 0; k < KN; ++k) {
        const float a0 = a(0, k), a1 = a(1, k);
#pragma unroll
        for (int h = 0; h < NC / 4; ++h) {
            const f32x4 b = ld4(B + k * pb + c0 + 4 * h);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[0][4 * h + e] += a0 * b[e];
                acc[1][4 * h + e] += a1 * b[e];
            }
        }
    }
}

template <typename T>
__device__ __forceinline__ float ldf(const void* p, int64_t i) {
    return io<T>::ld(reinterpret_cast<const T*>(p) + i);
}

// acc[y] += sum_k a(k) B[k][c0 + y], k < KN, y < NC (a multiple of 4): a
// 1 x NC register tile.
template <int KN, int NC, typename FA>
__device__ __forceinline__ void mm1n(float (&acc)[NC], FA a, const float* B, int pb, int c0) {
#pragma unroll 4
    for (int k = 0; k < KN; ++k) {
        const float a0 = a(k);
#pragma unroll
        for (int h = 0; h < NC / 4; ++h) {
            const f32x4 b = ld4(B + k * pb + c0 + 4 * h);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[4 * h + e] += a0 * b[e];
        }
    }
}

typedef uint32_t u32x2w __attribute__((ext_vector_type(2)));

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

}  // namespace gdr
