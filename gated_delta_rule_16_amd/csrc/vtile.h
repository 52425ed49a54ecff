// Load helpers of the backward kernel: 16-byte LDS reads, element loads of
// either input type, and raw vector loads of global rows.
#pragma once

#include "gdr_device.h"

namespace gdr {

__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

template <typename T>
__device__ __forceinline__ float ldf(const void* p, int64_t i) {
    return io<T>::ld(reinterpret_cast<const T*>(p) + i);
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
