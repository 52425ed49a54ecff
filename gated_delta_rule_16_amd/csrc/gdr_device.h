// Device-side helpers shared by the gfx950 kernels of libgdr.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gdr.h"

namespace gdr {

typedef uint16_t bf16_t;  // bfloat16 storage (upper half of an fp32)

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// log of the smallest normal float: decay gates are clamped to FLT_MIN
// before the log, so a gate of 0 is a full reset rather than -inf.
constexpr float kLogFltMin = -87.33654475f;

__device__ __forceinline__ float bf2f(bf16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// fp32 -> bf16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ bf16_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<bf16_t>(u >> 16);
}

template <typename T> struct io;
template <> struct io<float> {
    __device__ __forceinline__ static float ld(const float* p) { return *p; }
    __device__ __forceinline__ static void st(float* p, float x) { *p = x; }
};
template <> struct io<bf16_t> {
    __device__ __forceinline__ static float ld(const bf16_t* p) { return bf2f(*p); }
    __device__ __forceinline__ static void st(bf16_t* p, float x) { *p = f2bf(x); }
};

// Natural log of a decay gate, clamped so that 0 (or a denormal) maps to
// log(FLT_MIN).
__device__ __forceinline__ float safe_log(float a) {
    return fmaxf(logf(fmaxf(a, 1.17549435e-38f)), kLogFltMin);
}

// Scale that L2-normalises a q or k row with sum of squares ss
// (GDR_L2NORM_QK): x_hat = x / sqrt(ss + eps).
__device__ __forceinline__ float l2_inv(float ss) { return rsqrtf(ss + GDR_L2NORM_EPS); }

}  // namespace gdr
