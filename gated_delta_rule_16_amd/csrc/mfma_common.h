// bf16 matrix-core building blocks for the chunked kernels (gfx950).
//
// All products use v_mfma_f32_32x32x16_bf16: a 32x32 fp32 tile C += A B with
// a 16-deep contraction.  Lane layouts (lane l = 0..63, l32 = l % 32,
// hi = l / 32):
//   A operand  lane holds A[m = l32][k = 8 hi .. 8 hi + 7]
//   B operand  lane holds B[k = 8 hi .. 8 hi + 7][n = l32]
//   C tile     register r holds C[m = 8 (r / 4) + 4 hi + r % 4][n = l32]
// So both operands are read as 16 contiguous bytes from a row-major bf16
// matrix whose rows run along m (for A) or n (for B) and whose columns run
// along the contraction, and a C tile is naturally written transposed:
// C^T[n][m .. m + 3] is 4 contiguous values.  Every tile stored to LDS by
// these kernels is therefore kept "contraction-major" for its next use.
//
// Precision: a computed fp32 operand x enters as two bf16 terms,
// x = hi + lo with hi = bf16(x), lo = bf16(x - hi); products of two computed
// operands use hi*hi + hi*lo + lo*hi, products with one exact bf16 input use
// hi*x + lo*x.  Each product then carries ~16 significant bits while the
// matrix cores accumulate in fp32.
#pragma once

#include "gdr_device.h"

namespace gdr {

__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16-byte operand fragment: row `row` of a row-major bf16 matrix (pitch in
// elements), contraction offset `k` (a multiple of 8).
__device__ __forceinline__ bf16x8 frag(const bf16_t* base, int pitch, int row, int k) {
    return *reinterpret_cast<const bf16x8*>(base + row * pitch + k);
}

__device__ __forceinline__ void split_bf16(float x, bf16_t& h, bf16_t& l) {
    h = f2bf(x);
    l = f2bf(x - bf2f(h));
}

// Store 4 consecutive values x[0..3] at p as bf16 hi/lo pairs (8 bytes each).
__device__ __forceinline__ void st4_split(bf16_t* ph, bf16_t* pl, float x0, float x1, float x2,
                                          float x3) {
    bf16_t h0, h1, h2, h3, l0, l1, l2, l3;
    split_bf16(x0, h0, l0);
    split_bf16(x1, h1, l1);
    split_bf16(x2, h2, l2);
    split_bf16(x3, h3, l3);
    uint2 vh, vl;
    vh.x = (uint32_t)h0 | ((uint32_t)h1 << 16);
    vh.y = (uint32_t)h2 | ((uint32_t)h3 << 16);
    vl.x = (uint32_t)l0 | ((uint32_t)l1 << 16);
    vl.y = (uint32_t)l2 | ((uint32_t)l3 << 16);
    *reinterpret_cast<uint2*>(ph) = vh;
    *reinterpret_cast<uint2*>(pl) = vl;
}

// Workgroup barrier that orders LDS only: outstanding global loads (the
// next chunk's prefetch) stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace gdr
