// bf16 matrix-core building blocks for the chunked kernels (gfx950).
//
// The bf16 products use v_mfma_f32_16x16x32_bf16: a 16x16 fp32 tile C += A B
// with a 32-deep contraction.  Lane layouts (lane l = 0..63, g = l / 16,
// m = l % 16):
//   A operand  lane holds A[m][k = 8 g .. 8 g + 7]
//   B operand  lane holds B[k = 8 g .. 8 g + 7][n = m]
//   C tile     register r holds C[4 g + r][m]
// So both operands are 16 contiguous bytes of a row-major bf16 matrix whose
// rows run along m (for A) or n (for B) and whose columns run along the
// contraction; the kernels store their tiles in that "contraction-major"
// order, permuted within each 32-wide block where a later product wants the
// C layout of an earlier one as its operand.
//
// Precision: a computed fp32 operand x enters as two bf16 terms,
// x = hi + lo with hi = bf16(x), lo = bf16(x - hi); products of two computed
// operands use hi*hi + hi*lo + lo*hi, products with one exact bf16 input use
// hi*x + lo*x.  Each product then carries ~16 significant bits while the
// matrix cores accumulate in fp32.
#pragma once

#include "gdr_device.h"

namespace gdr {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// Two fp32 -> packed bf16 pair (v_cvt_pk_bf16_f32, round to nearest even).
__device__ __forceinline__ uint32_t cvt_pk(float a, float b) {
    const bf16x2_t v = __builtin_convertvector((f32x2_t){a, b}, bf16x2_t);
    return __builtin_bit_cast(uint32_t, v);
}

// Four fp32 values stored as bf16 (v_cvt_pk_bf16_f32: round to nearest
// even, NaN kept) at four byte offsets of a buffer resource.
__device__ __forceinline__ void store4_bf16(const f32x4& x, __amdgpu_buffer_rsrc_t r,
                                            const uint32_t (&off)[4]) {
    const uint32_t a = cvt_pk(x[0], x[1]), b = cvt_pk(x[2], x[3]);
    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)a, r, (int)off[0], 0, 0);
    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(a >> 16), r, (int)off[1], 0, 0);
    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)b, r, (int)off[2], 0, 0);
    __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(b >> 16), r, (int)off[3], 0, 0);
}

// hi/lo split of two values: hi = bf16(x), lo = bf16(x - hi).  The
// residuals x - hi come from v_dot2c_f32_bf16 on the packed hi pair,
// dot((hi_a, hi_b), (-1, 0)) + a (and (0, -1) for b): -hi is exact and the
// sum is x - hi, itself exact in fp32, so this matches the plain
// subtraction bit for bit while skipping the unpacking of hi.  The two
// constants live in SGPRs: as inline operands they are mis-encoded.
__device__ __forceinline__ void split2(float a, float b, uint32_t& h, uint32_t& l) {
    h = cvt_pk(a, b);
    uint32_t ka, kb;
    asm("s_mov_b32 %0, 0xbf80" : "=s"(ka));       // (-1, 0) as packed bf16
    asm("s_mov_b32 %0, 0xbf800000" : "=s"(kb));   // (0, -1)
    const bf16x2_t hp = __builtin_bit_cast(bf16x2_t, h);
    const float ra = __builtin_amdgcn_fdot2_f32_bf16(hp, __builtin_bit_cast(bf16x2_t, ka), a, false);
    const float rb = __builtin_amdgcn_fdot2_f32_bf16(hp, __builtin_bit_cast(bf16x2_t, kb), b, false);
    l = cvt_pk(ra, rb);
}

// Transposed LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane 4r + c supplies the address of 4 consecutive 16-bit elements; lane i
// of the group receives element (i & 3) of the chunk supplied by lane
// 4r + (i >> 2), for r = 0..3.  With lane 4r + c pointing at
// M[row0 + r][col0 + 4c] of a row-major matrix, lane i receives the column
// M[row0 .. row0 + 3][col0 + i].
__device__ __forceinline__ s16x4 lds_tr16(const bf16_t* p) {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)((__attribute__((address_space(3))) char*)(
            (__attribute__((address_space(3))) void*)(p))));
}

// fp32 matrix core 16x16x4: A lane l holds A[l % 16][l / 16], B lane l
// holds B[l / 16][l % 16]; C register r holds C[4 (l / 16) + r][l % 16].
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// DPP lane moves (v_mov_b32_dpp); lanes whose source is out of range read 0.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_mov(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                                         0, __builtin_bit_cast(int, x), CTRL, ROW_MASK, 0xF, false));
}

// Sum over the 4 lanes of each aligned quad (quad_perm xor 1, then xor 2).
__device__ __forceinline__ float quad_sum(float x) {
    x += dpp_mov<0xB1>(x);
    x += dpp_mov<0x4E>(x);
    return x;
}

// Inclusive prefix sum over the 64 lanes of a wave: within each row of 16
// lanes by row_shr 1, 2, 4, 8, then across rows by row_bcast 15 and 31.
__device__ __forceinline__ float wave_scan(float x) {
    x += dpp_mov<0x111>(x);
    x += dpp_mov<0x112>(x);
    x += dpp_mov<0x114>(x);
    x += dpp_mov<0x118>(x);
    x += dpp_mov<0x142, 0xA>(x);
    x += dpp_mov<0x143, 0xC>(x);
    return x;
}

typedef float f32x8 __attribute__((ext_vector_type(8)));

// fp32 x8 -> hi/lo bf16 operand fragments.
__device__ __forceinline__ void split8(const f32x8& x, bf16x8& h, bf16x8& l) {
    uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
    split2(x[0], x[1], h0, l0);
    split2(x[2], x[3], h1, l1);
    split2(x[4], x[5], h2, l2);
    split2(x[6], x[7], h3, l3);
    h = __builtin_bit_cast(bf16x8, u32x4{h0, h1, h2, h3});
    l = __builtin_bit_cast(bf16x8, u32x4{l0, l1, l2, l3});
}

__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Two 8-byte LDS reads (4 bf16 each) joined into one operand fragment.
__device__ __forceinline__ bf16x8 ld2x4(const bf16_t* p0, const bf16_t* p1) {
    const uint2 a = *reinterpret_cast<const uint2*>(p0);
    const uint2 b = *reinterpret_cast<const uint2*>(p1);
    return __builtin_bit_cast(bf16x8, u32x4{a.x, a.y, b.x, b.y});
}

// Workgroup barrier that orders LDS only: outstanding global loads (the
// next chunk's prefetch) stay in flight across it.
//
// The scalar branch after it is never taken (no launch has 2^32 - 1
// workgroups; if one did, it would only run a no-op).  It ends the basic
// block at the barrier, so the compiler lays each loop out with its code on
// its own side of the barriers instead of rotating part of one period's
// work past them; measured on the scalar-gate chunk kernel (B8 H16 T4096,
// interleaved launches) that is ~11% faster, and neutral to slightly faster
// on the channel-gate one.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    if (blockIdx.x == 0xffffffffu) asm volatile("s_nop 0" ::: "memory");
}

}  // namespace gdr
