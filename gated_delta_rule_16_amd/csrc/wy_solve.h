// T = (I + A)^{-1} for a 64x64 strictly lower-triangular fp32 A in LDS:
// the UT transform's triangular inverse, shared by the chunked kernels.
//
// Blocked in 16x16 blocks (A_ij, T_ij with i, j = 0..3):
//   T_ii = (I + A_ii)^{-1}                  forward substitution, one wave
//                                           per block, 4 lanes per column
//   T_10 = -T_11 A_10 T_00, T_32 = -T_33 A_32 T_22
//   [T_20 T_21; T_30 T_31] = -T_22' (A_21' T_11')   with the 32x32 blocks
//                                           T_11' = [T_00 0; T_10 T_11] etc.
// The products run on fp32 16x16x4 matrix cores (exact fp32 operands).
// Every workgroup thread must call it (it contains workgroup barriers).
// Inputs: Af [64][PF] (only blocks on/below the diagonal are read).
// Outputs: T as bf16 hi/lo in Th, Tl [64][P72] for every block on or below
// the diagonal; Tf [64][PF] is fp32 scratch; X holds 4 16x16 fp32 tiles.
#pragma once

#include "mfma_common.h"

namespace gdr {

constexpr int PF = 68;    // pitch (floats) of 64-wide fp32 tiles
constexpr int PX = 17;    // pitch (floats) of 16x16 scratch tiles
constexpr int P72 = 72;   // pitch (elements) of 64-wide bf16 tiles

// Store one fp32 16x16 tile held in the C layout of the 16x16x4 matrix core
// (register r: row 4 (lane / 16) + r, column lane % 16) into T's fp32 copy
// and its hi/lo bf16 copies, at block (R, C).
__device__ __forceinline__ void store_t_block(float* Tf, bf16_t* Th, bf16_t* Tl, const f32x4& t,
                                              int R, int C, bool keep_f32) {
    const int lane = threadIdx.x & 63;
    const int m = lane & 15, kq = lane >> 4;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int row = 16 * R + 4 * kq + r, col = 16 * C + m;
        if (keep_f32) Tf[row * PF + col] = t[r];
        bf16_t h, l;
        split_bf16(t[r], h, l);
        Th[row * P72 + col] = h;
        Tl[row * P72 + col] = l;
    }
}

__device__ __forceinline__ void solve_unit_lower_64(const float* Af, float* Tf, float* Xs,
                                                    bf16_t* Th, bf16_t* Tl) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int m16 = lane & 15;
    const int kq = lane >> 4;
    {
        // Diagonal block `wave`: lane 4c + q works on column c, summing
        // the rows s = q (mod 4): T_rc = delta_rc - sum_{s<r} A_rs T_sc.
        const int q = lane & 3, cidx = lane >> 2, base = 16 * wave;
        float a[16][4];
#pragma unroll
        for (int r = 1; r < 16; ++r)
#pragma unroll
            for (int u = 0; u <= ((r - 1) >> 2); ++u)
                a[r][u] = Af[(base + r) * PF + base + 4 * u + q];
        float t[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) t[u] = (4 * u + q == cidx) ? 1.f : 0.f;
#pragma unroll
        for (int r = 1; r < 16; ++r) {
            float part = 0.f;
#pragma unroll
            for (int u = 0; u <= ((r - 1) >> 2); ++u) part += a[r][u] * t[u];
            const float val = (r == cidx ? 1.f : 0.f) - quad_sum(part);
            if (q == (r & 3)) t[r >> 2] = val;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int row = base + 4 * u + q, col = base + cidx;
            Tf[row * PF + col] = t[u];
            bf16_t th, tl;
            split_bf16(t[u], th, tl);
            Th[row * P72 + col] = th;
            Tl[row * P72 + col] = tl;
        }
    }
    lds_barrier();
    if (wave < 2) {
        // T_10 = -T_11 A_10 T_00 (wave 0) and T_32 = -T_33 A_32 T_22 (wave 1)
        const int R = 2 * wave + 1, C = 2 * wave;
        float* X = Xs + wave * 16 * PX;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            acc = mfma_f32(Af[(16 * R + m16) * PF + 16 * C + 4 * ks + kq],
                           Tf[(16 * C + 4 * ks + kq) * PF + 16 * C + m16], acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) X[(4 * kq + r) * PX + m16] = acc[r];
        __builtin_amdgcn_s_waitcnt(0xc07f);
        __builtin_amdgcn_wave_barrier();
        f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            t = mfma_f32(Tf[(16 * R + m16) * PF + 16 * R + 4 * ks + kq],
                         X[(4 * ks + kq) * PX + m16], t);
        store_t_block(Tf, Th, Tl, -t, R, C, true);
    }
    lds_barrier();
    // Lower 32x32 block: Y = A_21 T_11, then T_21 = -T_22 Y, one 16x16
    // output block per wave: block row 2 + (wave >> 1), column wave & 1.
    const int yi = 2 + (wave >> 1), yj = wave & 1;
    {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        // T_11 block column yj has nonzero blocks in rows yj .. 1
        for (int ks = 4 * yj; ks < 8; ++ks)
            acc = mfma_f32(Af[(16 * yi + m16) * PF + 4 * ks + kq],
                           Tf[(4 * ks + kq) * PF + 16 * yj + m16], acc);
        float* Y = Xs + wave * 16 * PX;
#pragma unroll
        for (int r = 0; r < 4; ++r) Y[(4 * kq + r) * PX + m16] = acc[r];
    }
    lds_barrier();
    {
        f32x4 t = {0.f, 0.f, 0.f, 0.f};
        // T_22 block row yi has nonzero blocks in columns 2 .. yi; Y's
        // block row 2 + k (column yj) was written by wave 2 k + yj.
        for (int ks = 0; ks < 4 * (yi - 1); ++ks) {
            const float* Y = Xs + (2 * (ks >> 2) + yj) * 16 * PX;
            t = mfma_f32(Tf[(16 * yi + m16) * PF + 32 + 4 * ks + kq],
                         Y[(4 * (ks & 3) + kq) * PX + m16], t);
        }
        store_t_block(Tf, Th, Tl, -t, yi, yj, false);
    }
    lds_barrier();

}

}  // namespace gdr
