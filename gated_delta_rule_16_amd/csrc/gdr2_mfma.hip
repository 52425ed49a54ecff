// bf16-input path of gdr2_chunk_fwd: Gated Delta Rule-2 in chunks of 16
// tokens on gfx950 matrix cores, one fused pass over the sequence.
//
// The rule ("Gated DeltaNet-2", agihunt.info): per token, decay the state
// with the per-channel alpha_t on the key axis, read the old value along
// e_t = b_t (.) k_t, write the residual of w_t (.) v_t against that read
// along k_t.  The page states that in chunks the channel decay folds into an
// asymmetric rank-1 erase factor and the chunk is a triangular solve plus
// dense products.  With lambda_t = prod_{i<=t} alpha_i inside the chunk (per
// channel, elementwise) and lambda_C its value at the chunk's last token,
// unrolling the recurrence gives
//
//   A_sj  = sum_c e_sc k_jc lambda_sc / lambda_jc          j < s
//   P_rs  = sum_c q_rc k_sc lambda_rc / lambda_sc          s <= r
//   T     = (I + A)^{-1}
//   R_s   = w_s (.) v_s - S (e_s (.) lambda_s)
//   V_new = T R
//   o_r   = S (q_r (.) lambda_r) + sum_{s<=r} P_rs V_new_s
//   S    <- S diag(lambda_C) + sum_s V_new_s (k_s (.) lambda_C / lambda_s)^T
//         = (S + sum_s V_new_s (k_s / lambda_s)^T) diag(lambda_C)
//
// Chunks are 16 tokens so that one reference point (the chunk start) serves
// every decayed product: the row operands E = e (.) lambda and
// Q = q (.) lambda are <= 1 and shared by A, P, E S^T and Q S^T, and the
// column operand K' = k / lambda is shared by A, P and the state update.
// K' is bounded by 1 / lambda_C; a chunk where some channel decays below
// 2^-96 ("wide": K' could overflow) instead has A and P formed entry by
// entry from the log decays, and its update takes k (.) lambda_C / lambda.
//
// Work split: one workgroup per (b, h, 32 state rows), eight waves.
//   team A   waves 0, 1: wave a owns state rows 16 a .. 16 a + 15 as S^T
//            tiles in registers and walks the chunks in order: E S^T, R,
//            V_new = T R, Q S^T, o, the update.
//   team B   running ahead of it:
//            E0..E3 (waves 4..7), chunk c + 2: the elementwise pass --
//                 lambda by running products, 1 / lambda, the operands E, Q,
//                 K' as bf16 hi/lo pairs; wave 4 + j takes tokens 4j .. 4j+3
//                 (lane = channel pair) and forms the products of its
//                 prefix itself, so the waves never wait on each other;
//            AP-A (wave 2), chunk c + 1: A = E K'^T, T = (I + A)^{-1}, and
//                 the wide-chunk path;
//            AP-P (wave 3), chunk c + 1: P = Q K'^T, w (.) v.
// One workgroup barrier closes each period; LDS keeps three sets of the
// elementwise operands (chunk mod 3) and two of T, P, w (.) v (chunk mod 2).
//
// Products: v_mfma_f32_16x16x32_bf16 over the key dim, with the contraction
// order kappa (see kperm) that makes a pair of S^T accumulator tiles the B
// operand as they stand; v_mfma_f32_16x16x16_bf16 over tokens, whose C tile
// (rows 4 g + r, column m) is already the B operand of the next product.
// Every computed operand enters as a bf16 hi/lo pair (mfma_common.h).
#include <type_traits>

#include "launch.h"
#include "mfma_common.h"

namespace gdr {

namespace {

constexpr int CH = 16;            // tokens per chunk
constexpr int RB = 32;            // state rows per workgroup
constexpr int NA = RB / 16;       // team A waves
constexpr int NWAVE = NA + 6;
constexpr int P24 = 24;           // pitch of T, P (bf16) and w . v (fp32)
constexpr int PAF = 20;           // pitch of A (fp32)
constexpr float kLamMin = 1.2621774e-29f;   // 2^-96

struct Gdr2Params {
    int64_t T, H, BH;
    const bf16_t *q, *k, *v, *alpha, *erase, *write;
    const float* s0;
    void* o;
    float* s_final;
};

template <int DK>
struct Lay2 {
    static constexpr int PKN = DK + 16;            // K' row pitch (elements)
    // elementwise operands, chunk mod 3
    static constexpr int EH = 0;                    // E hi, lo [16][DK], operand order
    static constexpr int EL = EH + CH * DK * 2;
    static constexpr int QH = EL + CH * DK * 2;     // Q hi, lo [16][DK], operand order
    static constexpr int QL = QH + CH * DK * 2;
    static constexpr int KH = QL + CH * DK * 2;     // K' hi, lo [16][PKN], natural order
    static constexpr int KL = KH + CH * PKN * 2;
    static constexpr int LC = KL + CH * PKN * 2;    // lambda_C [DK] fp32, then the wide flag
    static constexpr int ESET = LC + DK * 4 + 16;
    // T, P, w . v, chunk mod 2
    static constexpr int TH = 0;                    // T hi, lo [16][P24]
    static constexpr int TL = TH + CH * P24 * 2;
    static constexpr int PH = TL + CH * P24 * 2;    // P hi, lo [16][P24]
    static constexpr int PL = PH + CH * P24 * 2;
    static constexpr int WV = PL + CH * P24 * 2;    // w . v [RB][P24] fp32, by state row
    static constexpr int TSET = WV + RB * P24 * 4;
    static constexpr int ER = 0;
    static constexpr int TR = ER + 3 * ESET;
    static constexpr int AF = TR + 2 * TSET;        // A fp32 [16][PAF] (AP-A)
    static constexpr int FG = AF + CH * PAF * 4;    // wide path: G fp32 [16][DK]
    static constexpr int FK = FG + CH * DK * 4;     //   k, b, q bf16 [16][DK]
    static constexpr int FB = FK + CH * DK * 2;
    static constexpr int FQ = FB + CH * DK * 2;
    static constexpr int TOTAL = FQ + CH * DK * 2;
    static_assert(ESET % 16 == 0 && TSET % 16 == 0 && KH % 16 == 0 && KL % 16 == 0, "alignment");
};

// Operand order of a contraction over 32 key channels: channel 16 h + 4 q + e
// of each block of 32 (h < 2, q < 4, e < 4) is stored at 8 q + 4 h + e, so
// the 8 values lane group q feeds an MFMA in kappa order are one 16-byte read.
__device__ __forceinline__ int kperm(int c) {
    return (c & ~31) | ((c & 12) << 1) | ((c & 16) >> 2) | (c & 3);
}

// Element offset of (row, stored column pc) in an operand-order tile:
// 16-byte unit u of row r is stored at u ^ (r mod DK / 8), so the 16 rows
// one lane group reads at one unit fall on distinct banks.
template <int DK>
__device__ __forceinline__ int kq_at(int row, int pc) {
    return row * DK + ((((pc >> 3) ^ (row & (DK / 8 - 1)))) << 3) + (pc & 7);
}

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ f32x4 mfma16k(const s16x4& a, const s16x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void split4(const f32x4& x, s16x4& h, s16x4& l) {
    uint32_t h0, h1, l0, l1;
    split2(x[0], x[1], h0, l0);
    split2(x[2], x[3], h1, l1);
    h = __builtin_bit_cast(s16x4, uint2{h0, h1});
    l = __builtin_bit_cast(s16x4, uint2{l0, l1});
}

__device__ __forceinline__ float lo_bf(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_bf(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

template <int DK, int DV, typename TOut>
__global__ __launch_bounds__(64 * NWAVE) void gdr2_bf16_kernel(Gdr2Params p) {
    using L = Lay2<DK>;
    constexpr int KJ = DK / 32;   // 32-deep contraction steps over the key dim
    constexpr int NS = DK / 16;   // S^T tiles per team A wave
    constexpr int NRB = DV / RB;
    static_assert(L::TOTAL <= 160 * 1024, "LDS budget");

    extern __shared__ __align__(16) unsigned char smem[];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int g = lane >> 4;
    const int m = lane & 15;

    // Workgroups are dealt to the 8 XCDs round-robin (blockIdx.x % 8); the
    // NRB row blocks of one head take the same XCD so that its key-side
    // tiles are read from HBM once and then hit that XCD's L2.
    const int64_t slot = blockIdx.x >> 3;
    const int64_t bh = (slot / NRB) * 8 + (blockIdx.x & 7);
    const int rbk = (int)(slot % NRB);
    if (bh >= p.BH) return;
    const int64_t H = p.H, T = p.T;
    const int64_t h = bh % H;
    const int64_t b = bh / H;
    const int row0 = rbk * RB;
    const int64_t nch = (T + CH - 1) / CH;

    auto eset = [&](int64_t c) { return smem + L::ER + (int)(c % 3) * L::ESET; };
    auto tset = [&](int64_t c) { return smem + L::TR + (int)(c & 1) * L::TSET; };
    auto bfp = [&](unsigned char* base, int off) { return reinterpret_cast<bf16_t*>(base + off); };
    auto wide_flag = [&](unsigned char* es) {
        return __builtin_amdgcn_readfirstlane(*reinterpret_cast<const int*>(es + L::LC + DK * 4));
    };

    const int64_t tstride = H * DK;   // elements between tokens of q, k, alpha, erase
    const int64_t kofs = (b * T * H + h) * DK;
    const int64_t vofs = (b * T * H + h) * DV + row0;

    if (wave < NA) {
        // =========================== team A ================================
        const int a = wave;
        const int i = 16 * a + m;   // state row (within the block) of this lane
        // sa[t][r] = S[i][16 t + 4 g + r]
        f32x4 sa[NS];
#pragma unroll
        for (int t = 0; t < NS; ++t) {
            sa[t] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (p.s0)
                sa[t] = *reinterpret_cast<const f32x4*>(p.s0 + ((bh * DV + row0 + i) * DK + 16 * t +
                                                                4 * g));
        }
        bf16x8 sh[KJ], sl[KJ];
#pragma unroll
        for (int j = 0; j < KJ; ++j)
            split8(f32x8{sa[2 * j][0], sa[2 * j][1], sa[2 * j][2], sa[2 * j][3], sa[2 * j + 1][0],
                         sa[2 * j + 1][1], sa[2 * j + 1][2], sa[2 * j + 1][3]},
                   sh[j], sl[j]);
        lds_barrier();
        lds_barrier();
        // o[t0 + 4 g + r][row0 + i] by buffer stores from a per-chunk
        // resource ending at the sequence end (stores past it are dropped)
        uint32_t ooff[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
            ooff[r] = (uint32_t)(((4 * g + r) * (int)(H * DV) + row0 + i) * (int)sizeof(TOut));
        TOut* obase = reinterpret_cast<TOut*>(p.o) + (b * T * H + h) * DV;
        for (int64_t c = 0; c < nch; ++c) {
            unsigned char* es = eset(c);
            unsigned char* ts = tset(c);
            const bf16_t* Eh = bfp(es, L::EH);
            const bf16_t* El = bfp(es, L::EL);
            const bf16_t* Qh = bfp(es, L::QH);
            const bf16_t* Ql = bfp(es, L::QL);
            const bf16_t* Kh = bfp(es, L::KH);
            const bf16_t* Kl = bfp(es, L::KL);
            const float* lc = reinterpret_cast<const float*>(es + L::LC);
            const int wide = wide_flag(es);

            // ---- E S^T (state chain) ---------------------------------------
            bf16x8 eh[KJ], el[KJ];
#pragma unroll
            for (int j = 0; j < KJ; ++j) {
                eh[j] = *reinterpret_cast<const bf16x8*>(Eh + kq_at<DK>(m, 32 * j + 8 * g));
                el[j] = *reinterpret_cast<const bf16x8*>(El + kq_at<DK>(m, 32 * j + 8 * g));
            }
            f32x4 k3[3] = {};
#pragma unroll
            for (int j = 0; j < KJ; ++j) {
                k3[0] = mfma16(eh[j], sh[j], k3[0]);
                k3[1] = mfma16(eh[j], sl[j], k3[1]);
                k3[2] = mfma16(el[j], sh[j], k3[2]);
            }
            const f32x4 wv = *reinterpret_cast<const f32x4*>(
                reinterpret_cast<const float*>(ts + L::WV) + i * P24 + 4 * g);
            const s16x4 th = *reinterpret_cast<const s16x4*>(bfp(ts, L::TH) + m * P24 + 4 * g);
            const s16x4 tl = *reinterpret_cast<const s16x4*>(bfp(ts, L::TL) + m * P24 + 4 * g);
            bf16x8 qh[KJ], ql[KJ];
#pragma unroll
            for (int j = 0; j < KJ; ++j) {
                qh[j] = *reinterpret_cast<const bf16x8*>(Qh + kq_at<DK>(m, 32 * j + 8 * g));
                ql[j] = *reinterpret_cast<const bf16x8*>(Ql + kq_at<DK>(m, 32 * j + 8 * g));
            }
            __builtin_amdgcn_sched_barrier(0);

            // ---- R = w.v - E S^T, beside Q S^T -----------------------------
            f32x4 q3[3] = {};
#pragma unroll
            for (int j = 0; j < KJ; ++j) {
                q3[0] = mfma16(qh[j], sh[j], q3[0]);
                q3[1] = mfma16(qh[j], sl[j], q3[1]);
                q3[2] = mfma16(ql[j], sh[j], q3[2]);
            }
            const f32x4 rr = wv - (k3[0] + k3[1] + k3[2]);
            s16x4 rh, rl;
            split4(rr, rh, rl);
            __builtin_amdgcn_sched_barrier(0);

            // ---- V_new = T R (state chain) ---------------------------------
            f32x4 v3[3];
            v3[0] = mfma16k(th, rh, f32x4{0.f, 0.f, 0.f, 0.f});
            v3[1] = mfma16k(th, rl, f32x4{0.f, 0.f, 0.f, 0.f});
            v3[2] = mfma16k(tl, rh, f32x4{0.f, 0.f, 0.f, 0.f});
            // K'^T[16 t + m][4 g + e] by transposed reads, lambda_C, P
            s16x4 kth[NS], ktl[NS];
#pragma unroll
            for (int t = 0; t < NS; ++t) {
                const int at = (4 * g + (m >> 2)) * L::PKN + 16 * t + 4 * (m & 3);
                kth[t] = lds_tr16(Kh + at);
                ktl[t] = lds_tr16(Kl + at);
            }
            f32x4 lam[NS];
#pragma unroll
            for (int t = 0; t < NS; ++t) lam[t] = *reinterpret_cast<const f32x4*>(lc + 16 * t + 4 * g);
            const s16x4 ph = *reinterpret_cast<const s16x4*>(bfp(ts, L::PH) + m * P24 + 4 * g);
            const s16x4 pl = *reinterpret_cast<const s16x4*>(bfp(ts, L::PL) + m * P24 + 4 * g);
            const f32x4 vn = v3[0] + v3[1] + v3[2];
            s16x4 nh, nl;
            split4(vn, nh, nl);
            __builtin_amdgcn_sched_barrier(0);

            // ---- o = Q S^T + P V_new -------------------------------------
            f32x4 o = q3[0] + q3[1] + q3[2];
            o = mfma16k(ph, nh, o);
            o = mfma16k(ph, nl, o);
            o = mfma16k(pl, nh, o);

            // ---- S^T <- (S^T + K'^T V_new) lambda_C --------------------------
            if (wide) {
#pragma unroll
                for (int t = 0; t < NS; ++t) sa[t] *= lam[t];
            }
#pragma unroll
            for (int t = 0; t < NS; ++t) {
                sa[t] = mfma16k(kth[t], nh, sa[t]);
                sa[t] = mfma16k(kth[t], nl, sa[t]);
                sa[t] = mfma16k(ktl[t], nh, sa[t]);
            }
            if (!wide) {
#pragma unroll
                for (int t = 0; t < NS; ++t) sa[t] *= lam[t];
            }
#pragma unroll
            for (int j = 0; j < KJ; ++j)
                split8(f32x8{sa[2 * j][0], sa[2 * j][1], sa[2 * j][2], sa[2 * j][3],
                             sa[2 * j + 1][0], sa[2 * j + 1][1], sa[2 * j + 1][2],
                             sa[2 * j + 1][3]},
                       sh[j], sl[j]);
            {
                const int64_t t0 = c * CH;
                const int n = (int)min((int64_t)CH, T - t0);
                const __amdgpu_buffer_rsrc_t ores = __builtin_amdgcn_make_buffer_rsrc(
                    obase + t0 * H * DV, (short)0, n * (int)(H * DV * sizeof(TOut)), 0x00020000);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    if constexpr (sizeof(TOut) == 4)
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o[r]), ores,
                                                              (int)ooff[r], 0, 0);
                    else
                        __builtin_amdgcn_raw_buffer_store_b16(f2bf(o[r]), ores, (int)ooff[r], 0, 0);
                }
            }
            lds_barrier();
        }
        if (p.s_final) {
#pragma unroll
            for (int t = 0; t < NS; ++t)
                *reinterpret_cast<f32x4*>(p.s_final + ((bh * DV + row0 + i) * DK + 16 * t + 4 * g)) =
                    sa[t];
        }
        return;
    }

    // ============================== team B =================================
    // Global loads: a uniform chunk base plus a 32-bit lane offset.  Rows
    // past the end of the sequence repeat its last token and are masked in
    // the arithmetic (alpha = 1, erase = write = 0).
    auto last_row = [&](int64_t cn) { return (int)min((int64_t)CH - 1, T - 1 - cn * CH); };
    auto n_live = [&](int64_t cn) { return (int)min((int64_t)CH, T - cn * CH); };

    // A role prepares chunk x in period x - lead (periods run from -2 to
    // nch - 1, each closed by the workgroup barrier).  Loading roles keep two
    // chunks in flight in three register buffers; loads are unconditional
    // (an index past the end repeats the last chunk) so that the wait before
    // each prepare covers just its buffer.
    auto run = [&](int lead, auto&& load, auto&& prepare, auto& fa, auto& fb, auto& fc) {
        for (int e = 0; e < 2 - lead; ++e) lds_barrier();
        load(0, fa);
        load(min((int64_t)1, nch - 1), fb);
        for (int64_t x = 0; x < nch; x += 3) {
            load(min(x + 2, nch - 1), fc);
            prepare(x, fa);
            lds_barrier();
            load(min(x + 3, nch - 1), fa);
            if (x + 1 < nch) {
                prepare(x + 1, fb);
                lds_barrier();
            }
            load(min(x + 4, nch - 1), fb);
            if (x + 2 < nch) {
                prepare(x + 2, fc);
                lds_barrier();
            }
        }
        for (int e = 0; e < lead; ++e) lds_barrier();
    };
    auto run_noload = [&](int lead, auto&& prepare) {
        for (int e = 0; e < 2 - lead; ++e) lds_barrier();
        for (int64_t x = 0; x < nch; ++x) {
            prepare(x);
            lds_barrier();
        }
        for (int e = 0; e < lead; ++e) lds_barrier();
    };
    const int cp = lane % (DK / 2);   // channel pair of the lane in the key-side passes

    // C[4 g + r][m] = sum_c X[m][c] K'[4 g + r][c] for X = E or Q (operand
    // order): lane (g, m) gets row m, columns 4 g .. 4 g + 3 of X K'^T.
    auto xk_product = [&](const bf16_t* Xh, const bf16_t* Xl, const bf16_t* Kh, const bf16_t* Kl) {
        f32x4 acc[3] = {};
#pragma unroll
        for (int j = 0; j < KJ; ++j) {
            const bf16x8 xh = *reinterpret_cast<const bf16x8*>(Xh + kq_at<DK>(m, 32 * j + 8 * g));
            const bf16x8 xl = *reinterpret_cast<const bf16x8*>(Xl + kq_at<DK>(m, 32 * j + 8 * g));
            const int at = m * L::PKN + 32 * j + 4 * g;
            const bf16x8 kh = ld2x4(Kh + at, Kh + at + 16);
            const bf16x8 kl = ld2x4(Kl + at, Kl + at + 16);
            acc[0] = mfma16(kh, xh, acc[0]);
            acc[1] = mfma16(kh, xl, acc[1]);
            acc[2] = mfma16(kl, xh, acc[2]);
        }
        return acc[0] + acc[1] + acc[2];
    };

    if (wave == NA) {
        // ------------------- AP-A: A, T = (I + A)^{-1} -----------------------
        float* Af = reinterpret_cast<float*>(smem + L::AF);
        // Wide chunk: A and P entry by entry from the log decays G (within
        // the chunk, per channel), and the update operand
        // k (.) lambda_C / lambda = k (.) e^{G_C - G} in place of K'.
        auto wide_chunk = [&](int64_t cn, unsigned char* es, unsigned char* ts) {
            float* Gf = reinterpret_cast<float*>(smem + L::FG);
            bf16_t* Fk = bfp(smem, L::FK);
            bf16_t* Fb = bfp(smem, L::FB);
            bf16_t* Fq = bfp(smem, L::FQ);
            const int n = n_live(cn), last = last_row(cn);
            const int64_t base = kofs + cn * CH * tstride + 2 * cp;
            float g0[CH], g1[CH];
            uint32_t kk[CH];
            float acc0 = 0.f, acc1 = 0.f;
#pragma unroll
            for (int t = 0; t < CH; ++t) {
                const int64_t at = base + min(t, last) * tstride;
                const uint32_t ua = *reinterpret_cast<const uint32_t*>(p.alpha + at);
                const uint32_t ub = *reinterpret_cast<const uint32_t*>(p.erase + at);
                const uint32_t uq = *reinterpret_cast<const uint32_t*>(p.q + at);
                kk[t] = *reinterpret_cast<const uint32_t*>(p.k + at);
                const bool live = t < n;
                acc0 += live ? safe_log(lo_bf(ua)) : 0.f;
                acc1 += live ? safe_log(hi_bf(ua)) : 0.f;
                g0[t] = acc0;
                g1[t] = acc1;
                *reinterpret_cast<float2*>(Gf + t * DK + 2 * cp) = float2{acc0, acc1};
                *reinterpret_cast<uint32_t*>(Fk + t * DK + 2 * cp) = kk[t];
                *reinterpret_cast<uint32_t*>(Fb + t * DK + 2 * cp) = live ? ub : 0u;
                *reinterpret_cast<uint32_t*>(Fq + t * DK + 2 * cp) = uq;
            }
            bf16_t* Kh = bfp(es, L::KH);
            bf16_t* Kl = bfp(es, L::KL);
#pragma unroll
            for (int t = 0; t < CH; ++t) {
                uint32_t xh, xl;
                split2(lo_bf(kk[t]) * __expf(g0[CH - 1] - g0[t]),
                       hi_bf(kk[t]) * __expf(g1[CH - 1] - g1[t]), xh, xl);
                *reinterpret_cast<uint32_t*>(Kh + t * L::PKN + 2 * cp) = xh;
                *reinterpret_cast<uint32_t*>(Kl + t * L::PKN + 2 * cp) = xl;
            }
            wave_lds_sync();
            bf16_t* Ph = bfp(ts, L::PH);
            bf16_t* Pl = bfp(ts, L::PL);
            // all 256 (r, s) pairs: s <= r are formed, the rest are zero
            for (int e = lane; e < CH * CH; e += 64) {
                const int r = e >> 4, s = e & 15;
                float av = 0.f, pv = 0.f;
                if (s <= r) {
                    for (int c = 0; c < DK; ++c) {
                        const float d = __expf(Gf[r * DK + c] - Gf[s * DK + c]);
                        const float ks = bf2f(Fk[s * DK + c]) * d;
                        pv += bf2f(Fq[r * DK + c]) * ks;
                        av += bf2f(Fb[r * DK + c]) * bf2f(Fk[r * DK + c]) * ks;
                    }
                }
                Af[r * PAF + s] = s < r ? av : 0.f;
                bf16_t xh, xl;
                split_bf16(pv, xh, xl);
                Ph[r * P24 + s] = xh;
                Pl[r * P24 + s] = xl;
            }
        };
        auto prepare = [&](int64_t cn) {
            unsigned char* es = eset(cn);
            unsigned char* ts = tset(cn);
            if (wide_flag(es)) {
                wide_chunk(cn, es, ts);
            } else {
                // C[4 g + r][m] = A[m][4 g + r]; kept for 4 g + r < m
                const f32x4 acc = xk_product(bfp(es, L::EH), bfp(es, L::EL), bfp(es, L::KH),
                                             bfp(es, L::KL));
                f32x4 av;
#pragma unroll
                for (int r = 0; r < 4; ++r) av[r] = 4 * g + r < m ? acc[r] : 0.f;
                *reinterpret_cast<f32x4*>(Af + m * PAF + 4 * g) = av;
            }
            wave_lds_sync();
            // X = (I + A)^{-1}: lane pair (rr, half) builds row rr from
            // X = I - X A, columns right to left, pushing each finished entry
            // into the columns left of it; A's strictly lower part is read
            // into registers first so the 16 dependent steps wait on nothing.
            const int rr = (lane >> 1) & 15, half = lane & 1;
            f32x4 lrow[CH][4];
#pragma unroll
            for (int q = 1; q < CH; ++q)
#pragma unroll
                for (int q4 = 0; q4 < (q + 3) / 4; ++q4)
                    lrow[q][q4] = *reinterpret_cast<const f32x4*>(Af + q * PAF + 4 * q4);
            __builtin_amdgcn_sched_barrier(0);
            float acc2[CH], x[CH];
#pragma unroll
            for (int cc = 0; cc < CH; ++cc) acc2[cc] = 0.f;
#pragma unroll
            for (int q = CH - 1; q >= 0; --q) {
                x[q] = (rr == q ? 1.f : 0.f) - acc2[q];
#pragma unroll
                for (int q4 = 0; q4 < (q + 3) / 4; ++q4)
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (4 * q4 + e < q) acc2[4 * q4 + e] += x[q] * lrow[q][q4][e];
            }
            // columns 8 half .. 8 half + 7 of row rr (bitwise select: a
            // conditional here becomes an indexed private array)
            const uint32_t msk = half ? 0xffffffffu : 0u;
            float xs[8];
#pragma unroll
            for (int e = 0; e < 8; ++e)
                xs[e] = __uint_as_float((__float_as_uint(x[8 + e]) & msk) |
                                        (__float_as_uint(x[e]) & ~msk));
            bf16x8 xh, xl;
            split8(f32x8{xs[0], xs[1], xs[2], xs[3], xs[4], xs[5], xs[6], xs[7]}, xh, xl);
            if (lane < 32) {
                *reinterpret_cast<bf16x8*>(bfp(ts, L::TH) + rr * P24 + 8 * half) = xh;
                *reinterpret_cast<bf16x8*>(bfp(ts, L::TL) + rr * P24 + 8 * half) = xl;
            }
        };
        run_noload(1, prepare);
    } else if (wave == NA + 1) {
        // ------------------------ AP-P: P, w . v ----------------------------
        // lane: token t = lane / 4, state rows 8 (lane % 4) .. + 7
        struct Buf {
            u32x4 v, w;
        };
        const int wt = lane >> 2, wr = 8 * (lane & 3);
        auto load = [&](int64_t cn, Buf& f) {
            const uint32_t off = (uint32_t)(min(wt, last_row(cn)) * (int)(H * DV) + wr) * 2u;
            const char* vb = reinterpret_cast<const char*>(p.v + vofs + cn * CH * H * DV);
            const char* wb = reinterpret_cast<const char*>(p.write + vofs + cn * CH * H * DV);
            f.v = *reinterpret_cast<const u32x4*>(vb + off);
            f.w = *reinterpret_cast<const u32x4*>(wb + off);
        };
        auto prepare = [&](int64_t cn, const Buf& f) {
            unsigned char* es = eset(cn);
            unsigned char* ts = tset(cn);
            if (!wide_flag(es)) {
                // C[4 g + r][m] = P[m][4 g + r]; kept for 4 g + r <= m
                const f32x4 acc = xk_product(bfp(es, L::QH), bfp(es, L::QL), bfp(es, L::KH),
                                             bfp(es, L::KL));
                f32x4 pv;
#pragma unroll
                for (int r = 0; r < 4; ++r) pv[r] = 4 * g + r <= m ? acc[r] : 0.f;
                s16x4 xh, xl;
                split4(pv, xh, xl);
                *reinterpret_cast<s16x4*>(bfp(ts, L::PH) + m * P24 + 4 * g) = xh;
                *reinterpret_cast<s16x4*>(bfp(ts, L::PL) + m * P24 + 4 * g) = xl;
            }
            const bool live = wt < n_live(cn);
            float* wv = reinterpret_cast<float*>(ts + L::WV);
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                wv[(wr + 2 * x) * P24 + wt] = live ? lo_bf(f.w[x]) * lo_bf(f.v[x]) : 0.f;
                wv[(wr + 2 * x + 1) * P24 + wt] = live ? hi_bf(f.w[x]) * hi_bf(f.v[x]) : 0.f;
            }
        };
        Buf fa, fb, fc;
        run(1, load, prepare, fa, fb, fc);
    } else {
        // ------------- E0..E3: lambda, 1 / lambda, E, Q, K' (hi/lo) ----------
        const int ej = wave - NA - 2;
        auto erole = [&](auto jc) {
            constexpr int J = decltype(jc)::value;
            constexpr int NPRE = 4 * J;    // rows before this wave's tokens
            struct Buf {
                uint32_t a[NPRE + 4];
                uint32_t k[4], b[4], q[4];
            };
            auto load = [&](int64_t cn, Buf& f) {
                const int last = last_row(cn);
                const int64_t cb = kofs + cn * CH * tstride;
                const bf16_t* ab = p.alpha + cb;
                const bf16_t* kb = p.k + cb;
                const bf16_t* bb = p.erase + cb;
                const bf16_t* qb = p.q + cb;
#pragma unroll
                for (int t = 0; t < NPRE + 4; ++t) {
                    const uint32_t off = (uint32_t)(min(t, last) * (int)tstride + 2 * cp);
                    f.a[t] = *reinterpret_cast<const uint32_t*>(ab + off);
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const uint32_t off = (uint32_t)(min(NPRE + u, last) * (int)tstride + 2 * cp);
                    f.k[u] = *reinterpret_cast<const uint32_t*>(kb + off);
                    f.b[u] = *reinterpret_cast<const uint32_t*>(bb + off);
                    f.q[u] = *reinterpret_cast<const uint32_t*>(qb + off);
                }
            };
            const int pc = kperm(2 * cp);
            auto prepare = [&](int64_t cn, const Buf& f) {
                unsigned char* es = eset(cn);
                const int n = n_live(cn);
                float l0 = 1.f, l1 = 1.f;
#pragma unroll
                for (int t = 0; t < NPRE; ++t) {
                    const bool live = t < n;
                    l0 *= live ? lo_bf(f.a[t]) : 1.f;
                    l1 *= live ? hi_bf(f.a[t]) : 1.f;
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int t = NPRE + u;
                    const bool live = t < n;
                    l0 *= live ? lo_bf(f.a[t]) : 1.f;
                    l1 *= live ? hi_bf(f.a[t]) : 1.f;
                    const float r0 = __builtin_amdgcn_rcpf(l0), r1 = __builtin_amdgcn_rcpf(l1);
                    const float k0 = lo_bf(f.k[u]), k1 = hi_bf(f.k[u]);
                    const float e0 = live ? lo_bf(f.b[u]) * k0 : 0.f;
                    const float e1 = live ? hi_bf(f.b[u]) * k1 : 0.f;
                    uint32_t xh, xl;
                    const int ot = kq_at<DK>(t, pc);
                    split2(e0 * l0, e1 * l1, xh, xl);
                    *reinterpret_cast<uint32_t*>(bfp(es, L::EH) + ot) = xh;
                    *reinterpret_cast<uint32_t*>(bfp(es, L::EL) + ot) = xl;
                    split2(lo_bf(f.q[u]) * l0, hi_bf(f.q[u]) * l1, xh, xl);
                    *reinterpret_cast<uint32_t*>(bfp(es, L::QH) + ot) = xh;
                    *reinterpret_cast<uint32_t*>(bfp(es, L::QL) + ot) = xl;
                    split2(k0 * r0, k1 * r1, xh, xl);
                    *reinterpret_cast<uint32_t*>(bfp(es, L::KH) + t * L::PKN + 2 * cp) = xh;
                    *reinterpret_cast<uint32_t*>(bfp(es, L::KL) + t * L::PKN + 2 * cp) = xl;
                }
                if constexpr (J == 3) {
                    float* lc = reinterpret_cast<float*>(es + L::LC);
                    *reinterpret_cast<float2*>(lc + 2 * cp) = float2{l0, l1};
                    const bool w = !(l0 >= kLamMin && l1 >= kLamMin);
                    const uint64_t any = __builtin_amdgcn_ballot_w64(w);
                    if (lane == 0) *reinterpret_cast<int*>(lc + DK) = any != 0 ? 1 : 0;
                }
            };
            Buf fa, fb, fc;
            run(2, load, prepare, fa, fb, fc);
        };
        if (ej == 0) erole(std::integral_constant<int, 0>{});
        else if (ej == 1) erole(std::integral_constant<int, 1>{});
        else if (ej == 2) erole(std::integral_constant<int, 2>{});
        else erole(std::integral_constant<int, 3>{});
    }
}

template <int DK, int DV, typename TOut>
hipError_t launch_t(const ChunkArgs& a) {
    Gdr2Params p;
    p.T = a.T;
    p.H = a.H;
    p.BH = a.B * a.H;
    p.q = (const bf16_t*)a.q;
    p.k = (const bf16_t*)a.k;
    p.v = (const bf16_t*)a.v;
    p.alpha = (const bf16_t*)a.alpha;
    p.erase = (const bf16_t*)a.erase;
    p.write = (const bf16_t*)a.write;
    p.s0 = a.s0;
    p.o = a.o;
    p.s_final = a.s_final;
    const size_t lds = Lay2<DK>::TOTAL;
    auto fn = gdr2_bf16_kernel<DK, DV, TOut>;
    hipError_t e =
        hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    // 8 * ceil(B*H / 8) heads' worth of row blocks; surplus workgroups exit
    const unsigned grid = (unsigned)(((a.B * a.H + 7) / 8) * 8 * (DV / RB));
    hipLaunchKernelGGL(fn, dim3(grid), dim3(64 * NWAVE), lds, a.stream, p);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_d(const ChunkArgs& a) {
    return a.out_bf16 ? launch_t<DK, DV, bf16_t>(a) : launch_t<DK, DV, float>(a);
}

}  // namespace

hipError_t launch_gdr2_bf16(const ChunkArgs& a) {
    if (a.Dk == 128 && a.Dv == 128) return launch_d<128, 128>(a);
    if (a.Dk == 128 && a.Dv == 64) return launch_d<128, 64>(a);
    if (a.Dk == 64 && a.Dv == 128) return launch_d<64, 128>(a);
    return launch_d<64, 64>(a);
}

}  // namespace gdr
