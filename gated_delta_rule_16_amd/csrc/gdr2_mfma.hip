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
//            E0..E3 (waves 4..7), chunk c + 3: the elementwise pass --
//                 lambda by running products, 1 / lambda, the operands E, Q,
//                 K'; each wave takes 3 to 5 tokens (lane = channel pair) and
//                 forms the products of the rows before them itself, so the
//                 waves never wait on each other;
//            AP-A (wave 2): A = E K'^T for chunk c + 2 (or the wide-chunk
//                 path), T = (I + A)^{-1} for chunk c + 1;
//            AP-P (wave 3), chunk c + 1: P = Q K'^T, w (.) v.
// With GDR_L2NORM_QK (template flag NORM), rho_t = 1 / |k_t| and
// pi_t = 1 / |q_t| enter as per-token scalars only; E, Q and K' stay those
// of the raw q, k.  Carrying V~ = diag(rho) V_new in place of V_new (a
// similarity transform of the solve) puts every rho on a row:
//   A~_sj = rho_s^2 A_sj,   T~ = (I + A~)^{-1} = diag(rho) T diag(rho)^{-1},
//   R~_s  = rho_s (w (.) v)_s - rho_s^2 (S E^T)_s,   V~ = T~ R~,
//   P~_rs = pi_r P_rs,   o_r = pi_r (Q S^T)_r + sum_s P~_rs V~_s,
//   S    <- (S + K'^T V~) diag(lambda_C)
// (A, P, E, K' those of the raw q, k; the rho_j of A's columns and P's
// columns cancel against V~).  The E waves write per-lane partial sums of
// k^2 and q^2; AP-A reduces them when it forms A and stores rho^2, pi and
// rho with the chunk's elementwise set.
// One workgroup barrier closes each period; LDS keeps four sets of the
// elementwise operands (chunk mod 4) and two of A, T, P and w (.) v.
//
// Products: v_mfma_f32_16x16x32_bf16 throughout.  Over the key dim with the
// contraction order kappa (see kperm) that makes a pair of S^T accumulator
// tiles the B operand as they stand; over the 16 tokens with two 16-deep
// halves side by side (hi and lo terms, see cat44), the C tile (rows
// 4 g + r, column m) of one product being the B operand of the next.  A
// 16-deep leftover term takes the 32-deep instruction with a zero half
// rather than v_mfma_f32_16x16x16_bf16: an accumulator chained from one
// instruction into the other has been read before it was written (stale
// first registers) when the compiler left four wait states between them.
//
// Precision: computed operands enter as bf16 hi/lo pairs (mfma_common.h)
// where it matters.  P, P V_new, Q S^T and the update take three terms.
// E (in E S^T and A), A itself and T enter as single bf16 values: E S^T
// and A only shape R's correction and T, whose relative error the
// substitution does not amplify; a simulation of this chunk algorithm
// against the fp64 recurrence (1024 tokens; decays from fast to near 1,
// with and without an initial state) puts the error at <= 2.3e-3 (o) and
// <= 1.8e-3 (S) of rms, against 2e-4 with every operand split.  The
// FULL form splits those three too (E's lo half beside E S^T and A, K''s
// lo half in A, T's lo half in T R: four more products a chunk in team A,
// two in AP-A); the sequence-split backward takes its segment start states
// from it, since its gradients inherit the states' error.
#include <type_traits>

#include "launch.h"
#include "mfma_common.h"

namespace gdr {

namespace {

constexpr int CH = 16;            // tokens per chunk
constexpr int RB = 32;            // state rows per workgroup
constexpr int NA = RB / 16;       // team A waves
constexpr int NWAVE = NA + 6;
constexpr int DEPTH = 3;          // periods between the elementwise pass and team A
constexpr int P24 = 24;           // pitch of T, P (bf16) and w . v (fp32)
constexpr int PAF = 20;           // pitch of A and wide-path P (fp32)
constexpr float kLamMin = 1.2621774e-29f;   // 2^-96

struct Gdr2Params {
    int64_t T, H, BH;
    const bf16_t *q, *k, *v, *alpha, *erase, *write;
    const float* s0;
    void* o;
    float* s_final;
};

template <int DK, bool NORM, bool FULL = false>
struct Lay2 {
    static constexpr int PKN = DK + 16;            // K' row pitch (elements)
    // elementwise operands, chunk mod 4
    static constexpr int EH = 0;                    // E [16][DK] bf16, operand order
    static constexpr int QH = EH + CH * DK * 2;     // Q hi, lo [16][DK], operand order
    static constexpr int QL = QH + CH * DK * 2;
    static constexpr int KH = QL + CH * DK * 2;     // K' hi, lo [16][PKN], natural order
    static constexpr int KL = KH + CH * PKN * 2;
    static constexpr int LC = KL + CH * PKN * 2;    // lambda_C [DK] fp32, then the wide flag
    static constexpr int NR = LC + DK * 4 + 16;     // NORM: rho^2, pi, rho [16] fp32 each
    static constexpr int EL = NR + (NORM ? 3 * CH * 4 : 0);   // FULL: E lo [16][DK]
    static constexpr int ESET = EL + (FULL ? CH * DK * 2 : 0);
    // T, P, w . v, chunk mod 2
    static constexpr int TH = 0;                    // T [16][P24] bf16
    static constexpr int PH = TH + CH * P24 * 2;    // P hi, lo [16][P24]
    static constexpr int PL = PH + CH * P24 * 2;
    static constexpr int WV = PL + CH * P24 * 2;    // w . v [RB][P24] fp32, by state row
    static constexpr int TL = WV + RB * P24 * 4;    // FULL: T lo [16][P24]
    static constexpr int TSET = TL + (FULL ? CH * P24 * 2 : 0);
    static constexpr int ER = 0;
    static constexpr int TR = ER + 4 * ESET;
    static constexpr int AF = TR + 2 * TSET;        // A fp32 [16][PAF], chunk mod 2
    static constexpr int WP = AF + 2 * CH * PAF * 4;   // wide-path P fp32 [16][PAF], chunk mod 2
    static constexpr int FG = WP + 2 * CH * PAF * 4;   // wide path: G fp32 [16][DK]
    static constexpr int FK = FG + CH * DK * 4;     //   k, b, q bf16 [16][DK]
    static constexpr int FB = FK + CH * DK * 2;
    static constexpr int FQ = FB + CH * DK * 2;
    // NORM: per-lane partial sums (k^2, q^2) [16 tokens][64 lanes] fp32 x2,
    // chunk mod 2, 16-byte units swizzled by token (see ps_at)
    static constexpr int PS = FQ + CH * DK * 2;
    static constexpr int TOTAL = PS + (NORM ? 2 * CH * 64 * 8 : 0);
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

__device__ __forceinline__ void split4(const f32x4& x, s16x4& h, s16x4& l) {
    uint32_t h0, h1, l0, l1;
    split2(x[0], x[1], h0, l0);
    split2(x[2], x[3], h1, l1);
    h = __builtin_bit_cast(s16x4, uint2{h0, h1});
    l = __builtin_bit_cast(s16x4, uint2{l0, l1});
}

// Two 4-element operand halves as one 8-element operand.
__device__ __forceinline__ bf16x8 cat44(const s16x4& a, const s16x4& b) {
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ float lo_bf(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float hi_bf(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// NORM factors of a chunk in its elementwise set: rho^2, pi, rho by token.
enum { NR_RHO2 = 0, NR_PI = CH, NR_RHO = 2 * CH };

// Float offset of lane l's (k^2, q^2) partial pair for token t: 16-byte unit
// l / 2 of the token's row, XOR-swizzled by 4 (t mod 4) so that the reducing
// lanes (4 tokens x 4 unit phases per 16 lanes) read distinct banks.
__device__ __forceinline__ int ps_at(int t, int l) {
    return t * 128 + 4 * ((l >> 1) ^ (4 * (t & 3))) + 2 * (l & 1);
}

template <int DK, int DV, typename TOut, bool NORM, bool FULL = false>
__global__ __launch_bounds__(64 * NWAVE) void gdr2_bf16_kernel(Gdr2Params p) {
    using L = Lay2<DK, NORM, FULL>;
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

    auto eset = [&](int64_t c) { return smem + L::ER + (int)(c & 3) * L::ESET; };
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
        for (int e = 0; e < DEPTH; ++e) lds_barrier();
        // o[t0 + 4 g + r][row0 + i] by buffer stores from a per-chunk
        // resource ending at the sequence end (stores past it are dropped)
        uint32_t ooff[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
            ooff[r] = (uint32_t)(((4 * g + r) * (int)(H * DV) + row0 + i) * (int)sizeof(TOut));
        TOut* obase = reinterpret_cast<TOut*>(p.o) + (b * T * H + h) * DV;
        // E and Q fragments of the next chunk are read during this one (its
        // elementwise set is complete two periods ahead)
        bf16x8 eh[KJ], qh[KJ], ql[KJ], el[FULL ? KJ : 1];
        auto read_eq = [&](int64_t c) {
            unsigned char* es = eset(c);
#pragma unroll
            for (int j = 0; j < KJ; ++j) {
                const int at = kq_at<DK>(m, 32 * j + 8 * g);
                eh[j] = *reinterpret_cast<const bf16x8*>(bfp(es, L::EH) + at);
                qh[j] = *reinterpret_cast<const bf16x8*>(bfp(es, L::QH) + at);
                ql[j] = *reinterpret_cast<const bf16x8*>(bfp(es, L::QL) + at);
                if constexpr (FULL) el[j] = *reinterpret_cast<const bf16x8*>(bfp(es, L::EL) + at);
            }
        };
        read_eq(0);
        for (int64_t c = 0; c < nch; ++c) {
            unsigned char* es = eset(c);
            unsigned char* ts = tset(c);
            const bf16_t* Kh = bfp(es, L::KH);
            const bf16_t* Kl = bfp(es, L::KL);
            const float* lc = reinterpret_cast<const float*>(es + L::LC);
            const float* nrc = reinterpret_cast<const float*>(es + L::NR);
            const int wide = wide_flag(es);
            // operands written in the previous period; their reads overlap
            // the products below
            const f32x4 wv = *reinterpret_cast<const f32x4*>(
                reinterpret_cast<const float*>(ts + L::WV) + i * P24 + 4 * g);
            const s16x4 th = *reinterpret_cast<const s16x4*>(bfp(ts, L::TH) + m * P24 + 4 * g);
            s16x4 tl = {0, 0, 0, 0};
            if constexpr (FULL) tl = *reinterpret_cast<const s16x4*>(bfp(ts, L::TL) + m * P24 + 4 * g);
            const s16x4 ph = *reinterpret_cast<const s16x4*>(bfp(ts, L::PH) + m * P24 + 4 * g);
            const s16x4 pl = *reinterpret_cast<const s16x4*>(bfp(ts, L::PL) + m * P24 + 4 * g);
            // K'^T[16 t + m][4 g + e] by transposed reads; lambda_C
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
            __builtin_amdgcn_sched_barrier(0);

            // ---- S as hi/lo B operands, slab by slab beside E S^T, Q S^T -----
            f32x4 k2[3] = {}, q3[3] = {};
#pragma unroll
            for (int j = 0; j < KJ; ++j) {
                bf16x8 sh, sl;
                split8(f32x8{sa[2 * j][0], sa[2 * j][1], sa[2 * j][2], sa[2 * j][3],
                             sa[2 * j + 1][0], sa[2 * j + 1][1], sa[2 * j + 1][2],
                             sa[2 * j + 1][3]},
                       sh, sl);
                k2[0] = mfma16(eh[j], sh, k2[0]);
                k2[1] = mfma16(eh[j], sl, k2[1]);
                if constexpr (FULL) k2[2] = mfma16(el[j], sh, k2[2]);
                q3[0] = mfma16(qh[j], sh, q3[0]);
                q3[1] = mfma16(qh[j], sl, q3[1]);
                q3[2] = mfma16(ql[j], sh, q3[2]);
            }
#pragma unroll
            for (int j = 0; j < KJ; ++j) {
                __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);   // this slab's split
                __builtin_amdgcn_sched_group_barrier(0x008, FULL ? 6 : 5, 0);   // its products
            }
            __builtin_amdgcn_sched_barrier(0);

            // ---- R = w.v - E S^T;  V_new = [T | T] [R_hi; R_lo] ---------------
            //      (NORM: R~ = rho w.v - rho^2 E S^T, w.v already scaled)
            s16x4 rh, rl;
            const f32x4 es2 = FULL ? k2[0] + k2[1] + k2[2] : k2[0] + k2[1];
            if constexpr (NORM)
                split4(wv - *reinterpret_cast<const f32x4*>(nrc + NR_RHO2 + 4 * g) * es2, rh, rl);
            else
                split4(wv - es2, rh, rl);
            f32x4 vn = mfma16(cat44(th, th), cat44(rh, rl), f32x4{0.f, 0.f, 0.f, 0.f});
            if constexpr (FULL)
                vn = mfma16(cat44(tl, s16x4{0, 0, 0, 0}), cat44(rh, s16x4{0, 0, 0, 0}), vn);
            s16x4 nh, nl;
            split4(vn, nh, nl);
            const bf16x8 nn = cat44(nh, nh);
            const bf16x8 nz = cat44(nl, s16x4{0, 0, 0, 0});

            // ---- o = Q S^T + [P_hi | P_lo] [N_hi; N_hi] + [P_hi | P_lo] [N_lo; 0]
            f32x4 o = q3[0] + q3[1] + q3[2];
            if constexpr (NORM) o *= *reinterpret_cast<const f32x4*>(nrc + NR_PI + 4 * g);
            const bf16x8 pp = cat44(ph, pl);
            o = mfma16(pp, nn, o);
            o = mfma16(pp, nz, o);

            // ---- S^T <- (S^T + K'^T V_new) lambda_C --------------------------
            if (wide) {
#pragma unroll
                for (int t = 0; t < NS; ++t) sa[t] *= lam[t];
            }
#pragma unroll
            for (int t = 0; t < NS; ++t) {
                const bf16x8 kk = cat44(kth[t], ktl[t]);
                sa[t] = mfma16(kk, nn, sa[t]);
                sa[t] = mfma16(kk, nz, sa[t]);
            }
            if (!wide) {
#pragma unroll
                for (int t = 0; t < NS; ++t) sa[t] *= lam[t];
            }
            {
                // p.o NULL: no o (an empty range drops every store)
                const int64_t t0 = c * CH;
                const int n = p.o ? (int)min((int64_t)CH, T - t0) : 0;
                const __amdgpu_buffer_rsrc_t ores = __builtin_amdgcn_make_buffer_rsrc(
                    obase + t0 * H * DV, (short)0, n * (int)(H * DV * sizeof(TOut)), 0x00020000);
                if constexpr (sizeof(TOut) == 4) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o[r]), ores,
                                                              (int)ooff[r], 0, 0);
                } else {
                    store4_bf16(o, ores, ooff);
                }
            }
            read_eq(c + 1);
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
    // Global loads: a uniform row base plus a 32-bit lane offset.  Rows past
    // the end of the sequence repeat its last token and are masked in the
    // arithmetic (alpha = 1, erase = write = 0).
    auto last_row = [&](int64_t cn) { return (int)min((int64_t)CH - 1, T - 1 - cn * CH); };
    auto n_live = [&](int64_t cn) { return (int)min((int64_t)CH, T - cn * CH); };

    // A role prepares chunk x in period x - lead (periods run from -DEPTH to
    // nch - 1, each closed by the workgroup barrier).  Loading roles keep two
    // chunks in flight in three register buffers; loads are unconditional
    // (an index past the end repeats the last chunk) so that the wait before
    // each prepare covers just its buffer.
    auto run = [&](int lead, auto&& load, auto&& prepare, auto& fa, auto& fb, auto& fc) {
        for (int e = 0; e < DEPTH - lead; ++e) lds_barrier();
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
    const int cp = lane % (DK / 2);   // channel pair of the lane in the key-side passes

    if (wave == NA) {
        // ------------- AP-A: A for chunk p + 2, T for chunk p + 1 -------------
        // Wide chunk: A and P entry by entry from the log decays G (within
        // the chunk, per channel), and the update operand
        // k (.) lambda_C / lambda = k (.) e^{G_C - G} in place of K'.
        auto wide_chunk = [&](int64_t cn, unsigned char* es, float* Af, float* Wp) {
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
                if constexpr (NORM) {
                    const float* nr = reinterpret_cast<const float*>(es + L::NR);
                    av *= nr[NR_RHO2 + r];
                    pv *= nr[NR_PI + r];
                }
                Af[r * PAF + s] = s < r ? av : 0.f;
                Wp[r * PAF + s] = pv;
            }
        };
        const int rr = (lane >> 1) & 15, half = lane & 1;
        for (int64_t pp = -DEPTH; pp < nch; ++pp) {
            const int64_t x2 = pp + 2, x1 = pp + 1;
            if (x2 >= 0 && x2 < nch) {
                unsigned char* es = eset(x2);
                float* Af = reinterpret_cast<float*>(smem + L::AF + (int)(x2 & 1) * CH * PAF * 4);
                // NORM: lane (t, u) = (lane / 4, lane % 4) loads units u, u + 4,
                // ... of token t's partial sums first, so that the loads
                // overlap A's own reads and products
                f32x4 psv[NORM ? DK / 16 : 1];
                if constexpr (NORM) {
                    const float* ps = reinterpret_cast<const float*>(smem + L::PS) +
                                      (int)(x2 & 1) * CH * 128;
                    const int t = lane >> 2, u = lane & 3;
#pragma unroll
                    for (int e = 0; e < DK / 16; ++e)
                        psv[e] = *reinterpret_cast<const f32x4*>(
                            ps + t * 128 + 4 * ((4 * e + u) ^ (4 * (t & 3))));
                }
                // |k_t|^2, |q_t|^2 summed over the quad; rho^2, pi, rho of
                // token t stored with the chunk's set; returns rho_t^2
                auto reduce_norm = [&]() {
                    float sk = 0.f, sq = 0.f;
#pragma unroll
                    for (int e = 0; e < (NORM ? DK / 16 : 0); ++e) {
                        sk += psv[e][0] + psv[e][2];
                        sq += psv[e][1] + psv[e][3];
                    }
                    sk = quad_sum(sk);
                    sq = quad_sum(sq);
                    const float rho = l2_inv(sk);
                    const int t = lane >> 2;
                    if ((lane & 3) == 0) {
                        float* nr = reinterpret_cast<float*>(es + L::NR);
                        nr[NR_RHO2 + t] = rho * rho;
                        nr[NR_PI + t] = l2_inv(sq);
                        nr[NR_RHO + t] = rho;
                    }
                    return rho * rho;
                };
                if (wide_flag(es)) {
                    if constexpr (NORM) {
                        reduce_norm();
                        wave_lds_sync();   // the entry-by-entry path reads them back
                    }
                    float* Wp = reinterpret_cast<float*>(smem + L::WP + (int)(x2 & 1) * CH * PAF * 4);
                    wide_chunk(x2, es, Af, Wp);
                } else {
                    // C[4 g + r][m] = sum_c E[m][c] K'[4 g + r][c] = A[m][4 g + r];
                    // kept for 4 g + r < m
                    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int j = 0; j < KJ; ++j) {
                        const bf16x8 xh = *reinterpret_cast<const bf16x8*>(
                            bfp(es, L::EH) + kq_at<DK>(m, 32 * j + 8 * g));
                        const int at = m * L::PKN + 32 * j + 4 * g;
                        const bf16x8 kh = ld2x4(bfp(es, L::KH) + at, bfp(es, L::KH) + at + 16);
                        acc = mfma16(kh, xh, acc);
                        if constexpr (FULL) {
                            const bf16x8 xl = *reinterpret_cast<const bf16x8*>(
                                bfp(es, L::EL) + kq_at<DK>(m, 32 * j + 8 * g));
                            const bf16x8 kl = ld2x4(bfp(es, L::KL) + at, bfp(es, L::KL) + at + 16);
                            acc = mfma16(kl, xh, acc);
                            acc = mfma16(kh, xl, acc);
                        }
                    }
                    f32x4 av;
#pragma unroll
                    for (int r = 0; r < 4; ++r) av[r] = 4 * g + r < m ? acc[r] : 0.f;
                    // NORM: row m of A~ takes rho_m^2, held by lane 4 m
                    if constexpr (NORM) av *= __shfl(reduce_norm(), 4 * m, 64);
                    *reinterpret_cast<f32x4*>(Af + m * PAF + 4 * g) = av;
                }
            }
            if (x1 >= 0 && x1 < nch) {
                // X = (I + A)^{-1}: lane pair (rr, half) builds row rr from
                // X = I - X A, columns right to left, pushing each finished
                // entry into the columns left of it; A's strictly lower part
                // is read into registers first so the 16 dependent steps wait
                // on nothing.
                const float* Af = reinterpret_cast<const float*>(smem + L::AF + (int)(x1 & 1) * CH * PAF * 4);
                f32x4 lrow[CH][4];
#pragma unroll
                for (int q = 1; q < CH; ++q)
#pragma unroll
                    for (int q4 = 0; q4 < (q + 3) / 4; ++q4)
                        lrow[q][q4] = *reinterpret_cast<const f32x4*>(Af + q * PAF + 4 * q4);
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
                if constexpr (FULL) {
                    uint32_t h[4], l[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) split2(xs[2 * e], xs[2 * e + 1], h[e], l[e]);
                    if (lane < 32) {
                        *reinterpret_cast<u32x4*>(bfp(tset(x1), L::TH) + rr * P24 + 8 * half) =
                            u32x4{h[0], h[1], h[2], h[3]};
                        *reinterpret_cast<u32x4*>(bfp(tset(x1), L::TL) + rr * P24 + 8 * half) =
                            u32x4{l[0], l[1], l[2], l[3]};
                    }
                } else {
                    const u32x4 xh = u32x4{cvt_pk(xs[0], xs[1]), cvt_pk(xs[2], xs[3]),
                                           cvt_pk(xs[4], xs[5]), cvt_pk(xs[6], xs[7])};
                    if (lane < 32)
                        *reinterpret_cast<u32x4*>(bfp(tset(x1), L::TH) + rr * P24 + 8 * half) = xh;
                }
            }
            lds_barrier();
        }
    } else if (wave == NA + 1) {
        // ------------------------ AP-P: P, w . v ----------------------------
        // lane: token t = lane / 4, state rows 8 (lane % 4) .. + 7
        struct Buf {
            u32x4 v, w;
        };
        const int wt = lane >> 2, wr = 8 * (lane & 3);
        auto load = [&](int64_t cn, Buf& f) {
            if (!p.v) {
                // no v (nor w): v = 0 (the sequence split's transition pass)
                f.v = u32x4{0u, 0u, 0u, 0u};
                f.w = u32x4{0u, 0u, 0u, 0u};
                return;
            }
            const uint32_t off = (uint32_t)(min(wt, last_row(cn)) * (int)(H * DV) + wr) * 2u;
            const char* vb = reinterpret_cast<const char*>(p.v + vofs + cn * CH * H * DV);
            const char* wb = reinterpret_cast<const char*>(p.write + vofs + cn * CH * H * DV);
            f.v = *reinterpret_cast<const u32x4*>(vb + off);
            f.w = *reinterpret_cast<const u32x4*>(wb + off);
        };
        auto prepare = [&](int64_t cn, const Buf& f) {
            unsigned char* es = eset(cn);
            unsigned char* ts = tset(cn);
            f32x4 pv;
            if (!wide_flag(es)) {
                // C[4 g + r][m] = sum_c Q[m][c] K'[4 g + r][c] = P[m][4 g + r];
                // kept for 4 g + r <= m
                f32x4 acc[3] = {};
#pragma unroll
                for (int j = 0; j < KJ; ++j) {
                    const int aq = kq_at<DK>(m, 32 * j + 8 * g);
                    const bf16x8 xh = *reinterpret_cast<const bf16x8*>(bfp(es, L::QH) + aq);
                    const bf16x8 xl = *reinterpret_cast<const bf16x8*>(bfp(es, L::QL) + aq);
                    const int at = m * L::PKN + 32 * j + 4 * g;
                    const bf16x8 kh = ld2x4(bfp(es, L::KH) + at, bfp(es, L::KH) + at + 16);
                    const bf16x8 kl = ld2x4(bfp(es, L::KL) + at, bfp(es, L::KL) + at + 16);
                    acc[0] = mfma16(kh, xh, acc[0]);
                    acc[1] = mfma16(kh, xl, acc[1]);
                    acc[2] = mfma16(kl, xh, acc[2]);
                }
                const f32x4 s = acc[0] + acc[1] + acc[2];
#pragma unroll
                for (int r = 0; r < 4; ++r) pv[r] = 4 * g + r <= m ? s[r] : 0.f;
                // NORM: P~ = pi_r P (the wide path's P already carries it)
                if constexpr (NORM) pv *= reinterpret_cast<const float*>(es + L::NR)[NR_PI + m];
            } else {
                const float* Wp = reinterpret_cast<const float*>(smem + L::WP + (int)(cn & 1) * CH * PAF * 4);
                pv = *reinterpret_cast<const f32x4*>(Wp + m * PAF + 4 * g);
            }
            s16x4 xh, xl;
            split4(pv, xh, xl);
            *reinterpret_cast<s16x4*>(bfp(ts, L::PH) + m * P24 + 4 * g) = xh;
            *reinterpret_cast<s16x4*>(bfp(ts, L::PL) + m * P24 + 4 * g) = xl;
            const bool live = wt < n_live(cn);
            float* wv = reinterpret_cast<float*>(ts + L::WV);
            // NORM: rho_t w.v, the first term of R~
            const float rw = NORM ? reinterpret_cast<const float*>(es + L::NR)[NR_RHO + wt] : 1.f;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                if constexpr (NORM) {
                    wv[(wr + 2 * x) * P24 + wt] = live ? lo_bf(f.w[x]) * lo_bf(f.v[x]) * rw : 0.f;
                    wv[(wr + 2 * x + 1) * P24 + wt] = live ? hi_bf(f.w[x]) * hi_bf(f.v[x]) * rw : 0.f;
                } else {
                    wv[(wr + 2 * x) * P24 + wt] = live ? lo_bf(f.w[x]) * lo_bf(f.v[x]) : 0.f;
                    wv[(wr + 2 * x + 1) * P24 + wt] = live ? hi_bf(f.w[x]) * hi_bf(f.v[x]) : 0.f;
                }
            }
        };
        Buf fa, fb, fc;
        run(1, load, prepare, fa, fb, fc);
    } else {
        // ------------- E0..E3: lambda, 1 / lambda, E, Q, K' -------------------
        const int ej = wave - NA - 2;
        auto erole = [&](auto t0c, auto ntc) {
            constexpr int T0 = decltype(t0c)::value;   // first token of this wave
            constexpr int NT = decltype(ntc)::value;   // tokens of this wave
            struct Buf {
                uint32_t a[T0 + NT];
                uint32_t k[NT], b[NT], q[NT];
            };
            // buffer loads: a per-chunk resource whose range ends at the
            // sequence end (rows past it read as 0), and per-row lane
            // offsets computed once
            int roff[T0 + NT];
#pragma unroll
            for (int t = 0; t < T0 + NT; ++t) roff[t] = t * (int)tstride * 2 + 4 * cp;
            auto load = [&](int64_t cn, Buf& f) {
                const int64_t cb = kofs + cn * CH * tstride;
                const int nbytes = n_live(cn) * (int)tstride * 2;
                const auto ra = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(p.alpha + cb), (short)0, nbytes, 0x00020000);
                const auto rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(p.k + cb), (short)0, nbytes, 0x00020000);
                const auto rb = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(p.erase + cb), (short)0, nbytes, 0x00020000);
                const auto rq = __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16_t*>(p.q + cb), (short)0, nbytes, 0x00020000);
#pragma unroll
                for (int t = 0; t < T0 + NT; ++t)
                    f.a[t] = __builtin_amdgcn_raw_buffer_load_b32(ra, roff[t], 0, 0);
#pragma unroll
                for (int u = 0; u < NT; ++u) {
                    f.k[u] = __builtin_amdgcn_raw_buffer_load_b32(rk, roff[T0 + u], 0, 0);
                    f.b[u] = __builtin_amdgcn_raw_buffer_load_b32(rb, roff[T0 + u], 0, 0);
                    f.q[u] = __builtin_amdgcn_raw_buffer_load_b32(rq, roff[T0 + u], 0, 0);
                }
            };
            const int pc = kperm(2 * cp);
            auto body = [&](int64_t cn, const Buf& f, int n, auto maskc) {
                constexpr bool MASK = decltype(maskc)::value;
                unsigned char* es = eset(cn);
                auto live = [&](int t) { return !MASK || t < n; };
                float l0 = 1.f, l1 = 1.f;
#pragma unroll
                for (int t = 0; t < T0; ++t) {
                    if (live(t)) {
                        l0 *= lo_bf(f.a[t]);
                        l1 *= hi_bf(f.a[t]);
                    }
                }
                if constexpr (NORM) {
                    // partial sums of k^2 and q^2 over this lane's channel
                    // pair (rows past the end read 0)
                    float* ps = reinterpret_cast<float*>(smem + L::PS) + (int)(cn & 1) * CH * 128;
#pragma unroll
                    for (int u = 0; u < NT; ++u) {
                        const float k0 = lo_bf(f.k[u]), k1 = hi_bf(f.k[u]);
                        const float q0 = lo_bf(f.q[u]), q1 = hi_bf(f.q[u]);
                        if (DK == 128 || lane < 32)
                            *reinterpret_cast<float2*>(ps + ps_at(T0 + u, lane)) =
                                float2{__builtin_fmaf(k1, k1, k0 * k0), __builtin_fmaf(q1, q1, q0 * q0)};
                    }
                }
#pragma unroll
                for (int u = 0; u < NT; ++u) {
                    const int t = T0 + u;
                    const bool lv = live(t);
                    if (lv) {
                        l0 *= lo_bf(f.a[t]);
                        l1 *= hi_bf(f.a[t]);
                    }
                    const float r0 = __builtin_amdgcn_rcpf(l0), r1 = __builtin_amdgcn_rcpf(l1);
                    const float k0 = lo_bf(f.k[u]), k1 = hi_bf(f.k[u]);
                    const float e0 = lv ? lo_bf(f.b[u]) * k0 : 0.f;
                    const float e1 = lv ? hi_bf(f.b[u]) * k1 : 0.f;
                    const int ot = kq_at<DK>(t, pc);
                    uint32_t xh, xl;
                    if constexpr (FULL) {
                        split2(e0 * l0, e1 * l1, xh, xl);
                        *reinterpret_cast<uint32_t*>(bfp(es, L::EH) + ot) = xh;
                        *reinterpret_cast<uint32_t*>(bfp(es, L::EL) + ot) = xl;
                    } else {
                        *reinterpret_cast<uint32_t*>(bfp(es, L::EH) + ot) = cvt_pk(e0 * l0, e1 * l1);
                    }
                    split2(lo_bf(f.q[u]) * l0, hi_bf(f.q[u]) * l1, xh, xl);
                    *reinterpret_cast<uint32_t*>(bfp(es, L::QH) + ot) = xh;
                    *reinterpret_cast<uint32_t*>(bfp(es, L::QL) + ot) = xl;
                    split2(k0 * r0, k1 * r1, xh, xl);
                    *reinterpret_cast<uint32_t*>(bfp(es, L::KH) + t * L::PKN + 2 * cp) = xh;
                    *reinterpret_cast<uint32_t*>(bfp(es, L::KL) + t * L::PKN + 2 * cp) = xl;
                }
                if constexpr (T0 + NT == CH) {
                    float* lc = reinterpret_cast<float*>(es + L::LC);
                    *reinterpret_cast<float2*>(lc + 2 * cp) = float2{l0, l1};
                    const bool w = !(l0 >= kLamMin && l1 >= kLamMin);
                    const uint64_t any = __builtin_amdgcn_ballot_w64(w);
                    if (lane == 0) *reinterpret_cast<int*>(lc + DK) = any != 0 ? 1 : 0;
                }
            };
            auto prepare = [&](int64_t cn, const Buf& f) {
                const int n = n_live(cn);
                if (n == CH)
                    body(cn, f, n, std::false_type{});
                else
                    body(cn, f, n, std::true_type{});
            };
            Buf fa, fb, fc;
            run(DEPTH, load, prepare, fa, fb, fc);
        };
        // tokens per wave 3, 3, 5, 5: waves 4 and 5 share their SIMDs with
        // team A, waves 6 and 7 with the lighter AP waves (measured best of
        // the splits tried: 4/4/4/4, 3/3/5/5, 3/4/5/4, 3/4/4/5, 2/2/6/6, 3/3/4/6, 2/3/5/6)
        if (ej == 0) erole(std::integral_constant<int, 0>{}, std::integral_constant<int, 3>{});
        else if (ej == 1) erole(std::integral_constant<int, 3>{}, std::integral_constant<int, 3>{});
        else if (ej == 2) erole(std::integral_constant<int, 6>{}, std::integral_constant<int, 5>{});
        else erole(std::integral_constant<int, 11>{}, std::integral_constant<int, 5>{});
    }
}

template <int DK, int DV, typename TOut, bool NORM, bool FULL = false>
hipError_t launch_n(const ChunkArgs& a) {
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
    const size_t lds = Lay2<DK, NORM, FULL>::TOTAL;
    auto fn = gdr2_bf16_kernel<DK, DV, TOut, NORM, FULL>;
    hipError_t e =
        hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    // 8 * ceil(B*H / 8) heads' worth of row blocks; surplus workgroups exit
    const unsigned grid = (unsigned)(((a.B * a.H + 7) / 8) * 8 * (DV / RB));
    hipLaunchKernelGGL(fn, dim3(grid), dim3(64 * NWAVE), lds, a.stream, p);
    return hipGetLastError();
}

template <int DK, int DV, typename TOut>
hipError_t launch_t(const ChunkArgs& a) {
    return a.l2norm ? launch_n<DK, DV, TOut, true>(a) : launch_n<DK, DV, TOut, false>(a);
}

template <int DK, int DV>
hipError_t launch_d(const ChunkArgs& a) {
    if (a.full) {
        // only the sequence split's state passes ask for it (no o)
        return a.l2norm ? launch_n<DK, DV, float, true, true>(a)
                        : launch_n<DK, DV, float, false, true>(a);
    }
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
