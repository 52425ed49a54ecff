// bf16-input path of gdr2_chunk_fwd: Gated Delta Rule-2 in chunks of 64 on
// gfx950 matrix cores.
//
// The rule ("Gated DeltaNet-2", agihunt.info): per token, decay the state
// with the per-channel alpha_t on the key axis, read the old value along
// e_t = b_t (.) k_t, write the residual of w_t (.) v_t against that read
// along k_t.  The page states that in chunks the channel decay folds into an
// asymmetric rank-1 erase factor and the chunk is a WY triangular solve plus
// dense products.  With G_rc = sum_{i<=r} log alpha_ic inside the chunk
// (per channel) and lambda_r = e^{G_r}, unrolling the recurrence gives
//
//   A_sj  = sum_c e_sc k_jc e^{G_sc - G_jc}                  j < s
//   P_rs  = sum_c q_rc k_sc e^{G_rc - G_sc}                  s <= r
//   T     = (I + A)^{-1}
//   R_s   = w_s (.) v_s - S (e_s (.) lambda_s)
//   V_new = T R
//   o_r   = S (q_r (.) lambda_r) + sum_{s<=r} P_rs V_new_s
//   S    <- S diag(lambda_C) + sum_s V_new_s (k_s (.) lambda_C / lambda_s)^T
//
// Decayed products A and P: the ratio e^{G_s - G_j} cannot be split into
// two bounded factors over a whole chunk, so rows are taken in blocks of 16
// with the position m just before the block as reference:
// e^{G_s - G_j} = e^{G_s - G_m} e^{G_m - G_j}.  Both factors are <= 1 for j
// in earlier blocks; on the block's own diagonal the second factor is <= the
// exponential of the block's decay range.  If that range passes 80 (natural
// log units) in any channel, the diagonal block is formed entry by entry.
//
// Work split: one 256-thread workgroup per (b, h, 32 state rows) — LDS
// holds the per-channel log decays as fp32, so 32 rows fit, not 64.
// Every product with a computed operand uses the bf16 hi/lo split.
#include "launch.h"
#include "mfma_common.h"
#include "wy_solve.h"

namespace gdr {

namespace {

constexpr int CH = 64;    // tokens per chunk
constexpr int RB = 32;    // state rows per workgroup
constexpr int NT = 256;
constexpr float kRangeMax = 80.f;   // widest factored decay range (natural log)


struct Gdr2Params {
    int64_t T, H, BH;
    const bf16_t *q, *k, *v, *alpha, *erase, *write;
    const float* s0;
    void* o;
    float* s_final;
};

template <int DK>
struct Smem2 {
    static constexpr int PK = DK + 8;   // bf16 row pitch
    static constexpr int PG = DK + 4;   // fp32 row pitch of G
    static constexpr int KB = 0;                                 // K [64][PK]
    static constexpr int GB = KB + 64 * PK * 2;                  // G [64][PG] fp32
    static constexpr int XR = GB + 64 * PG * 4;                  // Q | B | WV^T, then solve
    static constexpr int QB = XR;                                //   Q [64][PK]
    static constexpr int BB = QB + 64 * PK * 2;                  //   erase [64][PK]
    static constexpr int WV = BB + 64 * PK * 2;                  //   (w.v)^T fp32 [RB][PF]
    static constexpr int XR_IN = 2 * 64 * PK * 2 + RB * PF * 4;
    static constexpr int TF = XR;                                //   T fp32 [64][PF]
    static constexpr int TH = TF + 64 * PF * 4;                  //   T hi [64][P72]
    static constexpr int TL = TH + 64 * P72 * 2;                 //   T lo
    static constexpr int XS = TL + 64 * P72 * 2;                 //   4 x [16][PX] fp32
    static constexpr int XR_SOLVE = 64 * PF * 4 + 2 * 64 * P72 * 2 + 4 * 16 * PX * 4;
    static constexpr int SH = XR + (XR_IN > XR_SOLVE ? XR_IN : XR_SOLVE);  // S hi [RB][PK]
    static constexpr int SL = SH + RB * PK * 2;
    static constexpr int AN = SL + RB * PK * 2;                  // A fp32 [64][PF] | V_new^T
    static constexpr int AN_SZ = (64 * PF * 4) > (2 * RB * P72 * 2) ? (64 * PF * 4)
                                                                    : (2 * RB * P72 * 2);
    static constexpr int PP = AN + AN_SZ;                        // P hi, lo [64][P72]
    static constexpr int RM = PP + 2 * 64 * P72 * 2;             // R^T hi, lo [RB][P72]
    static constexpr int FL = RM + 2 * RB * P72 * 2;             // 4 wide-range flags
    static constexpr int TOTAL = FL + 16;
};

template <int DK, int DV, typename TOut>
__global__ __launch_bounds__(NT) void gdr2_bf16_kernel(Gdr2Params p) {
    using M = Smem2<DK>;
    constexpr int PK = M::PK;
    constexpr int PG = M::PG;
    constexpr int NRB = DV / RB;
    constexpr int KC = DK / 8;               // 16-byte pieces per key-side row
    constexpr int KLD = CH * KC / NT;
    constexpr int VC = RB / 8;               // 16-byte pieces per value-side row slice
    constexpr int VLD = (CH * VC + NT - 1) / NT;
    constexpr int KS = DK / 16;              // 32x32x16 k-steps over channels
    constexpr int KS32 = DK / 32;            // 16x16x32 k-steps over channels
    constexpr int NSW = DK / 32;             // S^T tiles (one per wave while < 4)
    static_assert(KLD * NT == CH * KC, "load split");
    static_assert(M::TOTAL <= 160 * 1024, "LDS budget");

    extern __shared__ __align__(16) unsigned char smem[];
    bf16_t* Kb = reinterpret_cast<bf16_t*>(smem + M::KB);
    float* Gs = reinterpret_cast<float*>(smem + M::GB);
    bf16_t* Qb = reinterpret_cast<bf16_t*>(smem + M::QB);
    bf16_t* Bb = reinterpret_cast<bf16_t*>(smem + M::BB);
    float* WVt = reinterpret_cast<float*>(smem + M::WV);
    float* Tf = reinterpret_cast<float*>(smem + M::TF);
    bf16_t* Th = reinterpret_cast<bf16_t*>(smem + M::TH);
    bf16_t* Tl = reinterpret_cast<bf16_t*>(smem + M::TL);
    float* Xs = reinterpret_cast<float*>(smem + M::XS);
    bf16_t* Sh = reinterpret_cast<bf16_t*>(smem + M::SH);
    bf16_t* Sl = reinterpret_cast<bf16_t*>(smem + M::SL);
    float* Af = reinterpret_cast<float*>(smem + M::AN);
    bf16_t* Nh = reinterpret_cast<bf16_t*>(smem + M::AN);
    bf16_t* Nl = Nh + RB * P72;
    bf16_t* Ph = reinterpret_cast<bf16_t*>(smem + M::PP);
    bf16_t* Pl = Ph + 64 * P72;
    bf16_t* Rh = reinterpret_cast<bf16_t*>(smem + M::RM);
    bf16_t* Rl = Rh + RB * P72;
    int* flags = reinterpret_cast<int*>(smem + M::FL);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int hi = lane >> 5;
    const int m16 = lane & 15;
    const int kq = lane >> 4;
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
    const int tb = wave >> 1;     // 32-token block of the (2), (4), (5) tiles
    const bool sideR = (wave & 1) == 0;   // waves 0, 2: R and V_new; 1, 3: Q S^T and o

    // ---- initial state: S^T tile `wave` (channels 32 wave ..) ------------
    f32x16 sacc = {};
    if (wave < NSW) {
        const int i = l32;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int c = wave * 32 + 8 * j + 4 * hi;
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
            if (p.s0)
                x = *reinterpret_cast<const f32x4*>(p.s0 + ((bh * DV + row0 + i) * DK + c));
            sacc[4 * j + 0] = x.x;
            sacc[4 * j + 1] = x.y;
            sacc[4 * j + 2] = x.z;
            sacc[4 * j + 3] = x.w;
            st4_split(Sh + i * PK + c, Sl + i * PK + c, x.x, x.y, x.z, x.w);
        }
    }

    // ---- register prefetch -------------------------------------------------
    const int64_t kbase = (b * T * H + h) * DK;
    const int64_t vbase = (b * T * H + h) * DV + row0;
    u32x4 pk[KLD], pq[KLD], pe[KLD], pa[KLD], pv[VLD], pw[VLD];
    auto prefetch = [&](int64_t t0) {
#pragma unroll
        for (int m = 0; m < KLD; ++m) {
            const int c = tid + NT * m;
            const int row = c / KC, col = (c % KC) * 8;
            const int64_t tok = t0 + row;
            if (tok < T) {
                const int64_t off = kbase + tok * H * DK + col;
                pk[m] = *reinterpret_cast<const u32x4*>(p.k + off);
                pq[m] = *reinterpret_cast<const u32x4*>(p.q + off);
                pe[m] = *reinterpret_cast<const u32x4*>(p.erase + off);
                pa[m] = *reinterpret_cast<const u32x4*>(p.alpha + off);
            } else {
                pk[m] = u32x4{0u, 0u, 0u, 0u};
                pq[m] = u32x4{0u, 0u, 0u, 0u};
                pe[m] = u32x4{0u, 0u, 0u, 0u};
                pa[m] = u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};  // 1.0
            }
        }
#pragma unroll
        for (int m = 0; m < VLD; ++m) {
            const int c = tid + NT * m;
            const int row = c / VC, col = (c % VC) * 8;
            const int64_t tok = t0 + row;
            if (c < CH * VC && tok < T) {
                const int64_t off = vbase + tok * H * DV + col;
                pv[m] = *reinterpret_cast<const u32x4*>(p.v + off);
                pw[m] = *reinterpret_cast<const u32x4*>(p.write + off);
            } else {
                pv[m] = u32x4{0u, 0u, 0u, 0u};
                pw[m] = u32x4{0u, 0u, 0u, 0u};
            }
        }
    };

    prefetch(0);
    const int64_t nch = (T + CH - 1) / CH;
    for (int64_t c = 0; c < nch; ++c) {
        const int64_t t0 = c * CH;
        const int n = (int)((T - t0) < CH ? (T - t0) : CH);
        lds_barrier();
        // ---- stage: K, Q, erase (bf16), log alpha (fp32), (w.v)^T (fp32) ---
#pragma unroll
        for (int m = 0; m < KLD; ++m) {
            const int cc = tid + NT * m;
            const int row = cc / KC, col = (cc % KC) * 8;
            *reinterpret_cast<u32x4*>(Kb + row * PK + col) = pk[m];
            *reinterpret_cast<u32x4*>(Qb + row * PK + col) = pq[m];
            *reinterpret_cast<u32x4*>(Bb + row * PK + col) = pe[m];
            const f32x8 a8 = f32x8{__uint_as_float(pa[m][0] << 16), __uint_as_float(pa[m][0] & 0xffff0000u),
                                   __uint_as_float(pa[m][1] << 16), __uint_as_float(pa[m][1] & 0xffff0000u),
                                   __uint_as_float(pa[m][2] << 16), __uint_as_float(pa[m][2] & 0xffff0000u),
                                   __uint_as_float(pa[m][3] << 16), __uint_as_float(pa[m][3] & 0xffff0000u)};
            f32x4 l0, l1;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                l0[e] = safe_log(a8[e]);
                l1[e] = safe_log(a8[4 + e]);
            }
            *reinterpret_cast<f32x4*>(Gs + row * PG + col) = l0;
            *reinterpret_cast<f32x4*>(Gs + row * PG + col + 4) = l1;
        }
#pragma unroll
        for (int m = 0; m < VLD; ++m) {
            const int cc = tid + NT * m;
            if (cc < CH * VC) {
                const int row = cc / VC, col = (cc % VC) * 8;
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    const float v0 = __uint_as_float(pv[m][x] << 16), v1 = __uint_as_float(pv[m][x] & 0xffff0000u);
                    const float w0 = __uint_as_float(pw[m][x] << 16), w1 = __uint_as_float(pw[m][x] & 0xffff0000u);
                    WVt[(col + 2 * x) * PF + row] = w0 * v0;
                    WVt[(col + 2 * x + 1) * PF + row] = w1 * v1;
                }
            }
        }
        if (tid < 4) flags[tid] = 0;
        if (c + 1 < nch) prefetch(t0 + CH);
        lds_barrier();
        // ---- cumulative log decay per channel (segments of 64 / SEG rows) ---
        {
            constexpr int SEG = NT / DK;            // threads per channel
            constexpr int LEN = CH / SEG;
            const int ch = tid % DK, sg = tid / DK;
            float acc = 0.f;
#pragma unroll
            for (int r = 0; r < LEN; ++r) {
                acc += Gs[(sg * LEN + r) * PG + ch];
                Gs[(sg * LEN + r) * PG + ch] = acc;
            }
            lds_barrier();
            float off = 0.f;
#pragma unroll
            for (int q2 = 0; q2 < SEG - 1; ++q2)
                if (q2 < sg) off += Gs[(q2 * LEN + LEN - 1) * PG + ch];
            lds_barrier();
            if (sg > 0) {
#pragma unroll
                for (int r = 0; r < LEN; ++r) Gs[(sg * LEN + r) * PG + ch] += off;
            }
            lds_barrier();
            // decay range of each 16-row block, per channel
            for (int e = tid; e < 4 * DK; e += NT) {
                const int I = e / DK, cc = e % DK;
                const float gm = I == 0 ? 0.f : Gs[(16 * I - 1) * PG + cc];
                if (gm - Gs[(16 * I + 15) * PG + cc] > kRangeMax) atomicOr(flags + I, 1);
            }
        }
        lds_barrier();

        // ---- (1) A and P, 16x16 blocks (I, J <= I): wave I takes row block I
        {
            const int I = wave;
            const int s = 16 * I + m16;          // operand row of this lane
            const float* gm_row = I == 0 ? nullptr : Gs + (16 * I - 1) * PG;
            bf16x8 eh[KS32], el[KS32], qh[KS32], ql[KS32];
#pragma unroll
            for (int ks = 0; ks < KS32; ++ks) {
                const int c0 = 32 * ks + 8 * kq;
                const f32x8 g = ld8f(Gs + s * PG + c0);
                const f32x8 gm = gm_row ? ld8f(gm_row + c0) : f32x8{0, 0, 0, 0, 0, 0, 0, 0};
                const f32x8 kk = ld8bf(Kb + s * PK + c0);
                const f32x8 bb = ld8bf(Bb + s * PK + c0);
                const f32x8 qq = ld8bf(Qb + s * PK + c0);
                f32x8 ev, qv;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float d = __expf(g[e] - gm[e]);
                    ev[e] = bb[e] * kk[e] * d;
                    qv[e] = qq[e] * d;
                }
                split8(ev, eh[ks], el[ks]);
                split8(qv, qh[ks], ql[ks]);
            }
            for (int J = 0; J <= I; ++J) {
                const int j = 16 * J + m16;
                f32x4 aa = {0.f, 0.f, 0.f, 0.f}, pp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS32; ++ks) {
                    const int c0 = 32 * ks + 8 * kq;
                    const f32x8 g = ld8f(Gs + j * PG + c0);
                    const f32x8 gm = gm_row ? ld8f(gm_row + c0) : f32x8{0, 0, 0, 0, 0, 0, 0, 0};
                    const f32x8 kk = ld8bf(Kb + j * PK + c0);
                    f32x8 kv;
#pragma unroll
                    for (int e = 0; e < 8; ++e) kv[e] = kk[e] * __expf(gm[e] - g[e]);
                    bf16x8 kh, kl;
                    split8(kv, kh, kl);
                    aa = mfma16(eh[ks], kh, aa);
                    aa = mfma16(eh[ks], kl, aa);
                    aa = mfma16(el[ks], kh, aa);
                    pp = mfma16(qh[ks], kh, pp);
                    pp = mfma16(qh[ks], kl, pp);
                    pp = mfma16(ql[ks], kh, pp);
                }
                if (J == I && flags[I] != 0) {
                    // wide decay range: this diagonal block entry by entry
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int rs = 16 * I + 4 * kq + r, rj = 16 * I + m16;
                        float a1 = 0.f, p1 = 0.f;
                        if (rj <= rs) {
                            for (int cc = 0; cc < DK; ++cc) {
                                const float d = __expf(Gs[rs * PG + cc] - Gs[rj * PG + cc]);
                                const float kj = bf2f(Kb[rj * PK + cc]) * d;
                                a1 += bf2f(Bb[rs * PK + cc]) * bf2f(Kb[rs * PK + cc]) * kj;
                                p1 += bf2f(Qb[rs * PK + cc]) * kj;
                            }
                        }
                        aa[r] = a1;
                        pp[r] = p1;
                    }
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int rs = 16 * I + 4 * kq + r, rj = 16 * J + m16;
                    Af[rs * PF + rj] = (J < I || rj < rs) ? aa[r] : 0.f;
                    bf16_t ph, pl;
                    split_bf16((J < I || rj <= rs) ? pp[r] : 0.f, ph, pl);
                    Ph[rs * P72 + rj] = ph;
                    Pl[rs * P72 + rj] = pl;
                }
            }
            if ((I & 1) == 0) {
                // P's upper block inside the diagonal 32x32 tile is zero
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int rs = 16 * I + 4 * kq + r, rj = 16 * (I + 1) + m16;
                    Ph[rs * P72 + rj] = 0;
                    Pl[rs * P72 + rj] = 0;
                }
            }
        }

        // ---- (2) R = w.v - S (e . lambda)  |  Q S^T with q . lambda ---------
        f32x16 qs = {};
        {
            const int srow = tb * 32 + l32;
            f32x16 acc = {};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int c0 = 16 * ks + 8 * hi;
                const f32x8 g = ld8f(Gs + srow * PG + c0);
                f32x8 x;
                if (sideR) {
                    const f32x8 kk = ld8bf(Kb + srow * PK + c0);
                    const f32x8 bb = ld8bf(Bb + srow * PK + c0);
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = bb[e] * kk[e] * __expf(g[e]);
                } else {
                    const f32x8 qq = ld8bf(Qb + srow * PK + c0);
#pragma unroll
                    for (int e = 0; e < 8; ++e) x[e] = qq[e] * __expf(g[e]);
                }
                bf16x8 xh, xl;
                split8(x, xh, xl);
                const bf16x8 sh = frag(Sh, PK, l32, c0);
                const bf16x8 sl = frag(Sl, PK, l32, c0);
                acc = mfma(xh, sh, acc);
                acc = mfma(xh, sl, acc);
                acc = mfma(xl, sh, acc);
            }
            if (sideR) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int s0 = tb * 32 + 8 * j + 4 * hi;
                    const f32x4 wv = *reinterpret_cast<const f32x4*>(WVt + l32 * PF + s0);
                    st4_split(Rh + l32 * P72 + s0, Rl + l32 * P72 + s0, wv[0] - acc[4 * j],
                              wv[1] - acc[4 * j + 1], wv[2] - acc[4 * j + 2], wv[3] - acc[4 * j + 3]);
                }
            } else {
                qs = acc;
            }
        }
        lds_barrier();

        // ---- (3) T = (I + A)^{-1} (Q, erase and w.v are dead: reuse) -------
        for (int e = tid; e < 2 * 16 * 16; e += NT) {
            const int blk = e >> 8, r = 32 * blk + ((e >> 4) & 15), s = 32 * blk + 16 + (e & 15);
            Th[r * P72 + s] = 0;
            Tl[r * P72 + s] = 0;
        }
        solve_unit_lower_64(Af, Tf, Xs, Th, Tl);

        // ---- (4) V_new = T R (waves 0, 2) ---------------------------------
        f32x16 vn = {};
        if (sideR) {
            const int nks = tb == 0 ? 2 : 4;
            for (int ks = 0; ks < nks; ++ks) {
                const int kk = ks * 16 + 8 * hi;
                const bf16x8 th = frag(Th, P72, tb * 32 + l32, kk);
                const bf16x8 tl = frag(Tl, P72, tb * 32 + l32, kk);
                const bf16x8 rh = frag(Rh, P72, l32, kk);
                const bf16x8 rl = frag(Rl, P72, l32, kk);
                vn = mfma(th, rh, vn);
                vn = mfma(th, rl, vn);
                vn = mfma(tl, rh, vn);
            }
        }
        lds_barrier();  // A is dead: its space takes V_new^T
        if (sideR) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r0 = tb * 32 + 8 * j + 4 * hi;
                st4_split(Nh + l32 * P72 + r0, Nl + l32 * P72 + r0, vn[4 * j], vn[4 * j + 1],
                          vn[4 * j + 2], vn[4 * j + 3]);
            }
        }
        lds_barrier();

        // ---- (5) o = Q S^T + P V_new (waves 1, 3) --------------------------
        if (!sideR) {
            const int nks = tb == 0 ? 2 : 4;
            for (int ks = 0; ks < nks; ++ks) {
                const int kk = ks * 16 + 8 * hi;
                const bf16x8 ph = frag(Ph, P72, tb * 32 + l32, kk);
                const bf16x8 pl = frag(Pl, P72, tb * 32 + l32, kk);
                const bf16x8 nh = frag(Nh, P72, l32, kk);
                const bf16x8 nl = frag(Nl, P72, l32, kk);
                qs = mfma(ph, nh, qs);
                qs = mfma(ph, nl, qs);
                qs = mfma(pl, nh, qs);
            }
            TOut* o = reinterpret_cast<TOut*>(p.o);
            const int i = row0 + l32;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = tb * 32 + 8 * j + 4 * hi + e;
                    if (r < n) io<TOut>::st(o + (((b * T + t0 + r) * H + h) * DV + i), qs[4 * j + e]);
                }
        }

        // ---- (6) S^T = diag(lambda_C) S^T + (K . lambda_C / lambda)^T V_new --
        if (wave < NSW) {
            const int cl = wave * 32 + l32;     // operand row (channel) of this lane
            const float gC = Gs[(CH - 1) * PG + cl];
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    sacc[4 * j + e] *= __expf(Gs[(CH - 1) * PG + wave * 32 + 8 * j + 4 * hi + e]);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8 kt = frag_tr(Kb, PK, ks * 16, wave * 32);
                f32x8 x;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int s = ks * 16 + 8 * hi + e;
                    x[e] = (float)kt[e] * __expf(gC - Gs[s * PG + cl]);
                }
                bf16x8 xh, xl;
                split8(x, xh, xl);
                const int kk = ks * 16 + 8 * hi;
                const bf16x8 nh = frag(Nh, P72, l32, kk);
                const bf16x8 nl = frag(Nl, P72, l32, kk);
                sacc = mfma(xh, nh, sacc);
                sacc = mfma(xh, nl, sacc);
                sacc = mfma(xl, nh, sacc);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int cc = wave * 32 + 8 * j + 4 * hi;
                st4_split(Sh + l32 * PK + cc, Sl + l32 * PK + cc, sacc[4 * j], sacc[4 * j + 1],
                          sacc[4 * j + 2], sacc[4 * j + 3]);
            }
        }
    }

    if (p.s_final && wave < NSW) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int cc = wave * 32 + 8 * j + 4 * hi;
            *reinterpret_cast<f32x4*>(p.s_final + ((bh * DV + row0 + l32) * DK + cc)) =
                f32x4{sacc[4 * j], sacc[4 * j + 1], sacc[4 * j + 2], sacc[4 * j + 3]};
        }
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
    const size_t lds = Smem2<DK>::TOTAL;
    auto fn = gdr2_bf16_kernel<DK, DV, TOut>;
    hipError_t e =
        hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    // 8 * ceil(B*H / 8) heads' worth of row blocks; surplus workgroups exit
    const unsigned grid = (unsigned)(((a.B * a.H + 7) / 8) * 8 * (DV / RB));
    hipLaunchKernelGGL(fn, dim3(grid), dim3(NT), lds, a.stream, p);
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
