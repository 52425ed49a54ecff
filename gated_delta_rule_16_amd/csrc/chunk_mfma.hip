// bf16-input path of gdr_chunk_fwd: the chunkwise UT/WY form of the gated
// delta rule on gfx950 bf16 matrix cores, one fused pass over the sequence.
//
// Chunk algebra (rows of the state S are value channels; within a chunk of
// C = 64 tokens, g_r = sum_{i<=r} log alpha_i, gamma_r = e^{g_r}; this is
// the review's section 3.7 system on meaningful96.github.io with Gamma_rs =
// e^{g_r - g_s}, the output mask carrying that decay and its diagonal, and
// U^g - W S^T regrouped as T R):
//
//   A_rs  = beta_r e^{g_r - g_s} k_r . k_s            s < r
//   T     = (I + A)^{-1}                              (depends on keys only)
//   R_s   = beta_s (v_s - gamma_s S k_s)              (needs the state)
//   V_new = T R
//   P_rs  = e^{g_r - g_s} q_r . k_s                   s <= r
//   o_r   = gamma_r S q_r + sum_{s<=r} P_rs V_new_s
//   S    <- gamma_C S + sum_s (e^{g_C - g_s} V_new_s) k_s^T
//
// Work split: one 256-thread workgroup (4 waves) per (b, h, 64 state rows);
// rows of S evolve independently given the key side, so Dv = 128 runs as
// two workgroups per head that both build A, T and P.  The workgroup walks
// the chunks in order with S resident: fp32 in matrix-core accumulators
// (as S^T tiles) and a bf16 hi/lo copy in LDS for use as an operand.  The
// next chunk's q, k, v, alpha, beta are loaded into registers while the
// current chunk computes.  Every matrix-core phase first issues all of its
// LDS operand reads and then its MFMAs, so reads stream behind the math.
//
// Per chunk (bf16 32x32x16 MFMA tiles unless noted, 4 waves):
//   (1) K K^T and K Q^T lower tiles -> A (fp32) and P (hi/lo)      48 MFMA
//   (2) K S^T -> R (hi/lo), Q S^T kept in registers              128 MFMA
//   (3) T = (I + A)^{-1} in 16x16 blocks: diagonal blocks by forward
//       substitution (4 lanes per column), then T_10, T_32, and the lower
//       32x32 block -T_22 A_21 T_11 on fp32 16x16x4 matrix cores
//   (4) V_new = T R -> V_new and decayed V_new (hi/lo)              36 MFMA
//   (5) o = gamma (Q S^T) + P V_new -> HBM                          36 MFMA
//   (6) S^T = gamma_C S^T + K^T V' (K^T read transposed from LDS)   64 MFMA
#include "launch.h"
#include "mfma_common.h"
#include "wy_solve.h"

namespace gdr {

namespace {

constexpr int CH = 64;    // tokens per chunk
constexpr int RB = 64;    // state rows per workgroup
constexpr int NT = 256;   // threads per workgroup

struct Bf16Params {
    int64_t T, H, BH;
    const bf16_t *q, *k, *v;
    const float *alpha, *beta;
    const float* s0;
    void* o;
    float* s_final;
};

template <int DK>
struct Smem {
    static constexpr int PK = DK + 8;  // pitch of K, Q, S rows (elements)
    static constexpr int KB = 0;                             // K [64][PK]
    static constexpr int QB = KB + 64 * PK * 2;              // Q [64][PK] | T fp32 [64][PF]
    static constexpr int QB_SZ = (64 * PK * 2) > (64 * PF * 4) ? (64 * PK * 2) : (64 * PF * 4);
    static constexpr int VB = QB + QB_SZ;                    // V [64][P72] | solve scratch
    static constexpr int VB_SZ = (64 * P72 * 2) > (4 * 16 * PX * 4) ? (64 * P72 * 2)
                                                                    : (4 * 16 * PX * 4);
    static constexpr int SH = VB + VB_SZ;                    // S hi [RB][PK]
    static constexpr int SL = SH + RB * PK * 2;              // S lo
    static constexpr int AN = SL + RB * PK * 2;              // A fp32 [64][PF] | V_new^T hi, lo
    static constexpr int AN_SZ = (64 * PF * 4) > (2 * RB * P72 * 2) ? (64 * PF * 4)
                                                                    : (2 * RB * P72 * 2);
    static constexpr int TT = AN + AN_SZ;                    // T hi, lo [64][P72]
    static constexpr int PP = TT + 2 * 64 * P72 * 2;         // P hi, lo [64][P72]
    static constexpr int RM = PP + 2 * 64 * P72 * 2;         // R^T hi, lo | V'^T hi, lo
    static constexpr int GT = RM + 2 * RB * P72 * 2;         // g, beta, gamma, decay-to-end
    static constexpr int TOTAL = GT + 4 * CH * 4;
};

template <int DK, int DV, typename TOut>
__global__ __launch_bounds__(NT) void chunk_bf16_kernel(Bf16Params p) {
    using M = Smem<DK>;
    constexpr int PK = M::PK;
    constexpr int NRB = DV / RB;
    constexpr int KC = DK / 8;               // 16-byte pieces per key row
    constexpr int KLD = CH * KC / NT;        // key (and query) pieces per thread
    constexpr int VC = RB / 8;               // 16-byte pieces per value row slice
    constexpr int VLD = CH * VC / NT;
    constexpr int NS = DK / 64;              // S^T tiles per wave
    constexpr int KS = DK / 16;              // k-steps over the key dim
    static_assert(KLD * NT == CH * KC && VLD * NT == CH * VC, "load split");
    static_assert(M::TOTAL <= 160 * 1024, "LDS budget");

    extern __shared__ __align__(16) unsigned char smem[];
    bf16_t* Kb = reinterpret_cast<bf16_t*>(smem + M::KB);
    bf16_t* Qb = reinterpret_cast<bf16_t*>(smem + M::QB);
    float* Tf = reinterpret_cast<float*>(smem + M::QB);
    bf16_t* Vb = reinterpret_cast<bf16_t*>(smem + M::VB);
    float* Xs = reinterpret_cast<float*>(smem + M::VB);
    bf16_t* Sh = reinterpret_cast<bf16_t*>(smem + M::SH);
    bf16_t* Sl = reinterpret_cast<bf16_t*>(smem + M::SL);
    float* Af = reinterpret_cast<float*>(smem + M::AN);
    bf16_t* Nh = reinterpret_cast<bf16_t*>(smem + M::AN);
    bf16_t* Nl = Nh + RB * P72;
    bf16_t* Th = reinterpret_cast<bf16_t*>(smem + M::TT);
    bf16_t* Tl = Th + 64 * P72;
    bf16_t* Ph = reinterpret_cast<bf16_t*>(smem + M::PP);
    bf16_t* Pl = Ph + 64 * P72;
    bf16_t* Rh = reinterpret_cast<bf16_t*>(smem + M::RM);
    bf16_t* Rl = Rh + RB * P72;
    bf16_t* Mh = Rh;
    bf16_t* Ml = Rl;
    float* g_s = reinterpret_cast<float*>(smem + M::GT);
    float* b_s = g_s + CH;
    float* gam_s = b_s + CH;
    float* dec_s = gam_s + CH;

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
    // tile of the 64 x 64 (token x state-row) products owned by this wave
    const int tb = wave >> 1;
    const int ib = wave & 1;

    // T's upper 16x16 blocks inside its diagonal 32x32 tiles are read as
    // zeros by (4); they are never written afterwards.
    for (int e = tid; e < 2 * 16 * 16; e += NT) {
        const int blk = e >> 8, r = 32 * blk + ((e >> 4) & 15), s = 32 * blk + 16 + (e & 15);
        Th[r * P72 + s] = 0;
        Tl[r * P72 + s] = 0;
    }

    // ---- initial state: S^T tiles in accumulators, hi/lo S in LDS --------
    f32x16 sacc[NS];
#pragma unroll
    for (int u = 0; u < NS; ++u) {
        const int t = wave * NS + u;
        const int dkb = t >> 1, ibs = t & 1;
        const int i = ibs * 32 + l32;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int dk = dkb * 32 + 8 * j + 4 * hi;
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
            if (p.s0)
                x = *reinterpret_cast<const f32x4*>(p.s0 + ((bh * DV + row0 + i) * DK + dk));
            sacc[u][4 * j + 0] = x.x;
            sacc[u][4 * j + 1] = x.y;
            sacc[u][4 * j + 2] = x.z;
            sacc[u][4 * j + 3] = x.w;
            st4_split(Sh + i * PK + dk, Sl + i * PK + dk, x.x, x.y, x.z, x.w);
        }
    }

    // ---- register prefetch of one chunk -----------------------------------
    const bf16_t* kbase = p.k + (b * T * H + h) * DK;
    const bf16_t* qbase = p.q + (b * T * H + h) * DK;
    const bf16_t* vbase = p.v + (b * T * H + h) * DV + row0;
    u32x4 pk[KLD], pq[KLD], pv[VLD];
    float pa = 1.f, pb = 0.f;
    auto prefetch = [&](int64_t t0) {
#pragma unroll
        for (int m = 0; m < KLD; ++m) {
            const int c = tid + NT * m;
            const int row = c / KC, col = (c % KC) * 8;
            const int64_t tok = t0 + row;
            if (tok < T) {
                const int64_t off = tok * H * DK + col;
                pk[m] = *reinterpret_cast<const u32x4*>(kbase + off);
                pq[m] = *reinterpret_cast<const u32x4*>(qbase + off);
            } else {
                pk[m] = u32x4{0u, 0u, 0u, 0u};
                pq[m] = u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int m = 0; m < VLD; ++m) {
            const int c = tid + NT * m;
            const int row = c / VC, col = (c % VC) * 8;
            const int64_t tok = t0 + row;
            if (tok < T)
                pv[m] = *reinterpret_cast<const u32x4*>(vbase + tok * H * DV + col);
            else
                pv[m] = u32x4{0u, 0u, 0u, 0u};
        }
        if (tid < CH) {
            const int64_t tok = t0 + tid;
            pa = tok < T ? p.alpha[(b * T + tok) * H + h] : 1.f;
            pb = tok < T ? p.beta[(b * T + tok) * H + h] : 0.f;
        }
    };

    prefetch(0);
    const int64_t nch = (T + CH - 1) / CH;
    for (int64_t c = 0; c < nch; ++c) {
        const int64_t t0 = c * CH;
        const int n = (int)((T - t0) < CH ? (T - t0) : CH);
        lds_barrier();
        // ---- stage the chunk (row-major; transposes come from tr reads) ----
#pragma unroll
        for (int m = 0; m < KLD; ++m) {
            const int cc = tid + NT * m;
            const int row = cc / KC, col = (cc % KC) * 8;
            *reinterpret_cast<u32x4*>(Kb + row * PK + col) = pk[m];
            *reinterpret_cast<u32x4*>(Qb + row * PK + col) = pq[m];
        }
#pragma unroll
        for (int m = 0; m < VLD; ++m) {
            const int cc = tid + NT * m;
            const int row = cc / VC, col = (cc % VC) * 8;
            *reinterpret_cast<u32x4*>(Vb + row * P72 + col) = pv[m];
        }
        if (wave == 0) {
            const float gx = wave_scan(safe_log(pa));   // cumulative log decay
            const float glast = __shfl(gx, 63, 64);
            g_s[lane] = gx;
            b_s[lane] = pb;
            gam_s[lane] = __expf(gx);
            dec_s[lane] = __expf(glast - gx);
        }
        if (c + 1 < nch) prefetch(t0 + CH);
        lds_barrier();

        // ---- (1) A and P from the lower 32x32 tiles of K K^T and K Q^T ----
        if (wave < 3) {
            const int sb = wave == 2 ? 1 : 0;   // tile rows: tokens s
            const int rt = wave == 0 ? 0 : 1;   // tile cols: tokens r
            bf16x8 fa[KS], fk[KS], fq[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int kk = ks * 16 + 8 * hi;
                fa[ks] = frag(Kb, PK, sb * 32 + l32, kk);
                fk[ks] = frag(Kb, PK, rt * 32 + l32, kk);
                fq[ks] = frag(Qb, PK, rt * 32 + l32, kk);
            }
            __builtin_amdgcn_sched_barrier(0);
            f32x16 akk = {}, apk = {};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                akk = mfma(fa[ks], fk[ks], akk);
                apk = mfma(fa[ks], fq[ks], apk);
            }
            const int r = rt * 32 + l32;
            const float gr = g_s[r], br = b_s[r];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int s0 = sb * 32 + 8 * j + 4 * hi;
                const f32x4 gs = *reinterpret_cast<const f32x4*>(g_s + s0);
                float av[4], pv4[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int s = s0 + e;
                    const float d = s <= r ? __expf(fminf(gr - gs[e], 0.f)) : 0.f;
                    av[e] = s < r ? br * d * akk[4 * j + e] : 0.f;
                    pv4[e] = d * apk[4 * j + e];
                }
                *reinterpret_cast<f32x4*>(Af + r * PF + s0) = f32x4{av[0], av[1], av[2], av[3]};
                st4_split(Ph + r * P72 + s0, Pl + r * P72 + s0, pv4[0], pv4[1], pv4[2], pv4[3]);
            }
        }

        // ---- (2) K S^T -> R;  Q S^T kept for the output --------------------
        f32x16 qs = {};
        {
            bf16x8 fk[KS], fq[KS], fh[KS], fl[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const int kk = ks * 16 + 8 * hi;
                fk[ks] = frag(Kb, PK, tb * 32 + l32, kk);
                fq[ks] = frag(Qb, PK, tb * 32 + l32, kk);
                fh[ks] = frag(Sh, PK, ib * 32 + l32, kk);
                fl[ks] = frag(Sl, PK, ib * 32 + l32, kk);
            }
            __builtin_amdgcn_sched_barrier(0);
            f32x16 aks = {};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                aks = mfma(fk[ks], fh[ks], aks);
                qs = mfma(fq[ks], fh[ks], qs);
                aks = mfma(fk[ks], fl[ks], aks);
                qs = mfma(fq[ks], fl[ks], qs);
            }
            const int i = ib * 32 + l32;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int s0 = tb * 32 + 8 * j + 4 * hi;
                // V[s0 .. s0+3][i] via a transposed read of the row-major tile
                const s16x4 vv = lds_tr16(Vb + (s0 + (m16 >> 2)) * P72 + ib * 32 +
                                          16 * (kq & 1) + 4 * (m16 & 3));
                const f32x4 bs = *reinterpret_cast<const f32x4*>(b_s + s0);
                const f32x4 gs = *reinterpret_cast<const f32x4*>(gam_s + s0);
                float r4[4];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    r4[e] = bs[e] * (bf2f((bf16_t)vv[e]) - gs[e] * aks[4 * j + e]);
                st4_split(Rh + i * P72 + s0, Rl + i * P72 + s0, r4[0], r4[1], r4[2], r4[3]);
            }
        }
        lds_barrier();

        // ---- (3) T = (I + A)^{-1} -----------------------------------------
        solve_unit_lower_64(Af, Tf, Xs, Th, Tl);

        // ---- (4) V_new = T R ------------------------------------------------
        f32x16 vn = {};
        {
            bf16x8 th[4], tl[4], rh[4], rl[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                if (ks < 2 || tb == 1) {   // T vanishes above its diagonal 32x32 tiles
                    const int kk = ks * 16 + 8 * hi;
                    th[ks] = frag(Th, P72, tb * 32 + l32, kk);
                    tl[ks] = frag(Tl, P72, tb * 32 + l32, kk);
                    rh[ks] = frag(Rh, P72, ib * 32 + l32, kk);
                    rl[ks] = frag(Rl, P72, ib * 32 + l32, kk);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                if (ks < 2 || tb == 1) {
                    vn = mfma(th[ks], rh[ks], vn);
                    vn = mfma(th[ks], rl[ks], vn);
                    vn = mfma(tl[ks], rh[ks], vn);
                }
            }
        }
        lds_barrier();  // R fully read (its space takes V'), A dead (takes V_new)
        {
            const int i = ib * 32 + l32;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int r0 = tb * 32 + 8 * j + 4 * hi;
                const f32x4 dd = *reinterpret_cast<const f32x4*>(dec_s + r0);
                st4_split(Nh + i * P72 + r0, Nl + i * P72 + r0, vn[4 * j], vn[4 * j + 1],
                          vn[4 * j + 2], vn[4 * j + 3]);
                st4_split(Mh + i * P72 + r0, Ml + i * P72 + r0, vn[4 * j] * dd[0],
                          vn[4 * j + 1] * dd[1], vn[4 * j + 2] * dd[2], vn[4 * j + 3] * dd[3]);
            }
        }
        lds_barrier();

        // ---- (5) o = gamma (Q S^T) + P V_new -------------------------------
        {
            bf16x8 ph[4], pl[4], nh[4], nl[4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                if (ks < 2 || tb == 1) {   // P vanishes above its diagonal tiles
                    const int kk = ks * 16 + 8 * hi;
                    ph[ks] = frag(Ph, P72, tb * 32 + l32, kk);
                    pl[ks] = frag(Pl, P72, tb * 32 + l32, kk);
                    nh[ks] = frag(Nh, P72, ib * 32 + l32, kk);
                    nl[ks] = frag(Nl, P72, ib * 32 + l32, kk);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const f32x4 gg = *reinterpret_cast<const f32x4*>(gam_s + tb * 32 + 8 * j + 4 * hi);
#pragma unroll
                for (int e = 0; e < 4; ++e) qs[4 * j + e] *= gg[e];
            }
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                if (ks < 2 || tb == 1) {
                    qs = mfma(ph[ks], nh[ks], qs);
                    qs = mfma(ph[ks], nl[ks], qs);
                    qs = mfma(pl[ks], nh[ks], qs);
                }
            }
        }
        // ---- (6) S^T = gamma_C S^T + K^T V' --------------------------------
        {
            bf16x8 ka[4], mh[NS][4], ml[NS][4];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int kk = ks * 16 + 8 * hi;
                ka[ks] = frag_tr(Kb, PK, ks * 16, (wave * NS >> 1) * 32);
#pragma unroll
                for (int u = 0; u < NS; ++u) {
                    const int ibs = (wave * NS + u) & 1;
                    mh[u][ks] = frag(Mh, P72, ibs * 32 + l32, kk);
                    ml[u][ks] = frag(Ml, P72, ibs * 32 + l32, kk);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            const float gC = __expf(g_s[CH - 1]);
#pragma unroll
            for (int u = 0; u < NS; ++u) sacc[u] *= gC;
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
#pragma unroll
                for (int u = 0; u < NS; ++u) {
                    sacc[u] = mfma(ka[ks], mh[u][ks], sacc[u]);
                    sacc[u] = mfma(ka[ks], ml[u][ks], sacc[u]);
                }
        }
        {
            TOut* o = reinterpret_cast<TOut*>(p.o);
            const int i = row0 + ib * 32 + l32;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int r = tb * 32 + 8 * j + 4 * hi + e;
                    if (r < n) io<TOut>::st(o + (((b * T + t0 + r) * H + h) * DV + i), qs[4 * j + e]);
                }
#pragma unroll
            for (int u = 0; u < NS; ++u) {
                const int t = wave * NS + u;
                const int dkb = t >> 1, ibs = t & 1;
                const int si = ibs * 32 + l32;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int dk = dkb * 32 + 8 * j + 4 * hi;
                    st4_split(Sh + si * PK + dk, Sl + si * PK + dk, sacc[u][4 * j],
                              sacc[u][4 * j + 1], sacc[u][4 * j + 2], sacc[u][4 * j + 3]);
                }
            }
        }
    }

    if (p.s_final) {
#pragma unroll
        for (int u = 0; u < NS; ++u) {
            const int t = wave * NS + u;
            const int dkb = t >> 1, ibs = t & 1;
            const int i = ibs * 32 + l32;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int dk = dkb * 32 + 8 * j + 4 * hi;
                *reinterpret_cast<f32x4*>(p.s_final + ((bh * DV + row0 + i) * DK + dk)) =
                    f32x4{sacc[u][4 * j], sacc[u][4 * j + 1], sacc[u][4 * j + 2], sacc[u][4 * j + 3]};
            }
        }
    }
}

template <int DK, int DV, typename TOut>
hipError_t launch_bf16_t(const ChunkArgs& a) {
    Bf16Params p;
    p.T = a.T;
    p.H = a.H;
    p.BH = a.B * a.H;
    p.q = (const bf16_t*)a.q;
    p.k = (const bf16_t*)a.k;
    p.v = (const bf16_t*)a.v;
    p.alpha = (const float*)a.alpha;
    p.beta = (const float*)a.beta;
    p.s0 = a.s0;
    p.o = a.o;
    p.s_final = a.s_final;
    const size_t lds = Smem<DK>::TOTAL;
    auto fn = chunk_bf16_kernel<DK, DV, TOut>;
    hipError_t e =
        hipFuncSetAttribute((const void*)fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    // 8 * ceil(B*H / 8) heads' worth of row blocks; surplus workgroups exit
    const unsigned grid = (unsigned)(((a.B * a.H + 7) / 8) * 8 * (DV / RB));
    hipLaunchKernelGGL(fn, dim3(grid), dim3(NT), lds, a.stream, p);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_bf16_d(const ChunkArgs& a) {
    return a.out_bf16 ? launch_bf16_t<DK, DV, bf16_t>(a) : launch_bf16_t<DK, DV, float>(a);
}

}  // namespace

hipError_t launch_chunk_bf16(const ChunkArgs& a) {
    if (a.Dk == 128 && a.Dv == 128) return launch_bf16_d<128, 128>(a);
    if (a.Dk == 128 && a.Dv == 64) return launch_bf16_d<128, 64>(a);
    if (a.Dk == 64 && a.Dv == 128) return launch_bf16_d<64, 128>(a);
    return launch_bf16_d<64, 64>(a);
}

}  // namespace gdr
