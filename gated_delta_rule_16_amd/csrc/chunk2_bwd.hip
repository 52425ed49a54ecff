// gdr2_chunk_bwd: reverse mode of Gated Delta Rule-2, chunk by chunk, in
// fp32 (matrix-core fp32 products, vector-ALU elsewhere).
//
// Per chunk of n <= 16 tokens (G the within-chunk cumulative log alpha per
// channel, lambda = e^G, E = b (.) k, Gamma_rsc = e^{G_rc - G_sc}, E~ = E (.)
// lambda, Q~ = q (.) lambda, K~ = k (.) e^{G_C - G}, lambda_C = e^{G_C}), the
// forward of gdr2_chunk_fwd is
//
//   A_rs = sum_c E_rc K_sc Gamma_rsc (s < r),  P_rs = sum_c Q_rc K_sc Gamma_rsc (s <= r)
//   T = (I + A)^{-1},  R = w (.) v - E~ S^T,  U = T R
//   O = Q~ S^T + P U,  S' = S diag(lambda_C) + U^T K~
//
// and with G' = dL/dS' carried back from the next chunk:
//
//   dU = P^T dO + K~ G'^T    dR = T^T dU    dP = dO U^T (s <= r)
//   dA = -T^T (dU R^T) T^T (s < r)          dw = dR (.) v,  dv = dR (.) w
//   dE~ = -dR S,  dQ~ = dO S,  dK~ = U G'
//   dE_rc = sum_s dA_rs K_sc Gamma_rsc + dE~ (.) lambda    (the decay inside the
//   dQ_rc = sum_s dP_rs K_sc Gamma_rsc + dQ~ (.) lambda     dot products: the
//   dK_sc = sum_r (dA_rs E_rc + dP_rs Q_rc) Gamma_rsc       GDN-2 summary's point
//           + dK~ (.) e^{G_C - G} + dE (.) b                 about its backward)
//   db = dE (.) k
//   dG = E (.) dE_A + Q (.) dQ_P - K (.) dK_AP + dE~ (.) E~ + dQ~ (.) Q~ - dK~ (.) K~
//        (+ sum_r dK~ (.) K~ + (sum_i G' (.) S) (.) lambda_C on the last token)
//   dS = G' diag(lambda_C) + dO^T Q~ - dR^T E~
//
// (dE_A, dQ_P, dK_AP the A and P parts), and dlog alpha is the reverse
// cumulative sum of dG inside the chunk, per channel.
//
// Factored decay.  Gamma_rsc = e^{G_rc} e^{-G_sc}, so with K^ = K (.) e^{-G}
// the decayed sums are plain products: A = E~ K^T, P = Q~ K^T,
// dE_A = lambda (.) (dA K^), dQ_P = lambda (.) (dP K^),
// dK_AP = e^{-G} (.) (dA^T E~ + dP^T Q~).  e^{-G} <= 1 / lambda_C, so a chunk
// where some channel has G_C < -60 ("wide") forms A, P and those sums entry
// by entry from the log decays instead; every other product is the same.
//
// Work split: one 256-thread workgroup (4 waves) per (b, h, 32 state rows)
// runs the forward over its rows (chunk-start states to the workspace), then
// walks the chunks in reverse.  dv, dw and dS_0 are final per workgroup; dq,
// dk, db and the within-chunk d log alpha (formed without the cancelling
// cumulative sum, see the combine below) go to per-row-block partials that
// a second kernel adds (and divides by alpha).  Every product is a set of
// 16 x 16 tiles on the fp32 matrix cores (v_mfma_f32_16x16x4f32: fp32
// operands and accumulation, the vector ALU's precision), the tiles of a
// phase dealt to the four waves; the triangular solves and the elementwise
// terms are vector ALU.  Per chunk the per-channel gradients stay in the registers of
// the wave that owns those channels, from the products to the HBM stores.
//
// The LDS footprint (~142 KB) allows one workgroup per CU, one wave per SIMD,
// so every global input of the next chunk (key-side rows, w, v, dL/do, the
// chunk-start state) is loaded into registers as raw words while the current
// chunk computes, and written to LDS at the top of the next iteration.
#include "gdr_device.h"
#include "launch.h"
#include "vtile.h"

namespace gdr {

namespace {

constexpr int C2 = 16;         // tokens per chunk
constexpr int R2 = 32;         // state rows per workgroup
constexpr int NT2 = 256;       // threads per workgroup
// Decays are kept in log2 units (G2 = G / ln 2) so that every exponential is
// one v_exp_f32; a chunk is wide when some channel's G_C < -60.
constexpr float WIDE2 = -60.f * 1.44269504f;

struct Bwd2Params {
    int64_t T, H, BTH;
    const void *q, *k, *v, *alpha, *erase, *write, *dout;
    const float *s0, *dsf;
    float *dv, *dw, *ds0;
    float* ck;                     // [BH][nch][Dv][Dk]
    float *pq, *pk, *pb, *pg;      // [BTH][Dk] accumulators of dq, dk, derase, d log alpha
                                   // (zero on entry)
    const float* tt;               // [BH][nch][16][16]: T of each chunk (gdn2_bwd_solve)
    bool l2norm;                   // q, k normalised on load (GDR_L2NORM_QK)
};

// LDS tables.  Pitches: key-side rows PK = 4 (mod 64), n x rows PR = 36,
// n x n PC = 20; with the operand order of mma16 these make both its row
// reads (16-byte) and its column reads (4-byte) free of bank conflicts.
template <int DK>
struct BL3 {
    static constexpr int PK = DK + 4;
    static constexpr int PC = 20;
    static constexpr int PR = 36;
    static constexpr int NK = C2 * PK;           // one token x key-dim table
    static constexpr int K = 0;
    static constexpr int Q = K + NK;
    static constexpr int E = Q + NK;             // b (.) k
    static constexpr int BB = E + NK;            // b
    static constexpr int GC = BB + NK;           // cumulative log2 alpha
    static constexpr int LM = GC + NK;           // lambda = e^G
    static constexpr int KT = LM + NK;           // K~
    static constexpr int QT = KT + NK;           // Q~
    static constexpr int ET = QT + NK;           // E~
    static constexpr int KH = ET + NK;           // K^ = K (.) e^{-G}
    static constexpr int S = KH + NK;            // [R2][PK] chunk-start state rows
    static constexpr int G = S + R2 * PK;        // [R2][PK] dL/dS' rows
    static constexpr int A = G + R2 * PK;        // n x n tiles [C2][PC]
    static constexpr int TM = A + C2 * PC;
    static constexpr int P = TM + C2 * PC;
    static constexpr int DP = P + C2 * PC;
    static constexpr int DT = DP + C2 * PC;      // dT, then dA
    static constexpr int Y = DT + C2 * PC;
    static constexpr int W = Y + C2 * PC;        // n x rows tiles [C2][PR]
    static constexpr int V = W + C2 * PR;
    static constexpr int DO = V + C2 * PR;
    static constexpr int R = DO + C2 * PR;
    static constexpr int U = R + C2 * PR;
    static constexpr int DU = U + C2 * PR;
    static constexpr int DR = DU + C2 * PR;
    static constexpr int GS = DR + C2 * PR;      // [DK] sum_i G'_ic S_ic
    static constexpr int WF = GS + DK;           // [4] per-wave "wide" flags
    static constexpr int TOTAL = WF + 4;
    static_assert(TOTAL * 4 <= 160 * 1024, "LDS budget");
    static_assert(PK % 64 == 4 && NK % 4 == 0 && S % 4 == 0 && G % 4 == 0, "pitches");
    static_assert(A % 4 == 0 && W % 4 == 0 && (Y - A) % 4 == 0, "16-byte rows");
};

// One chunk's global inputs for one thread, as raw words: key-side rows
// (token tid / 16, channels j0 .. j0 + NC) and a pair of state rows of w, v
// and dL/do (token tid / 16, rows 2 (tid % 16), + 1).
template <typename TIn, typename TD, int NC>
struct Pre2 {
    static constexpr int WK = NC / packed<TIn>::PER_WORD;
    static constexpr int WP = 2 / packed<TIn>::PER_WORD;
    static constexpr int WD = 2 / packed<TD>::PER_WORD;
    uint32_t k[WK], b[WK], a[WK], q[WK];
    uint32_t w[WP], v[WP], d[WD];
};

struct Solve2Params {
    int64_t T, H, nch, nchunks;
    const void *k, *alpha, *erase;
    float* tt;                     // [B H nch][16][16]
    bool l2norm;
};

// one element of a row of TIn at index i of a buffer, as fp32
template <typename TIn>
__device__ __forceinline__ float bload1(__amdgpu_buffer_rsrc_t r, int i) {
    if constexpr (sizeof(TIn) == 2)
        return __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, 2 * i, 0, 0) << 16);
    else
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, 4 * i, 0, 0));
}

// T = (I + A)^{-1} of every chunk, A_rs = sum_c E_rc K_sc 2^{G_rc - G_sc}
// (s < r), formed as the main kernel formed it (the factored decay, or entry
// by entry in a wide chunk): it depends on the chunk's keys, erase and decay
// only, so the chunks are solved side by side here and the sweeps read T.
// One 64-thread workgroup per (b, h, chunk); lane l takes channels
// l + 64 j of every token.
template <int DK, typename TIn>
__global__ __launch_bounds__(64) void gdn2_bwd_solve(Solve2Params p) {
    constexpr int PK = DK + 4, PC = 20, NQK = DK / 16, CPL = DK / 64;
    __shared__ __align__(16) float t1[C2 * PK], t2[C2 * PK], t3[C2 * PK], As[C2 * PC], Ts[C2 * PC];
    const int lane = threadIdx.x, l16 = lane & 15, lg = lane >> 4;
    const int64_t ci = blockIdx.x;
    const int64_t bh = ci / p.nch, c = ci % p.nch;
    const int64_t h = bh % p.H, b = bh / p.H;
    const int n = (int)min((int64_t)C2, p.T - c * C2);
    const int64_t tb = (b * p.T + c * C2) * p.H + h;
    const int HDK = (int)(p.H * DK);
    constexpr int SI = sizeof(TIn);
    const __amdgpu_buffer_rsrc_t rk =
        rsrc(reinterpret_cast<const TIn*>(p.k) + tb * DK, n * HDK * SI);
    const __amdgpu_buffer_rsrc_t re =
        rsrc(reinterpret_cast<const TIn*>(p.erase) + tb * DK, n * HDK * SI);
    const __amdgpu_buffer_rsrc_t ra =
        rsrc(reinterpret_cast<const TIn*>(p.alpha) + tb * DK, n * HDK * SI);
    // rows past the chunk's end: zero keys and erase, alpha = 1
    float kv[C2][CPL], ev[C2][CPL], gv[C2][CPL];
#pragma unroll
    for (int t = 0; t < C2; ++t)
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int i = t * HDK + lane + 64 * j;
            kv[t][j] = bload1<TIn>(rk, i);
            ev[t][j] = bload1<TIn>(re, i);
            const float a = bload1<TIn>(ra, i);
            gv[t][j] = t < n ? safe_log2(a) : 0.f;
        }
    if (p.l2norm) {
#pragma unroll
        for (int t = 0; t < C2; ++t) {
            float ss = 0.f;
#pragma unroll
            for (int j = 0; j < CPL; ++j) ss += kv[t][j] * kv[t][j];
#pragma unroll
            for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
            const float kn = l2_inv(ss);
#pragma unroll
            for (int j = 0; j < CPL; ++j) kv[t][j] *= kn;
        }
    }
    bool wide_here = false;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        float g = 0.f;
#pragma unroll
        for (int t = 0; t < C2; ++t) {
            g += gv[t][j];
            gv[t][j] = g;            // within-chunk cumulative log2 alpha
            ev[t][j] *= kv[t][j];    // E = erase (.) k
        }
        wide_here |= g < WIDE2;
    }
    const bool wide = __ballot(wide_here) != 0;
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    if (!wide) {
        // A = E~ K^T, E~ = E (.) 2^G, K^ = K (.) 2^-G
#pragma unroll
        for (int t = 0; t < C2; ++t)
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                t1[t * PK + lane + 64 * j] = ev[t][j] * ex2(gv[t][j]);
                t2[t * PK + lane + 64 * j] = kv[t][j] * ex2(fminf(-gv[t][j], 120.f));
            }
        wave_sync();
        const f32x4 acc = mma16<NQK, true, true>(zero4, t1, PK, t2, PK, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * lg + i;
            As[r * PC + l16] = l16 < r ? acc[i] : 0.f;
        }
    } else {
        // entry by entry from the log decays: lane (r = 4 lg + i, s = l16)
#pragma unroll
        for (int t = 0; t < C2; ++t)
#pragma unroll
            for (int j = 0; j < CPL; ++j) {
                t1[t * PK + lane + 64 * j] = ev[t][j];
                t2[t * PK + lane + 64 * j] = kv[t][j];
                t3[t * PK + lane + 64 * j] = gv[t][j];
            }
        wave_sync();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * lg + i;
            float av = 0.f;
            if (l16 < r) {
                for (int cc = 0; cc < DK; cc += 4) {
                    const f32x4 er = ld4(t1 + r * PK + cc), ks = ld4(t2 + l16 * PK + cc);
                    const f32x4 gr = ld4(t3 + r * PK + cc), gs = ld4(t3 + l16 * PK + cc);
#pragma unroll
                    for (int z = 0; z < 4; ++z) av += er[z] * ks[z] * ex2(gr[z] - gs[z]);
                }
            }
            As[r * PC + l16] = av;
        }
    }
    wave_sync();
    // T = (I + A)^{-1}: lane 4 c + q owns column c and the rows m = q (mod
    // 4); row r is delta_rc - sum_{m < r} A_rm T_mc, joined by a quad sum
    {
        const int cl = lane >> 2, q = lane & 3;
        float tq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < C2; ++r) {
            float part = 0.f;
#pragma unroll
            for (int j = 0; j < 4; ++j) part += As[r * PC + 4 * j + q] * tq[j];
            part = qsum(part);
            const float t = r < cl ? 0.f : (r == cl ? 1.f : 0.f) - part;
            if ((r & 3) == q) tq[r >> 2] = t;
            if (q == 0) Ts[r * PC + cl] = t;
        }
    }
    wave_sync();
    const int r = lane >> 2, c4 = 4 * (lane & 3);
    *reinterpret_cast<f32x4*>(p.tt + ci * 256 + r * 16 + c4) = ld4(Ts + r * PC + c4);
}

template <int DK, int DV, typename TIn, typename TD>
__global__ __launch_bounds__(NT2) void chunk2_bwd_kernel(Bwd2Params p) {
    using L = BL3<DK>;
    constexpr int NRB = DV / R2;
    constexpr int NC = DK / 16;
    constexpr int NQK = DK / 16;                // 16-deep blocks over the key dim
    constexpr int CTW = DK / 64;                // channel tiles per wave
    constexpr int NSV = R2 * DK / 4 / NT2;      // 16-byte state pieces per thread
    extern __shared__ __align__(16) float sm[];
    float* Ks = sm + L::K;
    float* Qs = sm + L::Q;
    float* Es = sm + L::E;
    float* Bs = sm + L::BB;
    float* Gc = sm + L::GC;
    float* Lm = sm + L::LM;
    float* Kt = sm + L::KT;
    float* Qt = sm + L::QT;
    float* Et = sm + L::ET;
    float* Kh = sm + L::KH;
    float* Ss = sm + L::S;
    float* Gs = sm + L::G;
    float* As = sm + L::A;
    float* Ts = sm + L::TM;
    float* Ps = sm + L::P;
    float* dPs = sm + L::DP;
    float* dTs = sm + L::DT;
    float* Ys = sm + L::Y;
    float* Wsm = sm + L::W;
    float* Vsm = sm + L::V;
    float* dOs = sm + L::DO;
    float* Rs = sm + L::R;
    float* Us = sm + L::U;
    float* dUs = sm + L::DU;
    float* dRs = sm + L::DR;
    int* WFs = reinterpret_cast<int*>(sm + L::WF);
    float* GSc = sm + L::GS;

    const int tid = threadIdx.x;
    const int wv = tid >> 6, lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
    const int rb = blockIdx.x % NRB;
    const int64_t bh = blockIdx.x / NRB;
    const int64_t h = bh % p.H;
    const int64_t b = bh / p.H;
    const int64_t T = p.T, H = p.H;
    const int row0 = rb * R2;
    const int64_t nch = (T + C2 - 1) / C2;
    float* ckb = p.ck + bh * nch * DV * DK;
    auto tok = [&](int64_t t) { return (b * T + t) * H + h; };
    const int tr = tid >> 4;                   // this thread's token for the loads
    const int j0 = NC * (tid & 15);            // .. and its key channels
    const int i2 = 2 * (tid & 15);             // .. and its pair of state rows
    auto chunk_len = [&](int64_t c) { return (int)min((int64_t)C2, T - c * C2); };

    using PF = Pre2<TIn, TD, NC>;
    auto fetch = [&](PF& x, int64_t c, bool bwd) {
        if (tr < chunk_len(c)) {
            const int64_t tk = tok(c * C2 + tr);
            ldw(x.k, reinterpret_cast<const TIn*>(p.k) + tk * DK + j0);
            ldw(x.b, reinterpret_cast<const TIn*>(p.erase) + tk * DK + j0);
            ldw(x.a, reinterpret_cast<const TIn*>(p.alpha) + tk * DK + j0);
            ldw(x.w, reinterpret_cast<const TIn*>(p.write) + tk * DV + row0 + i2);
            if (bwd) ldw(x.q, reinterpret_cast<const TIn*>(p.q) + tk * DK + j0);
            ldw(x.v, reinterpret_cast<const TIn*>(p.v) + tk * DV + row0 + i2);
            if (bwd) ldw(x.d, reinterpret_cast<const TD*>(p.dout) + tk * DV + row0 + i2);
        }
    };
    // rows >= n: zero tokens with alpha = 1
    auto commit = [&](const PF& x, int64_t c, bool bwd) {
        const bool live = tr < chunk_len(c);
        const int at = tr * L::PK + j0;
        // GDR_L2NORM_QK: the 16 lanes of a token (one DPP row) hold its row
        float kn = 1.f, qn = 1.f;
        if (p.l2norm) {
            float sk = 0.f, sq = 0.f;
#pragma unroll
            for (int y = 0; y < NC; ++y) {
                const float kk = live ? packed<TIn>::at(x.k, y) : 0.f;
                const float qq = (live && bwd) ? packed<TIn>::at(x.q, y) : 0.f;
                sk += kk * kk;
                sq += qq * qq;
            }
            kn = l2_inv(rsum16(sk));
            qn = l2_inv(rsum16(sq));
        }
#pragma unroll
        for (int y0 = 0; y0 < NC; y0 += 4) {
            f32x4 kv, bv, ev, gv, qv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int y = y0 + e;
                kv[e] = live ? packed<TIn>::at(x.k, y) * kn : 0.f;
                bv[e] = live ? packed<TIn>::at(x.b, y) : 0.f;
                gv[e] = live ? safe_log2(packed<TIn>::at(x.a, y)) : 0.f;
                ev[e] = bv[e] * kv[e];
                qv[e] = (live && bwd) ? packed<TIn>::at(x.q, y) * qn : 0.f;
            }
            *reinterpret_cast<f32x4*>(Ks + at + y0) = kv;
            *reinterpret_cast<f32x4*>(Bs + at + y0) = bv;
            *reinterpret_cast<f32x4*>(Es + at + y0) = ev;
            *reinterpret_cast<f32x4*>(Gc + at + y0) = gv;
            if (bwd) *reinterpret_cast<f32x4*>(Qs + at + y0) = qv;
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int o = tr * L::PR + i2 + e;
            Wsm[o] = live ? packed<TIn>::at(x.w, e) : 0.f;
            Vsm[o] = live ? packed<TIn>::at(x.v, e) : 0.f;
            if (bwd) dOs[o] = live ? packed<TD>::at(x.d, e) : 0.f;
        }
    };
    auto fetch_s = [&](f32x4 (&sv)[NSV], int64_t c) {
#pragma unroll
        for (int it = 0; it < NSV; ++it) {
            const int e4 = tid + it * NT2;
            const int i = e4 / (DK / 4), j = 4 * (e4 % (DK / 4));
            sv[it] = *reinterpret_cast<const f32x4*>(ckb + (c * DV + row0 + i) * DK + j);
        }
    };
    auto put_s = [&](const f32x4 (&sv)[NSV], float* dst) {
#pragma unroll
        for (int it = 0; it < NSV; ++it) {
            const int e4 = tid + it * NT2;
            const int i = e4 / (DK / 4), j = 4 * (e4 % (DK / 4));
            *reinterpret_cast<f32x4*>(dst + i * L::PK + j) = sv[it];
        }
    };
    // after a barrier: G by a scan down the tokens per channel (and whether
    // the chunk is wide), then the decay tables; ends on a barrier
    auto tables = [&](bool bwd) {
        bool wide_here = false;
        if (tid < DK) {
            float g[C2];
#pragma unroll
            for (int r = 0; r < C2; ++r) g[r] = Gc[r * L::PK + tid];
#pragma unroll
            for (int r = 1; r < C2; ++r) g[r] += g[r - 1];
#pragma unroll
            for (int r = 0; r < C2; ++r) Gc[r * L::PK + tid] = g[r];
            wide_here = g[C2 - 1] < WIDE2;
        }
        // per-wave flags, read after the closing barrier
        const bool wide_wave = __ballot(wide_here) != 0;
        if (lane == 0) WFs[wv] = wide_wave;
        __syncthreads();
        const int at = tr * L::PK + j0;
#pragma unroll
        for (int y0 = 0; y0 < NC; y0 += 4) {
            const f32x4 g = ld4(Gc + at + y0), gC = ld4(Gc + (C2 - 1) * L::PK + j0 + y0);
            const f32x4 k = ld4(Ks + at + y0), e = ld4(Es + at + y0);
            f32x4 lm, kt, et, kh;
#pragma unroll
            for (int z = 0; z < 4; ++z) {
                lm[z] = ex2(g[z]);
                kt[z] = k[z] * ex2(gC[z] - g[z]);
                et[z] = e[z] * lm[z];
                // used in narrow chunks only (-g < 87 there); clamped so that a
                // wide chunk's unused entries stay finite
                kh[z] = k[z] * ex2(fminf(-g[z], 120.f));
            }
            *reinterpret_cast<f32x4*>(Lm + at + y0) = lm;
            *reinterpret_cast<f32x4*>(Kt + at + y0) = kt;
            *reinterpret_cast<f32x4*>(Et + at + y0) = et;
            *reinterpret_cast<f32x4*>(Kh + at + y0) = kh;
            if (bwd) {
                const f32x4 q = ld4(Qs + at + y0);
                f32x4 qt;
#pragma unroll
                for (int z = 0; z < 4; ++z) qt[z] = q[z] * lm[z];
                *reinterpret_cast<f32x4*>(Qt + at + y0) = qt;
            }
        }
        __syncthreads();
        return (WFs[0] | WFs[1] | WFs[2] | WFs[3]) != 0;
    };
    // wide chunks: A (s < r) and P (s <= r) entry by entry from the log
    // decays, one thread per (r, s)
    auto ap_entries = [&](bool bwd) {
        const int r = tid >> 4, s = tid & 15;
        float av = 0.f, pv = 0.f;
        if (s <= r) {
#pragma unroll 4
            for (int c = 0; c < DK; c += 4) {
                const f32x4 ks = ld4(Ks + s * L::PK + c), gr = ld4(Gc + r * L::PK + c);
                const f32x4 gs = ld4(Gc + s * L::PK + c), er = ld4(Es + r * L::PK + c);
                f32x4 qr = {0.f, 0.f, 0.f, 0.f};
                if (bwd) qr = ld4(Qs + r * L::PK + c);
#pragma unroll
                for (int z = 0; z < 4; ++z) {
                    const float kd = ks[z] * ex2(gr[z] - gs[z]);
                    av += er[z] * kd;
                    pv += qr[z] * kd;
                }
            }
        }
        As[r * L::PC + s] = s < r ? av : 0.f;
        if (bwd) Ps[r * L::PC + s] = pv;
    };
    // a 16 x 16 n x n tile from this wave's accumulator, masked to s < r
    // (strict) or s <= r
    auto put_nn = [&](const f32x4& acc, float* D, bool strict) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * lg + i;
            D[r * L::PC + l16] = (strict ? l16 < r : l16 <= r) ? acc[i] : 0.f;
        }
    };
    // R tile t (rows 16 t ..): R = w (.) v - E~ S^T
    auto r_tile = [&](int t) {
        f32x4 acc = mma16<NQK, true, true>(f32x4{0.f, 0.f, 0.f, 0.f}, Et, L::PK,
                                           Ss + 16 * t * L::PK, L::PK);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int o = (4 * lg + i) * L::PR + 16 * t + l16;
            Rs[o] = Wsm[o] * Vsm[o] - acc[i];
        }
    };
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

    // ======================= forward: chunk-start states =====================
    {
        f32x4 sv[NSV];
        if (p.s0) {
#pragma unroll
            for (int it = 0; it < NSV; ++it) {
                const int e4 = tid + it * NT2;
                const int i = e4 / (DK / 4), j = 4 * (e4 % (DK / 4));
                sv[it] = *reinterpret_cast<const f32x4*>(p.s0 + (bh * DV + row0 + i) * DK + j);
            }
        } else {
#pragma unroll
            for (int it = 0; it < NSV; ++it) sv[it] = zero4;
        }
        put_s(sv, Ss);
    }
    // this thread's entry of a chunk's T (from gdn2_bwd_solve)
    float tv;
    auto fetch_t = [&](int64_t c) { tv = p.tt[(bh * nch + c) * 256 + tid]; };
    auto commit_t = [&]() { Ts[(tid >> 4) * L::PC + (tid & 15)] = tv; };
    PF x;
    fetch(x, 0, false);
    fetch_t(0);
    for (int64_t c = 0; c < nch; ++c) {
        __syncthreads();
#pragma unroll
        for (int it = 0; it < NSV; ++it) {
            const int e4 = tid + it * NT2;
            const int i = e4 / (DK / 4), j = 4 * (e4 % (DK / 4));
            *reinterpret_cast<f32x4*>(ckb + (c * DV + row0 + i) * DK + j) =
                ld4(Ss + i * L::PK + j);
        }
        commit(x, c, false);
        commit_t();
        if (c + 1 < nch) {
            fetch(x, c + 1, false);
            fetch_t(c + 1);
        }
        __syncthreads();
        tables(false);
        // R, then U = T R, on row tile wv (waves 0, 1)
        if (wv < 2) {
            const int t = wv;
            r_tile(t);
            wave_sync();
            const f32x4 acc = mma16<1, true, false>(zero4, Ts, L::PC, Rs + 16 * t, L::PR);
#pragma unroll
            for (int i = 0; i < 4; ++i) Us[(4 * lg + i) * L::PR + 16 * t + l16] = acc[i];
        }
        __syncthreads();
        // S <- S diag(lambda_C) + U^T K~: row tiles a, this wave's channel tiles
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) {
            const int t = CTW * wv + ct, cc = 16 * t + l16;
            const float lmC = Lm[(C2 - 1) * L::PK + cc];
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                f32x4 acc;
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] = Ss[(16 * a + 4 * lg + i) * L::PK + cc] * lmC;
                acc = mma16<1, false, false>(acc, Us + 16 * a, L::PR, Kt + 16 * t, L::PK);
#pragma unroll
                for (int i = 0; i < 4; ++i) Ss[(16 * a + 4 * lg + i) * L::PK + cc] = acc[i];
            }
        }
    }

    // ======================= reverse sweep ====================================
    __syncthreads();
    {
        f32x4 gv[NSV];
#pragma unroll
        for (int it = 0; it < NSV; ++it) {
            const int e4 = tid + it * NT2;
            const int i = e4 / (DK / 4), j = 4 * (e4 % (DK / 4));
            gv[it] = p.dsf ? *reinterpret_cast<const f32x4*>(p.dsf + (bh * DV + row0 + i) * DK + j)
                           : zero4;
        }
        put_s(gv, Gs);
    }
    f32x4 sv[NSV];
    fetch(x, nch - 1, true);
    fetch_s(sv, nch - 1);
    fetch_t(nch - 1);
    // nothing in flight on entry: the compiler can then count the stores
    // each chunk issues after its prefetch instead of waiting for them all
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    for (int64_t c = nch - 1; c >= 0; --c) {
        const int64_t t0 = c * C2;
        const int n = chunk_len(c);
        __syncthreads();
        put_s(sv, Ss);
        commit(x, c, true);
        commit_t();
        if (c > 0) {
            fetch(x, c - 1, true);
            fetch_s(sv, c - 1);
            fetch_t(c - 1);
        }
        __syncthreads();
        const bool wide = tables(true);
        // ---- (T from gdn2_bwd_solve)  wave 0: P and K~ G'^T rows 16..31
        //      (into dU);  wave 1: K~ G'^T rows 0..15;  waves 2, 3: R rows
        //      0..15, 16..31  (wide chunks: P entry by entry by all threads
        //      first)
        if (wide) {
            ap_entries(true);
            __syncthreads();
        }
        if (wv < 2) {
            if (wv == 0 && !wide)
                put_nn(mma16<NQK, true, true>(zero4, Qt, L::PK, Kh, L::PK), Ps, false);
            const int t = 1 - wv;
            const f32x4 acc = mma16<NQK, true, true>(zero4, Kt, L::PK, Gs + 16 * t * L::PK, L::PK);
#pragma unroll
            for (int i = 0; i < 4; ++i) dUs[(4 * lg + i) * L::PR + 16 * t + l16] = acc[i];
        } else {
            r_tile(wv - 2);
        }
        __syncthreads();
        // ---- U = T R (waves 0, 1);  dU = K~ G'^T + P^T dO (waves 2, 3);
        //      then sum_i G' (.) S per channel, DK / 4 channels per wave:
        //      lane = channel group cg (4 channels, 16-byte reads) + NG x row
        //      group, its rows summed, then the row groups by shuffles
        {
            constexpr int NG = DK / 16, RPL = NG / 2;
            const int cg = lane % NG, rg = lane / NG, c0 = DK / 4 * wv + 4 * cg;
            f32x4 sacc = zero4;
#pragma unroll
            for (int m = 0; m < RPL; ++m) {
                const int i = RPL * rg + m;
                const f32x4 gv = ld4(Gs + i * L::PK + c0), sv4 = ld4(Ss + i * L::PK + c0);
#pragma unroll
                for (int z = 0; z < 4; ++z) sacc[z] += gv[z] * sv4[z];
            }
#pragma unroll
            for (int m = NG; m < 64; m *= 2)
#pragma unroll
                for (int z = 0; z < 4; ++z) sacc[z] += __shfl_xor(sacc[z], m, 64);
            if (rg == 0) *reinterpret_cast<f32x4*>(GSc + c0) = sacc;
        }
        if (wv < 2) {
            const int t = wv;
            const f32x4 acc = mma16<1, true, false>(zero4, Ts, L::PC, Rs + 16 * t, L::PR);
#pragma unroll
            for (int i = 0; i < 4; ++i) Us[(4 * lg + i) * L::PR + 16 * t + l16] = acc[i];
        } else {
            const int t = wv - 2;
            f32x4 acc;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = dUs[(4 * lg + i) * L::PR + 16 * t + l16];
            acc = mma16<1, false, false>(acc, Ps, L::PC, dOs + 16 * t, L::PR);
#pragma unroll
            for (int i = 0; i < 4; ++i) dUs[(4 * lg + i) * L::PR + 16 * t + l16] = acc[i];
        }
        __syncthreads();
        // ---- dR = T^T dU (waves 0, 1; dw, dv to HBM);  dP = dO U^T (wave 2);
        //      dT = dU R^T and dA (wave 3)
        if (wv < 2) {
            const int t = wv;
            const f32x4 acc = mma16<1, false, false>(zero4, Ts, L::PC, dUs + 16 * t, L::PR);
            // stores past the chunk's last token are dropped by the range
            const int bytes = n * (int)(p.H * DV) * 4;
            const __amdgpu_buffer_rsrc_t rw = rsrc(p.dw + tok(t0) * DV, bytes);
            const __amdgpu_buffer_rsrc_t rv = rsrc(p.dv + tok(t0) * DV, bytes);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * lg + i, o = r * L::PR + 16 * t + l16;
                dRs[o] = acc[i];
                const int off = (r * (int)(p.H * DV) + row0 + 16 * t + l16) * 4;
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i] * Vsm[o]), rw, off, 0, 0);
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i] * Wsm[o]), rv, off, 0, 0);
            }
        } else if (wv == 2) {
            put_nn(mma16<2, true, true>(zero4, dOs, L::PR, Us, L::PR), dPs, false);
        } else {
            // dT = dU R^T, Y = dT T^T, then dA = -T^T Y (strict) over dT
            put_nn(mma16<2, true, true>(zero4, dUs, L::PR, Rs, L::PR), dTs, true);
            wave_sync();
            const f32x4 y = mma16<1, true, true>(zero4, dTs, L::PC, Ts, L::PC);
#pragma unroll
            for (int i = 0; i < 4; ++i) Ys[(4 * lg + i) * L::PC + l16] = y[i];
            wave_sync();
            put_nn(mma16<1, false, false, true>(zero4, Ts, L::PC, Ys, L::PC), dTs, true);
        }
        __syncthreads();
        // ---- this wave's channel tiles: dE~ = -dR S, dQ~ = dO S, dK~ = U G';
        //      the dP parts of dQ_P and dK_AP
        f32x4 dEt[CTW], dQt[CTW], dKt[CTW], dEa[CTW], dQa[CTW], dKa[CTW];
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) {
            const int t = CTW * wv + ct;
            dEt[ct] = mma16<2, true, false, true>(zero4, dRs, L::PR, Ss + 16 * t, L::PK);
            dQt[ct] = mma16<2, true, false>(zero4, dOs, L::PR, Ss + 16 * t, L::PK);
            dKt[ct] = mma16<2, true, false>(zero4, Us, L::PR, Gs + 16 * t, L::PK);
            if (!wide) {
                dQa[ct] = mma16<1, true, false>(zero4, dPs, L::PC, Kh + 16 * t, L::PK);
                dKa[ct] = mma16<1, false, false>(zero4, dPs, L::PC, Qt + 16 * t, L::PK);
            }
        }
        const float* dAs = dTs;
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) {
            const int t = CTW * wv + ct, cc = 16 * t + l16;
            if (!wide) {
                dEa[ct] = mma16<1, true, false>(zero4, dAs, L::PC, Kh + 16 * t, L::PK);
                dKa[ct] = mma16<1, false, false>(dKa[ct], dAs, L::PC, Et + 16 * t, L::PK);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int at = (4 * lg + i) * L::PK + cc;
                    const float lm = Lm[at];
                    dEa[ct][i] *= lm;
                    dQa[ct][i] *= lm;
                    dKa[ct][i] *= ex2(-Gc[at]);
                }
            } else {
                // entry by entry: token r = 4 lg + i, channel cc
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 4 * lg + i;
                    const float gr = Gc[r * L::PK + cc];
                    float ea = 0.f, qa = 0.f, ka = 0.f;
                    for (int s = 0; s <= r; ++s) {
                        const float kd = Ks[s * L::PK + cc] * ex2(gr - Gc[s * L::PK + cc]);
                        ea += dAs[r * L::PC + s] * kd;
                        qa += dPs[r * L::PC + s] * kd;
                    }
                    for (int r2 = r; r2 < C2; ++r2)
                        ka += (dAs[r2 * L::PC + r] * Es[r2 * L::PK + cc] +
                               dPs[r2 * L::PC + r] * Qs[r2 * L::PK + cc]) *
                              ex2(Gc[r2 * L::PK + cc] - gr);
                    dEa[ct][i] = ea;
                    dQa[ct][i] = qa;
                    dKa[ct][i] = ka;
                }
            }
            // ---- combine: dq, dk, db and d log alpha partials to HBM.
            // d log alpha_t collects, inside the chunk, the suffix sums
            // (t' >= t) of dE~ (.) E~ + dQ~ (.) Q~, the prefix sums (t' < t)
            // of dK~ (.) K~ (K~ depends on alpha_t for tokens before t), the
            // lambda_C term, and the pair terms pr = E (.) dE_A + Q (.) dQ_P
            // - K (.) dK_AP, which sum to zero over the chunk: their suffix
            // sum equals minus their prefix sum, and the half of the chunk
            // nearer each end takes the form with fewer terms (the two share
            // every pair on the far side, which would cancel in fp32).
            const float gC = Gc[(C2 - 1) * L::PK + cc], lmC = Lm[(C2 - 1) * L::PK + cc];
            float oq[4], ok[4], ob[4], pr[4], tl[4], kk4[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int at = (4 * lg + i) * L::PK + cc;
                const float lm = Lm[at], kk = Ks[at], g = Gc[at];
                const float dE = dEa[ct][i] + dEt[ct][i] * lm;
                oq[i] = dQa[ct][i] + dQt[ct][i] * lm;
                ok[i] = dKa[ct][i] + dKt[ct][i] * ex2(gC - g) + dE * Bs[at];
                ob[i] = dE * kk;
                kk4[i] = dKt[ct][i] * Kt[at];
                tl[i] = dEt[ct][i] * Et[at] + dQt[ct][i] * Qt[at];
                pr[i] = Es[at] * dEa[ct][i] + Qs[at] * dQa[ct][i] - kk * dKa[ct][i];
            }
            // totals of the four token groups of this channel (lanes l16 + 16 g)
            const float sp = pr[0] + pr[1] + pr[2] + pr[3];
            const float st = tl[0] + tl[1] + tl[2] + tl[3];
            const float sk = kk4[0] + kk4[1] + kk4[2] + kk4[3];
            float ap = 0.f, bp = 0.f, at_ = 0.f, bk = 0.f;
#pragma unroll
            for (int g2 = 0; g2 < 4; ++g2) {
                const float vp = __shfl(sp, l16 + 16 * g2, 64);
                const float vt = __shfl(st, l16 + 16 * g2, 64);
                const float vk = __shfl(sk, l16 + 16 * g2, 64);
                if (g2 > lg) { ap += vp; at_ += vt; }
                if (g2 < lg) { bp += vp; bk += vk; }
            }
            const float lam = GSc[cc] * lmC;
            float dl[4];
            {
                float sufp = ap, suft = at_, prep = bp, prek = bk;
                float pp[4], pk4[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {   // prefixes, tokens before 4 lg + i
                    pp[i] = prep;
                    pk4[i] = prek;
                    prep += pr[i];
                    prek += kk4[i];
                }
#pragma unroll
                for (int i = 3; i >= 0; --i) {  // suffixes, tokens from 4 lg + i
                    sufp += pr[i];
                    suft += tl[i];
                    dl[i] = suft + pk4[i] + lam + (lg >= 2 ? sufp : -pp[i]);
                }
            }
            // this row block's share, added by fp32 atomics in L2; tokens
            // past the chunk's end are dropped by the range
            {
                const int bytes = n * (int)(p.H * DK) * 4;
                const int64_t base = tok(t0) * DK;
                const __amdgpu_buffer_rsrc_t rq = rsrc(p.pq + base, bytes);
                const __amdgpu_buffer_rsrc_t rk = rsrc(p.pk + base, bytes);
                const __amdgpu_buffer_rsrc_t rb_ = rsrc(p.pb + base, bytes);
                const __amdgpu_buffer_rsrc_t rg = rsrc(p.pg + base, bytes);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int off = ((4 * lg + i) * (int)(p.H * DK) + cc) * 4;
                    __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(oq[i], rq, off, 0, 0);
                    __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(ok[i], rk, off, 0, 0);
                    __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(ob[i], rb_, off, 0, 0);
                    __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(dl[i], rg, off, 0, 0);
                }
            }
            // ---- G' <- G' diag(lambda_C) + dO^T Q~ - dR^T E~ on this wave's
            //      channels (only this wave reads them in this chunk)
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                f32x4 acc;
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] = Gs[(16 * a + 4 * lg + i) * L::PK + cc] * lmC;
                acc = mma16<1, false, false>(acc, dOs + 16 * a, L::PR, Qt + 16 * t, L::PK);
                acc = mma16<1, false, false, true>(acc, dRs + 16 * a, L::PR, Et + 16 * t, L::PK);
#pragma unroll
                for (int i = 0; i < 4; ++i) Gs[(16 * a + 4 * lg + i) * L::PK + cc] = acc[i];
            }
        }
    }
    __syncthreads();
    if (p.ds0) {
#pragma unroll
        for (int it = 0; it < NSV; ++it) {
            const int e4 = tid + it * NT2;
            const int i = e4 / (DK / 4), j = 4 * (e4 % (DK / 4));
            *reinterpret_cast<f32x4*>(p.ds0 + (bh * DV + row0 + i) * DK + j) =
                ld4(Gs + i * L::PK + j);
        }
    }
}

// dalpha = d log alpha / alpha, alpha clamped to FLT_MIN as in the forward's log
template <typename TIn>
__global__ __launch_bounds__(256) void bwd2_dalpha(int64_t n, const float* __restrict__ dl,
                                                   const void* alpha, float* __restrict__ da) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    da[i] = dl[i] / fmaxf(ldf<TIn>(alpha, i), 1.17549435e-38f);
}

template <int DK, int DV, typename TIn, typename TD>
hipError_t launch_main(const Bwd2Params& p, int64_t BH, hipStream_t st) {
    const size_t lds = sizeof(float) * BL3<DK>::TOTAL;
    auto fn = chunk2_bwd_kernel<DK, DV, TIn, TD>;
    hipError_t e = hipFuncSetAttribute((const void*)fn,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fn, dim3((unsigned)(BH * (DV / R2))), dim3(NT2), lds, st, p);
    return hipGetLastError();
}

template <int DK, int DV, typename TIn, typename TD>
hipError_t launch_bwd2_t(const Bwd2Args& a) {
    const int64_t BH = a.B * a.H, BTH = a.B * a.T * a.H;
    const int64_t nch = (a.T + C2 - 1) / C2;
    Bwd2Params p{};
    p.T = a.T;
    p.H = a.H;
    p.BTH = BTH;
    p.q = a.q;
    p.k = a.k;
    p.v = a.v;
    p.alpha = a.alpha;
    p.erase = a.erase;
    p.write = a.write;
    p.dout = a.dout;
    p.s0 = a.s0;
    p.dsf = a.ds_final;
    p.dv = a.dv;
    p.dw = a.dwrite;
    p.ds0 = a.ds0;
    p.ck = reinterpret_cast<float*>(a.workspace);
    float* tt = p.ck + BH * nch * DV * DK;
    p.tt = tt;
    // accumulators: dq, dk and derase go straight into the outputs unless the
    // fused norm's reverse mode follows; d log alpha always in the workspace
    float* w = tt + BH * nch * 256;
    const int64_t nqk = BTH * DK;
    p.pq = a.l2norm ? w : a.dq;
    p.pk = a.l2norm ? w + nqk : a.dk;
    p.pb = a.l2norm ? w + 2 * nqk : a.derase;
    p.pg = w + 3 * nqk;
    p.l2norm = a.l2norm;
    hipError_t e = hipSuccess;
    for (float* acc : {p.pq, p.pk, p.pb, p.pg})
        if (e == hipSuccess) e = launch_zero(acc, nqk * 4, a.stream);
    if (e != hipSuccess) return e;
    // T of every chunk first
    Solve2Params sp{};
    sp.T = a.T;
    sp.H = a.H;
    sp.nch = nch;
    sp.nchunks = BH * nch;
    sp.k = a.k;
    sp.alpha = a.alpha;
    sp.erase = a.erase;
    sp.tt = tt;
    sp.l2norm = a.l2norm;
    hipLaunchKernelGGL((gdn2_bwd_solve<DK, TIn>), dim3((unsigned)(BH * nch)), dim3(64), 0, a.stream,
                       sp);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_main<DK, DV, TIn, TD>(p, BH, a.stream);
    if (e != hipSuccess) return e;
    if (a.l2norm) {
        hipLaunchKernelGGL((bwd_reduce_rows_norm<1, DK, TIn, true>),
                           dim3((unsigned)((BTH + 3) / 4)), dim3(256), 0, a.stream, BTH, p.pq, p.pk,
                           p.pb, p.pg, a.q, a.k, a.alpha, a.dq, a.dk, a.derase, a.dalpha);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((bwd2_dalpha<TIn>), dim3((unsigned)((nqk + 255) / 256)), dim3(256), 0,
                       a.stream, nqk, p.pg, a.alpha, a.dalpha);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_bwd2_d(const Bwd2Args& a) {
    if (a.in_bf16)
        return a.dout_bf16 ? launch_bwd2_t<DK, DV, bf16_t, bf16_t>(a)
                           : launch_bwd2_t<DK, DV, bf16_t, float>(a);
    return a.dout_bf16 ? launch_bwd2_t<DK, DV, float, bf16_t>(a)
                       : launch_bwd2_t<DK, DV, float, float>(a);
}

}  // namespace

size_t bwd2_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv) {
    const int64_t nch = (T + C2 - 1) / C2;
    const int64_t nrb = Dv / R2;
    (void)nrb;
    return sizeof(float) * (size_t)(B * H * nch * Dv * Dk + B * H * nch * 256 + 4 * B * T * H * Dk);
}

hipError_t launch_chunk2_bwd(const Bwd2Args& a) {
    if (a.Dk == 128 && a.Dv == 128) return launch_bwd2_d<128, 128>(a);
    if (a.Dk == 128 && a.Dv == 64) return launch_bwd2_d<128, 64>(a);
    if (a.Dk == 64 && a.Dv == 128) return launch_bwd2_d<64, 128>(a);
    return launch_bwd2_d<64, 64>(a);
}

}  // namespace gdr
