// gdr2_chunk_bwd: reverse mode of Gated Delta Rule-2, chunk by chunk, in
// fp32 vector-ALU arithmetic.
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
// Work split as in gdr_chunk_bwd: one 256-thread workgroup per (b, h, 32
// state rows) runs the forward over its rows (chunk-start states to the
// workspace), then walks the chunks in reverse; dv, dw and dS_0 are final
// per workgroup, dq, dk, db and dG go to per-row-block partials that a
// second kernel adds (and turns dG into dalpha).  Chunks are 16 tokens so
// that the per-channel decay tables of a chunk fit in LDS beside the state.
//
// The LDS footprint allows one workgroup per CU, one wave per SIMD, so
// nothing hides memory latency but the kernel itself: every global input of
// the next chunk (key-side rows, w, v, dL/do and the chunk-start state) is
// loaded into registers as raw words while the current chunk computes, and
// written to LDS at the top of the next iteration.  Thread t owns token
// t / 16 and key channels NC (t % 16) .. + NC for the key-side loads and for
// the per-channel gradient terms, so those need no further exchange.
#include "gdr_device.h"
#include "launch.h"
#include "vtile.h"

namespace gdr {

namespace {

constexpr int C2 = 16;     // tokens per chunk
constexpr int R2 = 32;     // state rows per workgroup
constexpr int NT2 = 256;   // threads per workgroup

struct Bwd2Params {
    int64_t T, H, BTH;
    const void *q, *k, *v, *alpha, *erase, *write, *dout;
    const float *s0, *dsf;
    float *dv, *dw, *ds0;
    float* ck;                     // [BH][nch][Dv][Dk]
    float *pq, *pk, *pb, *pg;      // [NRB][BTH][Dk] each
};

template <int DK>
struct BL2 {
    static constexpr int PK = DK + 4;
    static constexpr int PC = C2 + 1;
    static constexpr int PR = R2 + 1;
    static constexpr int NK = C2 * PK;           // one token x key-dim table
    static constexpr int K = 0;
    static constexpr int Q = K + NK;
    static constexpr int E = Q + NK;             // b (.) k
    static constexpr int BB = E + NK;            // b
    static constexpr int GC = BB + NK;           // cumulative log alpha
    static constexpr int LM = GC + NK;           // lambda = e^G
    static constexpr int KT = LM + NK;           // K~
    static constexpr int QT = KT + NK;           // Q~
    static constexpr int ET = QT + NK;           // E~
    static constexpr int SCR = ET + NK;          // dK~ (.) K~ (column sums)
    static constexpr int DG = SCR + NK;          // dG partial, staged
    static constexpr int S = DG + NK;            // [R2][PK] chunk-start state rows
    static constexpr int G = S + R2 * PK;        // [R2][PK] dL/dS' rows
    static constexpr int A = G + R2 * PK;        // n x n tiles [C2][PC]
    static constexpr int TM = A + C2 * PC;
    static constexpr int P = TM + C2 * PC;
    static constexpr int DP = P + C2 * PC;
    static constexpr int DT = DP + C2 * PC;
    static constexpr int DA = DT + C2 * PC;
    static constexpr int WV = DA + C2 * PC;      // n x rows tiles [C2][PR]
    static constexpr int W = WV + C2 * PR;
    static constexpr int V = W + C2 * PR;
    static constexpr int DO = V + C2 * PR;
    static constexpr int R = DO + C2 * PR;
    static constexpr int U = R + C2 * PR;
    static constexpr int DU = U + C2 * PR;
    static constexpr int DR = DU + C2 * PR;
    static constexpr int TOTAL = DR + C2 * PR;
    static_assert(TOTAL * 4 <= 160 * 1024, "LDS budget");
    static_assert(PK % 4 == 0 && NK % 4 == 0 && S % 4 == 0 && G % 4 == 0, "16-byte rows");
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

template <int DK, int DV, typename TIn, typename TD>
__global__ __launch_bounds__(NT2) void chunk2_bwd_kernel(Bwd2Params p) {
    using L = BL2<DK>;
    constexpr int NRB = DV / R2;
    constexpr int NC = DK / 16;
    constexpr int NSV = R2 * DK / 4 / NT2;     // 16-byte state pieces per thread
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
    float* Scr = sm + L::SCR;
    float* Dg = sm + L::DG;
    float* Ss = sm + L::S;
    float* Gs = sm + L::G;
    float* As = sm + L::A;
    float* Ts = sm + L::TM;
    float* Ps = sm + L::P;
    float* dPs = sm + L::DP;
    float* dTs = sm + L::DT;
    float* dAs = sm + L::DA;
    float* WVs = sm + L::WV;
    float* Wsm = sm + L::W;
    float* Vsm = sm + L::V;
    float* dOs = sm + L::DO;
    float* Rs = sm + L::R;
    float* Us = sm + L::U;
    float* dUs = sm + L::DU;
    float* dRs = sm + L::DR;

    const int tid = threadIdx.x;
    const int rb = blockIdx.x % NRB;
    const int64_t bh = blockIdx.x / NRB;
    const int64_t h = bh % p.H;
    const int64_t b = bh / p.H;
    const int64_t T = p.T, H = p.H;
    const int row0 = rb * R2;
    const int64_t nch = (T + C2 - 1) / C2;
    float* ckb = p.ck + bh * nch * DV * DK;
    auto tok = [&](int64_t t) { return (b * T + t) * H + h; };
    const int tr = tid >> 4;                   // this thread's token in the chunk
    const int j0 = NC * (tid & 15);            // .. and its key channels
    const int i2 = 2 * (tid & 15);             // .. and its pair of state rows
    const int i0 = 2 * (tid >> 4);             // state-update tile: rows i0, i0 + 1
    auto chunk_len = [&](int64_t c) { return (int)min((int64_t)C2, T - c * C2); };

    using PF = Pre2<TIn, TD, NC>;
    auto fetch = [&](PF& x, int64_t c, bool bwd) {
        if (tr < chunk_len(c)) {
            const int64_t tk = tok(c * C2 + tr);
            const TIn* kp = reinterpret_cast<const TIn*>(p.k) + tk * DK + j0;
            ldw(x.k, kp);
            ldw(x.b, reinterpret_cast<const TIn*>(p.erase) + tk * DK + j0);
            ldw(x.a, reinterpret_cast<const TIn*>(p.alpha) + tk * DK + j0);
            if (bwd) ldw(x.q, reinterpret_cast<const TIn*>(p.q) + tk * DK + j0);
            ldw(x.w, reinterpret_cast<const TIn*>(p.write) + tk * DV + row0 + i2);
            ldw(x.v, reinterpret_cast<const TIn*>(p.v) + tk * DV + row0 + i2);
            if (bwd) ldw(x.d, reinterpret_cast<const TD*>(p.dout) + tk * DV + row0 + i2);
        }
    };
    // rows >= n: zero tokens with alpha = 1
    auto commit = [&](const PF& x, int64_t c, bool bwd) {
        const bool live = tr < chunk_len(c);
        const int at = tr * L::PK + j0;
#pragma unroll
        for (int y0 = 0; y0 < NC; y0 += 4) {
            f32x4 kv, bv, ev, gv, qv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int y = y0 + e;
                kv[e] = live ? packed<TIn>::at(x.k, y) : 0.f;
                bv[e] = live ? packed<TIn>::at(x.b, y) : 0.f;
                ev[e] = bv[e] * kv[e];
                gv[e] = live ? safe_log(packed<TIn>::at(x.a, y)) : 0.f;
                qv[e] = (live && bwd) ? packed<TIn>::at(x.q, y) : 0.f;
            }
            *reinterpret_cast<f32x4*>(Ks + at + y0) = kv;
            *reinterpret_cast<f32x4*>(Bs + at + y0) = bv;
            *reinterpret_cast<f32x4*>(Es + at + y0) = ev;
            *reinterpret_cast<f32x4*>(Gc + at + y0) = gv;
            if (bwd) *reinterpret_cast<f32x4*>(Qs + at + y0) = qv;
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const float wv = live ? packed<TIn>::at(x.w, e) : 0.f;
            const float vv = live ? packed<TIn>::at(x.v, e) : 0.f;
            const int o = tr * L::PR + i2 + e;
            WVs[o] = wv * vv;
            Wsm[o] = wv;
            Vsm[o] = vv;
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
    // after a barrier: G by a scan down the tokens per channel, then the
    // decay tables (two barriers inside)
    auto tables = [&](bool bwd) {
        if (tid < DK) {
            float g[C2];
#pragma unroll
            for (int r = 0; r < C2; ++r) g[r] = Gc[r * L::PK + tid];
#pragma unroll
            for (int r = 1; r < C2; ++r) g[r] += g[r - 1];
#pragma unroll
            for (int r = 0; r < C2; ++r) Gc[r * L::PK + tid] = g[r];
        }
        __syncthreads();
        {
            const int at = tr * L::PK + j0;
#pragma unroll
            for (int y0 = 0; y0 < NC; y0 += 4) {
                const f32x4 g = ld4(Gc + at + y0), gC = ld4(Gc + (C2 - 1) * L::PK + j0 + y0);
                const f32x4 k = ld4(Ks + at + y0), e = ld4(Es + at + y0);
                f32x4 lm, kt, et, qt;
#pragma unroll
                for (int z = 0; z < 4; ++z) {
                    lm[z] = __expf(g[z]);
                    kt[z] = k[z] * __expf(gC[z] - g[z]);
                    et[z] = e[z] * lm[z];
                }
                *reinterpret_cast<f32x4*>(Lm + at + y0) = lm;
                *reinterpret_cast<f32x4*>(Kt + at + y0) = kt;
                *reinterpret_cast<f32x4*>(Et + at + y0) = et;
                if (bwd) {
                    const f32x4 q = ld4(Qs + at + y0);
#pragma unroll
                    for (int z = 0; z < 4; ++z) qt[z] = q[z] * lm[z];
                    *reinterpret_cast<f32x4*>(Qt + at + y0) = qt;
                }
            }
        }
        __syncthreads();
    };
    // A (s < r) and P (s <= r), the decay inside the dot product; R = w.v - E~ S^T
    auto form_ap_r = [&](bool bwd) {
        {
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
                        const float kd = ks[z] * __expf(gr[z] - gs[z]);
                        av += er[z] * kd;
                        pv += qr[z] * kd;
                    }
                }
            }
            As[r * L::PC + s] = s < r ? av : 0.f;
            if (bwd) Ps[r * L::PC + s] = pv;
        }
#pragma unroll
        for (int it = 0; it < C2 * R2 / NT2; ++it) {
            const int e = tid + it * NT2;
            const int r = e / R2, i = e % R2;
            float x = 0.f;
#pragma unroll 8
            for (int c = 0; c < DK; c += 4) {
                const f32x4 a = ld4(Et + r * L::PK + c), sv = ld4(Ss + i * L::PK + c);
                x += a[0] * sv[0] + a[1] * sv[1] + a[2] * sv[2] + a[3] * sv[3];
            }
            Rs[r * L::PR + i] = WVs[r * L::PR + i] - x;
        }
    };

    PF x;
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
            for (int it = 0; it < NSV; ++it) sv[it] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        put_s(sv, Ss);
    }
    fetch(x, 0, false);
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
        if (c + 1 < nch) fetch(x, c + 1, false);
        __syncthreads();
        tables(false);
        form_ap_r(false);
        __syncthreads();
        // (I + A) U = R by forward substitution, one thread per state row
        if (tid < R2) {
            const int i = tid;
            float u[C2];
#pragma unroll
            for (int r = 0; r < C2; ++r) {
                float v = Rs[r * L::PR + i];
#pragma unroll
                for (int s = 0; s < r; ++s) v -= As[r * L::PC + s] * u[s];
                u[r] = v;
                Us[r * L::PR + i] = v;
            }
        }
        __syncthreads();
        // S <- S diag(lambda_C) + U^T K~ (each thread rewrites only what it read)
        {
            float acc[2][NC];
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int y = 0; y < NC; ++y)
                    acc[a][y] = Ss[(i0 + a) * L::PK + j0 + y] * Lm[(C2 - 1) * L::PK + j0 + y];
            mm2n<C2, NC>(acc, [&](int a, int r) { return Us[r * L::PR + i0 + a]; }, Kt, L::PK, j0);
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int y = 0; y < NC; ++y) Ss[(i0 + a) * L::PK + j0 + y] = acc[a][y];
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
                           : f32x4{0.f, 0.f, 0.f, 0.f};
        }
        put_s(gv, Gs);
    }
    const int64_t poff = (int64_t)rb * p.BTH * DK;
    f32x4 sv[NSV];
    fetch(x, nch - 1, true);
    fetch_s(sv, nch - 1);
    for (int64_t c = nch - 1; c >= 0; --c) {
        const int64_t t0 = c * C2;
        const int n = chunk_len(c);
        __syncthreads();
        put_s(sv, Ss);
        commit(x, c, true);
        if (c > 0) {
            fetch(x, c - 1, true);
            fetch_s(sv, c - 1);
        }
        __syncthreads();
        tables(true);
        form_ap_r(true);
        __syncthreads();
        // T = (I + A)^{-1}, one thread per column, the column in registers
        if (tid < C2) {
            const int cc = tid;
            float tc[C2];
#pragma unroll
            for (int r = 0; r < C2; ++r) {
                float v = r == cc ? 1.f : 0.f;
#pragma unroll
                for (int m = 0; m < r; ++m) v -= As[r * L::PC + m] * tc[m];
                tc[r] = r < cc ? 0.f : v;
                Ts[r * L::PC + cc] = tc[r];
            }
        }
        __syncthreads();
        // U = T R;  dU = P^T dO + K~ G'^T
#pragma unroll
        for (int it = 0; it < C2 * R2 / NT2; ++it) {
            const int e = tid + it * NT2;
            const int r = e / R2, i = e % R2;
            float u = 0.f, du = 0.f;
            for (int s = 0; s <= r; ++s) u += Ts[r * L::PC + s] * Rs[s * L::PR + i];
            for (int s = r; s < C2; ++s) du += Ps[s * L::PC + r] * dOs[s * L::PR + i];
#pragma unroll 8
            for (int cc = 0; cc < DK; cc += 4) {
                const f32x4 kt = ld4(Kt + r * L::PK + cc), gv = ld4(Gs + i * L::PK + cc);
                du += kt[0] * gv[0] + kt[1] * gv[1] + kt[2] * gv[2] + kt[3] * gv[3];
            }
            Us[r * L::PR + i] = u;
            dUs[r * L::PR + i] = du;
        }
        __syncthreads();
        // dR = T^T dU (dw = dR (.) v, dv = dR (.) w to HBM);  dP = dO U^T (s <= r)
#pragma unroll
        for (int it = 0; it < C2 * R2 / NT2; ++it) {
            const int e = tid + it * NT2;
            const int r = e / R2, i = e % R2;
            float v = 0.f;
            for (int s = r; s < C2; ++s) v += Ts[s * L::PC + r] * dUs[s * L::PR + i];
            dRs[r * L::PR + i] = v;
            if (r < n) {
                const int64_t off = tok(t0 + r) * DV + row0 + i;
                p.dw[off] = v * Vsm[r * L::PR + i];
                p.dv[off] = v * Wsm[r * L::PR + i];
            }
        }
        {
            const int r = tid >> 4, s = tid & 15;
            float v = 0.f;
            if (s <= r) {
#pragma unroll 8
                for (int i = 0; i < R2; ++i) v += dOs[r * L::PR + i] * Us[s * L::PR + i];
            }
            dPs[r * L::PC + s] = v;
        }
        __syncthreads();
        {   // dT = dU R^T, strict lower
            const int r = tid >> 4, s = tid & 15;
            float v = 0.f;
            if (s < r) {
#pragma unroll 8
                for (int i = 0; i < R2; ++i) v += dUs[r * L::PR + i] * Rs[s * L::PR + i];
            }
            dTs[r * L::PC + s] = v;
        }
        __syncthreads();
        {   // Y = dT T^T into dA's tile
            const int r = tid >> 4, s = tid & 15;
            float v = 0.f;
            for (int bb = 0; bb <= s && bb < r; ++bb) v += dTs[r * L::PC + bb] * Ts[s * L::PC + bb];
            dAs[r * L::PC + s] = v;
        }
        __syncthreads();
        {   // dA = -T^T Y, strict lower, into dT's tile
            const int r = tid >> 4, s = tid & 15;
            float v = 0.f;
            if (s < r)
                for (int a = r; a < C2; ++a) v -= Ts[a * L::PC + r] * dAs[a * L::PC + s];
            dTs[r * L::PC + s] = v;
        }
        __syncthreads();
        const float* dA = dTs;
        // ---- per (token tr, channels j0 .. j0 + NC - 1)
        {
            const int r = tr;
            float dEt[NC] = {}, dQt[NC] = {}, dKt[NC] = {};
            mm1n<R2, NC>(dEt, [&](int i) { return -dRs[r * L::PR + i]; }, Ss, L::PK, j0);
            mm1n<R2, NC>(dQt, [&](int i) { return dOs[r * L::PR + i]; }, Ss, L::PK, j0);
            mm1n<R2, NC>(dKt, [&](int i) { return Us[r * L::PR + i]; }, Gs, L::PK, j0);
            float gr[NC];
#pragma unroll
            for (int y0 = 0; y0 < NC; y0 += 4) {
                const f32x4 g = ld4(Gc + r * L::PK + j0 + y0);
#pragma unroll
                for (int z = 0; z < 4; ++z) gr[y0 + z] = g[z];
            }
            float dEa[NC] = {}, dQa[NC] = {}, dKa[NC] = {};
            for (int s = 0; s <= r; ++s) {
                const float da = dA[r * L::PC + s], dp = dPs[r * L::PC + s];
#pragma unroll
                for (int y0 = 0; y0 < NC; y0 += 4) {
                    const f32x4 ks = ld4(Ks + s * L::PK + j0 + y0), gs = ld4(Gc + s * L::PK + j0 + y0);
#pragma unroll
                    for (int z = 0; z < 4; ++z) {
                        const float kd = ks[z] * __expf(gr[y0 + z] - gs[z]);
                        dEa[y0 + z] += da * kd;
                        dQa[y0 + z] += dp * kd;
                    }
                }
            }
            for (int r2 = r; r2 < C2; ++r2) {
                const float da = dA[r2 * L::PC + r], dp = dPs[r2 * L::PC + r];
#pragma unroll
                for (int y0 = 0; y0 < NC; y0 += 4) {
                    const f32x4 g2 = ld4(Gc + r2 * L::PK + j0 + y0);
                    const f32x4 e2 = ld4(Es + r2 * L::PK + j0 + y0), q2 = ld4(Qs + r2 * L::PK + j0 + y0);
#pragma unroll
                    for (int z = 0; z < 4; ++z)
                        dKa[y0 + z] += (da * e2[z] + dp * q2[z]) * __expf(g2[z] - gr[y0 + z]);
                }
            }
            float oq[NC], ok[NC], ob[NC];
#pragma unroll
            for (int y0 = 0; y0 < NC; y0 += 4) {
                const int at = r * L::PK + j0 + y0;
                const f32x4 lm = ld4(Lm + at), ks = ld4(Ks + at), bs = ld4(Bs + at);
                const f32x4 es = ld4(Es + at), qs = ld4(Qs + at), kt = ld4(Kt + at);
                const f32x4 et = ld4(Et + at), qt = ld4(Qt + at);
                const f32x4 gC = ld4(Gc + (C2 - 1) * L::PK + j0 + y0);
                f32x4 scr, dg;
#pragma unroll
                for (int z = 0; z < 4; ++z) {
                    const int y = y0 + z;
                    const float dE = dEa[y] + dEt[y] * lm[z];
                    oq[y] = dQa[y] + dQt[y] * lm[z];
                    const float kdec = __expf(gC[z] - gr[y]);
                    ok[y] = dKa[y] + dKt[y] * kdec + dE * bs[z];
                    ob[y] = dE * ks[z];
                    const float ktk = dKt[y] * kt[z];
                    scr[z] = ktk;
                    dg[z] = es[z] * dEa[y] + qs[z] * dQa[y] - ks[z] * dKa[y] + dEt[y] * et[z] +
                            dQt[y] * qt[z] - ktk;
                }
                *reinterpret_cast<f32x4*>(Scr + at) = scr;
                *reinterpret_cast<f32x4*>(Dg + at) = dg;
            }
            if (r < n) {
                const int64_t o = poff + tok(t0 + r) * DK + j0;
#pragma unroll
                for (int hh = 0; hh < NC / 4; ++hh) {
                    *reinterpret_cast<f32x4*>(p.pq + o + 4 * hh) =
                        f32x4{oq[4 * hh], oq[4 * hh + 1], oq[4 * hh + 2], oq[4 * hh + 3]};
                    *reinterpret_cast<f32x4*>(p.pk + o + 4 * hh) =
                        f32x4{ok[4 * hh], ok[4 * hh + 1], ok[4 * hh + 2], ok[4 * hh + 3]};
                    *reinterpret_cast<f32x4*>(p.pb + o + 4 * hh) =
                        f32x4{ob[4 * hh], ob[4 * hh + 1], ob[4 * hh + 2], ob[4 * hh + 3]};
                }
            }
        }
        __syncthreads();
        // ---- dG: the last live token takes sum_r dK~ (.) K~ and (sum_i G' (.) S) (.) lambda_C
        //      (padding tokens have log alpha = 0, so G_C is the last live token's G)
        if (tid < DK) {
            const int cc = tid;
            float cs = 0.f, gs2 = 0.f;
#pragma unroll
            for (int r = 0; r < C2; ++r) cs += Scr[r * L::PK + cc];
#pragma unroll 8
            for (int i = 0; i < R2; ++i) gs2 += Gs[i * L::PK + cc] * Ss[i * L::PK + cc];
            Dg[(n - 1) * L::PK + cc] += cs + gs2 * Lm[(C2 - 1) * L::PK + cc];
        }
        __syncthreads();
        if (tr < n) {
            const int64_t o = poff + tok(t0 + tr) * DK + j0;
#pragma unroll
            for (int y0 = 0; y0 < NC; y0 += 4)
                *reinterpret_cast<f32x4*>(p.pg + o + y0) = ld4(Dg + tr * L::PK + j0 + y0);
        }
        // ---- G' <- G' diag(lambda_C) + dO^T Q~ - dR^T E~ (each thread its own entries)
        {
            float acc[2][NC];
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int y = 0; y < NC; ++y)
                    acc[a][y] = Gs[(i0 + a) * L::PK + j0 + y] * Lm[(C2 - 1) * L::PK + j0 + y];
            mm2n<C2, NC>(acc, [&](int a, int r) { return dOs[r * L::PR + i0 + a]; }, Qt, L::PK, j0);
            mm2n<C2, NC>(acc, [&](int a, int r) { return -dRs[r * L::PR + i0 + a]; }, Et, L::PK, j0);
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int y = 0; y < NC; ++y) Gs[(i0 + a) * L::PK + j0 + y] = acc[a][y];
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

// dq, dk, derase: the sum of the row blocks' partials
template <int NRB>
__global__ __launch_bounds__(256) void bwd2_reduce_qkb(int64_t n, const float* __restrict__ pq,
                                                       const float* __restrict__ pk,
                                                       const float* __restrict__ pb,
                                                       float* __restrict__ dq, float* __restrict__ dk,
                                                       float* __restrict__ db) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    float a = 0.f, b = 0.f, c = 0.f;
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
        a += pq[r * n + i];
        b += pk[r * n + i];
        c += pb[r * n + i];
    }
    dq[i] = a;
    dk[i] = b;
    db[i] = c;
}

// dalpha: one thread per (b, h, chunk, channel); dlog alpha is the reverse
// cumulative sum of dG inside the chunk, dalpha = dlog alpha / alpha (alpha
// clamped to FLT_MIN as in the forward's logarithm)
template <int NRB, typename TIn>
__global__ __launch_bounds__(256) void bwd2_reduce_alpha(int64_t B, int64_t T, int64_t H, int DK,
                                                         int64_t BTH, const float* __restrict__ pg,
                                                         const void* alpha, float* __restrict__ da) {
    const int64_t nch = (T + C2 - 1) / C2;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= B * H * nch * DK) return;
    const int cc = (int)(idx % DK);
    const int64_t rest = idx / DK;
    const int64_t c = rest % nch, bh = rest / nch;
    const int64_t h = bh % H, b = bh / H;
    const int64_t t0 = c * C2, t1 = min(t0 + C2, T);
    float acc = 0.f;
    for (int64_t t = t1 - 1; t >= t0; --t) {
        const int64_t i = ((b * T + t) * H + h) * DK + cc;
        float g = 0.f;
#pragma unroll
        for (int r = 0; r < NRB; ++r) g += pg[r * BTH * DK + i];
        acc += g;
        da[i] = acc / fmaxf(ldf<TIn>(alpha, i), 1.17549435e-38f);
    }
}

template <int DK, int DV, typename TIn, typename TD>
hipError_t launch_bwd2_t(const Bwd2Args& a) {
    constexpr int NRB = DV / R2;
    const int64_t BH = a.B * a.H, BTH = a.B * a.T * a.H;
    const int64_t nch = (a.T + C2 - 1) / C2;
    Bwd2Params p;
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
    float* ws = reinterpret_cast<float*>(a.workspace);
    p.ck = ws;
    p.pq = p.ck + BH * nch * DV * DK;
    p.pk = p.pq + NRB * BTH * DK;
    p.pb = p.pk + NRB * BTH * DK;
    p.pg = p.pb + NRB * BTH * DK;
    const size_t lds = sizeof(float) * BL2<DK>::TOTAL;
    auto fn = chunk2_bwd_kernel<DK, DV, TIn, TD>;
    hipError_t e = hipFuncSetAttribute((const void*)fn,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fn, dim3((unsigned)(BH * NRB)), dim3(NT2), lds, a.stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nqk = BTH * DK;
    hipLaunchKernelGGL((bwd2_reduce_qkb<NRB>), dim3((unsigned)((nqk + 255) / 256)), dim3(256), 0,
                       a.stream, nqk, p.pq, p.pk, p.pb, a.dq, a.dk, a.derase);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t na = BH * nch * DK;
    hipLaunchKernelGGL((bwd2_reduce_alpha<NRB, TIn>), dim3((unsigned)((na + 255) / 256)), dim3(256),
                       0, a.stream, a.B, a.T, a.H, (int)DK, BTH, p.pg, a.alpha, a.dalpha);
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
    return sizeof(float) * (size_t)(B * H * nch * Dv * Dk + 4 * nrb * B * T * H * Dk);
}

hipError_t launch_chunk2_bwd(const Bwd2Args& a) {
    if (a.Dk == 128 && a.Dv == 128) return launch_bwd2_d<128, 128>(a);
    if (a.Dk == 128 && a.Dv == 64) return launch_bwd2_d<128, 64>(a);
    if (a.Dk == 64 && a.Dv == 128) return launch_bwd2_d<64, 128>(a);
    return launch_bwd2_d<64, 64>(a);
}

}  // namespace gdr
