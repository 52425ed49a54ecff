// gdr_chunk_bwd: reverse mode of the scalar-gate rule, chunk by chunk, in
// fp32 vector-ALU arithmetic.
//
// Per chunk of n <= 32 tokens (g the within-chunk cumulative log alpha,
// gamma = e^g, D_r = e^{g_C - g_r}, Gamma_rs = e^{g_r - g_s}; the forward of
// gdr_chunk_fwd written with R = diag(beta) V - W S^T, W = diag(beta gamma) K,
// U = T R the new values, P the decayed Q K^T incl. its diagonal):
//
//   O  = diag(gamma) Q S^T + P U,   S' = gamma_C S + U^T diag(D) K
//
// the gradients, G = dL/dS' carried back from the next chunk, are
//
//   dU = P^T dO + diag(D) K G^T        dR = T^T dU       dV = diag(beta) dR
//   dP = dO U^T (s <= r)               dT = dU R^T       dA = -T^T dT T^T (s < r)
//   dW = -dR S
//   dQ = diag(gamma) dO S + (dP o Gamma) K
//   dK = diag(D) U G + (dP o Gamma)^T Q + diag(beta gamma) dW
//        + diag(beta) (dA o Gamma) K + (diag(beta) (dA o Gamma))^T K
//   dS = gamma_C G + dO^T diag(gamma) Q - dR^T W      (G of the chunk before)
//
// and dbeta, dg collect every place beta, gamma, Gamma, D and gamma_C enter;
// dlog alpha is the reverse cumulative sum of dg inside the chunk.  (This is
// the chain rule through the chunkwise form of the rule from "Gated Delta
// Networks" (agihunt.info, "Method") and the GDN review on
// meaningful96.github.io, section 3.7; the GDN-2 summary's remark that a
// chunked backward carries the gates inside its dot products is visible in
// the Gamma and D factors.)
//
// Work split: one 256-thread workgroup per (b, h, 32 state rows).  Rows of S
// and of G evolve independently given the key side, so dV and dS_0 are
// final per workgroup; dQ, dK, dbeta and dg are sums over the value rows,
// linear in each workgroup's share: every workgroup writes its partial, and
// a second kernel adds the Dv / 32 partials and forms dalpha.  The
// workgroup first runs the forward over its rows, writing the chunk-start
// states to the workspace, then walks the chunks in reverse, recomputing
// the chunk's A, T, R, U and P from the stored state.
#include "gdr_device.h"
#include "launch.h"
#include "vtile.h"

namespace gdr {

namespace {

constexpr int BC = 32;    // tokens per chunk
constexpr int BR = 32;    // state rows per workgroup
constexpr int BNT = 256;  // threads per workgroup

struct BwdParams {
    int64_t T, H, BH, BTH;
    const void *q, *k, *v, *dout;
    const float *alpha, *beta, *s0, *dsf;
    float *dv, *ds0;
    float* ck;                         // [BH][nch][Dv][Dk]
    float *pq, *pk, *pb, *pg;          // [NRB][BTH][Dk] x2, [NRB][BTH] x2
};

template <int DK>
struct BL {
    static constexpr int PK = DK + 4;            // 16-byte rows for vector reads
    static constexpr int PC = BC + 1;
    static constexpr int PR = BR + 1;
    static constexpr int K = 0;                  // [BC][PK]
    static constexpr int Q = K + BC * PK;        // [BC][PK]
    static constexpr int S = Q + BC * PK;        // [BR][PK] chunk-start state rows
    static constexpr int G = S + BR * PK;        // [BR][PK] dL/dS' rows
    static constexpr int KK = G + BR * PK;       // n x n tiles [BC][PC]
    static constexpr int QK = KK + BC * PC;
    static constexpr int A = QK + BC * PC;
    static constexpr int TM = A + BC * PC;
    static constexpr int P = TM + BC * PC;
    static constexpr int DP = P + BC * PC;
    static constexpr int DT = DP + BC * PC;
    static constexpr int DA = DT + BC * PC;
    static constexpr int V = DA + BC * PC;       // n x rows tiles [BC][PR]
    static constexpr int DO = V + BC * PR;
    static constexpr int KS = DO + BC * PR;
    static constexpr int QS = KS + BC * PR;
    static constexpr int KG = QS + BC * PR;
    static constexpr int R = KG + BC * PR;
    static constexpr int U = R + BC * PR;
    static constexpr int DU = U + BC * PR;
    static constexpr int DR = DU + BC * PR;
    static constexpr int GM = DR + BC * PR;      // [BC][PC] Gamma_rs = e^{min(g_r - g_s, 0)}
    static constexpr int GG = GM + BC * PC;      // [BC] g
    static constexpr int BE = GG + BC;           // [BC] beta
    static constexpr int GA = BE + BC;           // [BC] gamma = e^g
    static constexpr int DD = GA + BC;           // [BC] D = e^{g_C - g}
    static constexpr int RED = DD + BC;          // [BC][8] row reductions
    static constexpr int MISC = RED + BC * 8;    // [8]
    static constexpr int TOTAL = MISC + 8;
    static_assert(TOTAL * 4 <= 160 * 1024, "LDS budget");
    static_assert(PK % 4 == 0 && Q % 4 == 0 && S % 4 == 0 && G % 4 == 0, "16-byte rows");
};

template <int DK, int DV, typename TIn, typename TD>
__global__ __launch_bounds__(BNT) void chunk_bwd_kernel(BwdParams p) {
    using L = BL<DK>;
    constexpr int NRB = DV / BR;
    extern __shared__ __align__(16) float sm[];
    float* Ks = sm + L::K;
    float* Qs = sm + L::Q;
    float* Ss = sm + L::S;
    float* Gs = sm + L::G;
    float* KKs = sm + L::KK;
    float* QKs = sm + L::QK;
    float* As = sm + L::A;
    float* Ts = sm + L::TM;
    float* Ps = sm + L::P;
    float* dPs = sm + L::DP;
    float* dTs = sm + L::DT;
    float* dAs = sm + L::DA;
    float* Vs = sm + L::V;
    float* dOs = sm + L::DO;
    float* KSs = sm + L::KS;
    float* QSs = sm + L::QS;
    float* KGs = sm + L::KG;
    float* Rs = sm + L::R;
    float* Us = sm + L::U;
    float* dUs = sm + L::DU;
    float* dRs = sm + L::DR;
    float* gs = sm + L::GG;
    float* bes = sm + L::BE;
    float* gms = sm + L::GM;
    float* gas = sm + L::GA;
    float* dds = sm + L::DD;
    float* red = sm + L::RED;
    float* misc = sm + L::MISC;

    const int tid = threadIdx.x;
    const int rb = blockIdx.x % NRB;
    const int64_t bh = blockIdx.x / NRB;
    const int64_t h = bh % p.H;
    const int64_t b = bh / p.H;
    const int64_t T = p.T, H = p.H;
    const int row0 = rb * BR;
    const int64_t nch = (T + BC - 1) / BC;
    float* ckb = p.ck + bh * nch * DV * DK;

    auto tok = [&](int64_t t) { return (b * T + t) * H + h; };   // token-head index

    // ---- chunk inputs into LDS (rows >= n: zero tokens, alpha = 1, beta = 0)
    auto load_chunk = [&](int64_t t0, int n, bool with_q) {
        for (int e = tid; e < BC * DK; e += BNT) {
            const int r = e / DK, j = e % DK;
            float kv = 0.f, qv = 0.f;
            if (r < n) {
                kv = ldf<TIn>(p.k, tok(t0 + r) * DK + j);
                if (with_q) qv = ldf<TIn>(p.q, tok(t0 + r) * DK + j);
            }
            Ks[r * L::PK + j] = kv;
            if (with_q) Qs[r * L::PK + j] = qv;
        }
        for (int e = tid; e < BC * BR; e += BNT) {
            const int r = e / BR, i = e % BR;
            float vv = 0.f, dov = 0.f;
            if (r < n) {
                vv = ldf<TIn>(p.v, tok(t0 + r) * DV + row0 + i);
                if (with_q) dov = ldf<TD>(p.dout, tok(t0 + r) * DV + row0 + i);
            }
            Vs[r * L::PR + i] = vv;
            if (with_q) dOs[r * L::PR + i] = dov;
        }
        if (tid < 64) {
            // g = within-chunk cumulative log alpha by a wave scan; beta
            const int r = tid;
            float lg = 0.f, be = 0.f;
            if (r < n) {
                lg = safe_log(p.alpha[tok(t0 + r)]);
                be = p.beta[tok(t0 + r)];
            }
#pragma unroll
            for (int m = 1; m < 64; m <<= 1) {
                const float x = __shfl_up(lg, m, 64);
                if (tid >= m) lg += x;
            }
            if (r < BC) {
                gs[r] = lg;
                bes[r] = be;
            }
        }
    };
    // the chunk's decay tables (after load_chunk and a barrier)
    auto tables = [&]() {
        for (int e = tid; e < BC * BC; e += BNT) {
            const int r = e / BC, c = e % BC;
            gms[r * L::PC + c] = __expf(fminf(gs[r] - gs[c], 0.f));
        }
        if (tid < BC) {
            gas[tid] = __expf(gs[tid]);
            dds[tid] = __expf(gs[BC - 1] - gs[tid]);
        }
    };
    auto Gam = [&](int r, int c) { return gms[r * L::PC + c]; };

    // KK (and QK) = K K^T (Q K^T) over the key dim
    // 32 x 32 products over the key dim: thread = 2 x 2 tile (rows r0, r0 + 1;
    // columns c0, c0 + 1)
    const int r0 = 2 * (tid >> 4), c0 = 2 * (tid & 15);
    auto put22 = [&](float* D, int pd, const float (&c)[2][2]) {
        D[r0 * pd + c0] = c[0][0];
        D[r0 * pd + c0 + 1] = c[0][1];
        D[(r0 + 1) * pd + c0] = c[1][0];
        D[(r0 + 1) * pd + c0 + 1] = c[1][1];
    };
    auto gram = [&](bool with_q) {
        float c[2][2];
        dot22<DK>(Ks, L::PK, r0, Ks, L::PK, c0, c);
        put22(KKs, L::PC, c);
        if (with_q) {
            dot22<DK>(Qs, L::PK, r0, Ks, L::PK, c0, c);
            put22(QKs, L::PC, c);
        }
    };
    // X S^T for X = K (and Q): [BC][rows]
    auto xs = [&](bool with_q) {
        float c[2][2];
        dot22<DK>(Ks, L::PK, r0, Ss, L::PK, c0, c);
        put22(KSs, L::PR, c);
        if (with_q) {
            dot22<DK>(Qs, L::PK, r0, Ss, L::PK, c0, c);
            put22(QSs, L::PR, c);
        }
    };
    // [rows] x DK tiles: thread = rows 2 (tid / 16), +1; columns NC (tid % 16) .. + NC - 1
    constexpr int NC = DK / 16;
    const int i0 = 2 * (tid >> 4), j0 = NC * (tid & 15);
    // A (strict lower), R = beta V - beta gamma K S^T
    auto form_a_r = [&]() {
        for (int e = tid; e < BC * BC; e += BNT) {
            const int r = e / BC, s = e % BC;
            As[r * L::PC + s] = s < r ? bes[r] * Gam(r, s) * KKs[r * L::PC + s] : 0.f;
        }
        for (int e = tid; e < BC * BR; e += BNT) {
            const int r = e / BR, i = e % BR;
            Rs[r * L::PR + i] = bes[r] * (Vs[r * L::PR + i] - gas[r] * KSs[r * L::PR + i]);
        }
    };

    // ======================= forward: chunk-start states =====================
    for (int e = tid; e < BR * DK; e += BNT) {
        const int i = e / DK, j = e % DK;
        Ss[i * L::PK + j] = p.s0 ? p.s0[(bh * DV + row0 + i) * DK + j] : 0.f;
    }
    for (int64_t c = 0; c < nch; ++c) {
        const int64_t t0 = c * BC;
        const int n = (int)min((int64_t)BC, T - t0);
        __syncthreads();
        for (int e = tid; e < BR * DK; e += BNT) {
            const int i = e / DK, j = e % DK;
            ckb[(c * DV + row0 + i) * DK + j] = Ss[i * L::PK + j];
        }
        load_chunk(t0, n, false);
        __syncthreads();
        tables();
        gram(false);
        xs(false);
        __syncthreads();
        form_a_r();
        __syncthreads();
        // (I + A) U = R by forward substitution, one thread per state row,
        // the row's column of U in registers
        if (tid < BR) {
            const int i = tid;
            float u[BC];
#pragma unroll
            for (int r = 0; r < BC; ++r) {
                float x = Rs[r * L::PR + i];
#pragma unroll
                for (int c = 0; c < r; ++c) x -= As[r * L::PC + c] * u[c];
                u[r] = x;
                Us[r * L::PR + i] = x;
            }
        }
        __syncthreads();
        // S <- gamma_C S + U^T diag(D) K
        const float gCe = __expf(gs[BC - 1]);
        {
            float acc[2][NC];
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int y = 0; y < NC; ++y) acc[x][y] = gCe * Ss[(i0 + x) * L::PK + j0 + y];
            mm2n<BC, NC>(acc, [&](int x, int r) { return dds[r] * Us[r * L::PR + i0 + x]; }, Ks, L::PK, j0);
            // each thread rewrites only the S entries it read
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int y = 0; y < NC; ++y) Ss[(i0 + x) * L::PK + j0 + y] = acc[x][y];
        }
    }

    // ======================= reverse sweep ====================================
    __syncthreads();
    for (int e = tid; e < BR * DK; e += BNT) {
        const int i = e / DK, j = e % DK;
        Gs[i * L::PK + j] = p.dsf ? p.dsf[(bh * DV + row0 + i) * DK + j] : 0.f;
    }
    float* pqb = p.pq + (int64_t)rb * p.BTH * DK;
    float* pkb = p.pk + (int64_t)rb * p.BTH * DK;
    float* pbb = p.pb + (int64_t)rb * p.BTH;
    float* pgb = p.pg + (int64_t)rb * p.BTH;
    for (int64_t c = nch - 1; c >= 0; --c) {
        const int64_t t0 = c * BC;
        const int n = (int)min((int64_t)BC, T - t0);
        __syncthreads();
        for (int e = tid; e < BR * DK; e += BNT) {
            const int i = e / DK, j = e % DK;
            Ss[i * L::PK + j] = ckb[(c * DV + row0 + i) * DK + j];
        }
        load_chunk(t0, n, true);
        __syncthreads();
        tables();
        gram(true);
        xs(true);
        // K G^T [BC][rows]
        {
            float c[2][2];
            dot22<DK>(Ks, L::PK, r0, Gs, L::PK, c0, c);
            put22(KGs, L::PR, c);
        }
        __syncthreads();
        form_a_r();
        for (int e = tid; e < BC * BC; e += BNT) {
            const int r = e / BC, s = e % BC;
            Ps[r * L::PC + s] = s <= r ? Gam(r, s) * QKs[r * L::PC + s] : 0.f;
        }
        __syncthreads();
        // T = (I + A)^{-1}, one thread per column c: T_rc = -sum_{c<=m<r} A_rm T_mc,
        // the column in registers (entries above the diagonal are zero)
        if (tid < BC) {
            const int c = tid;
            float tc[BC];
#pragma unroll
            for (int r = 0; r < BC; ++r) {
                float x = r == c ? 1.f : 0.f;
#pragma unroll
                for (int m = 0; m < r; ++m) x -= As[r * L::PC + m] * tc[m];
                tc[r] = r < c ? 0.f : x;
                Ts[r * L::PC + c] = tc[r];
            }
        }
        __syncthreads();
        // U = T R;  dU = P^T dO + diag(D) K G^T
        const float gCe = __expf(gs[BC - 1]);
        for (int e = tid; e < BC * BR; e += BNT) {
            const int r = e / BR, i = e % BR;
            float u = 0.f, du = dds[r] * KGs[r * L::PR + i];
            for (int s = 0; s <= r; ++s) u += Ts[r * L::PC + s] * Rs[s * L::PR + i];
            for (int s = r; s < BC; ++s) du += Ps[s * L::PC + r] * dOs[s * L::PR + i];
            Us[r * L::PR + i] = u;
            dUs[r * L::PR + i] = du;
        }
        __syncthreads();
        // dR = T^T dU (and dV = beta dR to HBM);  dP = dO U^T (s <= r)
        for (int e = tid; e < BC * BR; e += BNT) {
            const int r = e / BR, i = e % BR;
            float x = 0.f;
            for (int s = r; s < BC; ++s) x += Ts[s * L::PC + r] * dUs[s * L::PR + i];
            dRs[r * L::PR + i] = x;
            if (r < n) p.dv[tok(t0 + r) * DV + row0 + i] = bes[r] * x;
        }
        for (int e = tid; e < BC * BC; e += BNT) {
            const int r = e / BC, s = e % BC;
            float x = 0.f;
            if (s <= r)
                for (int i = 0; i < BR; ++i) x += dOs[r * L::PR + i] * Us[s * L::PR + i];
            dPs[r * L::PC + s] = x;
        }
        __syncthreads();
        // dT = dU R^T (strict lower part is all dA needs)
        for (int e = tid; e < BC * BC; e += BNT) {
            const int r = e / BC, s = e % BC;
            float x = 0.f;
            if (s < r)
                for (int i = 0; i < BR; ++i) x += dUs[r * L::PR + i] * Rs[s * L::PR + i];
            dTs[r * L::PC + s] = x;
        }
        __syncthreads();
        // Y = dT T^T into dA's tile (Y_rs = sum_{b <= s} dT_rb T_sb, r > b)
        for (int e = tid; e < BC * BC; e += BNT) {
            const int r = e / BC, s = e % BC;
            float x = 0.f;
            for (int bb = 0; bb <= s && bb < r; ++bb) x += dTs[r * L::PC + bb] * Ts[s * L::PC + bb];
            dAs[r * L::PC + s] = x;
        }
        __syncthreads();
        // dA = -T^T Y, strict lower (dA_rs = -sum_{a >= r} T_ar Y_as); into dT's tile
        for (int e = tid; e < BC * BC; e += BNT) {
            const int r = e / BC, s = e % BC;
            float x = 0.f;
            if (s < r)
                for (int a = r; a < BC; ++a) x -= Ts[a * L::PC + r] * dAs[a * L::PC + s];
            dTs[r * L::PC + s] = x;
        }
        __syncthreads();
        float* dAf = dTs;   // dA from here on
        // M1 = dP o Gamma, its transpose, and M3 = B + B^T with B = diag(beta)
        // (dA o Gamma), into tiles that are free by now (K G^T, Q K^T, K S^T)
        float* M1 = KGs;
        float* M1T = QKs;
        float* M3 = KSs;
        for (int e = tid; e < BC * BC; e += BNT) {
            const int r = e / BC, c = e % BC;
            const float m1 = dPs[r * L::PC + c] * Gam(r, c);
            M1[r * L::PC + c] = m1;
            M1T[c * L::PC + r] = m1;
            M3[r * L::PC + c] = bes[r] * dAf[r * L::PC + c] * Gam(r, c) +
                                bes[c] * dAf[c * L::PC + r] * Gam(c, r);
        }
        __syncthreads();
        // ---- dQ, dK partials on 2 x 8 tiles (token rows r, r + 1; key
        //      columns j0 .. j0 + 7); row sums of dW.K and K.(U G)
        {
            const int ra = i0;   // token rows of this thread's tile
            float aq[2][NC] = {}, ak[2][NC] = {}, dw[2][NC] = {};
            mm2n<BR, NC>(aq, [&](int x, int i) { return dOs[(ra + x) * L::PR + i]; }, Ss, L::PK, j0);
            mm2n<BR, NC>(ak, [&](int x, int i) { return Us[(ra + x) * L::PR + i]; }, Gs, L::PK, j0);
            mm2n<BR, NC>(dw, [&](int x, int i) { return -dRs[(ra + x) * L::PR + i]; }, Ss, L::PK, j0);
            float wk[2] = {0.f, 0.f}, kug[2] = {0.f, 0.f};
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int r = ra + x;
                const float gr = gas[r], Dr = dds[r], bg = bes[r] * gr;
#pragma unroll
                for (int y = 0; y < NC; ++y) {
                    const float kj = Ks[r * L::PK + j0 + y];
                    kug[x] += kj * ak[x][y];
                    wk[x] += kj * dw[x][y];
                    aq[x][y] *= gr;
                    ak[x][y] = Dr * ak[x][y] + bg * dw[x][y];
                }
            }
            mm2n<BC, NC>(aq, [&](int x, int c) { return M1[(ra + x) * L::PC + c]; }, Ks, L::PK, j0);
            mm2n<BC, NC>(ak, [&](int x, int c) { return M1T[(ra + x) * L::PC + c]; }, Qs, L::PK, j0);
            mm2n<BC, NC>(ak, [&](int x, int c) { return M3[(ra + x) * L::PC + c]; }, Ks, L::PK, j0);
#pragma unroll
            for (int x = 0; x < 2; ++x) {
                const int r = ra + x;
                if (r < n) {
                    float* qd = pqb + tok(t0 + r) * DK + j0;
                    float* kd = pkb + tok(t0 + r) * DK + j0;
#pragma unroll
                    for (int h = 0; h < NC / 4; ++h) {
                        *reinterpret_cast<f32x4*>(qd + 4 * h) =
                            f32x4{aq[x][4 * h], aq[x][4 * h + 1], aq[x][4 * h + 2], aq[x][4 * h + 3]};
                        *reinterpret_cast<f32x4*>(kd + 4 * h) =
                            f32x4{ak[x][4 * h], ak[x][4 * h + 1], ak[x][4 * h + 2], ak[x][4 * h + 3]};
                    }
                }
#pragma unroll
                for (int m = 1; m < 16; m <<= 1) {
                    wk[x] += __shfl_xor(wk[x], m, 64);
                    kug[x] += __shfl_xor(kug[x], m, 64);
                }
            }
            if ((tid & 15) == 0) {
                red[ra * 8 + 0] = wk[0];
                red[ra * 8 + 1] = kug[0];
                red[(ra + 1) * 8 + 0] = wk[1];
                red[(ra + 1) * 8 + 1] = kug[1];
            }
        }
        // sum over the rows of S o G (for gamma_C)
        {
            float x = 0.f;
            for (int e = tid; e < BR * DK; e += BNT) {
                const int i = e / DK, j = e % DK;
                x += Ss[i * L::PK + j] * Gs[i * L::PK + j];
            }
#pragma unroll
            for (int m = 1; m < 64; m <<= 1) x += __shfl_xor(x, m, 64);
            if ((tid & 63) == 0) misc[tid >> 6] = x;
        }
        __syncthreads();
        // ---- dbeta, dg per token (one thread per token row)
        if (tid < BC) {
            const int r = tid;
            const float be = bes[r], gr = gas[r], Dr = dds[r];
            const float wk = red[r * 8 + 0], dD = red[r * 8 + 1];
            float vdr = 0.f, dos = 0.f;
            for (int i = 0; i < BR; ++i) {
                vdr += Vs[r * L::PR + i] * dRs[r * L::PR + i];
                dos += dOs[r * L::PR + i] * QSs[r * L::PR + i];
            }
            float akk = 0.f, pp = 0.f, aa = 0.f;
            for (int s = 0; s < BC; ++s) {
                akk += dAf[r * L::PC + s] * Gam(r, s) * KKs[r * L::PC + s];
                pp += dPs[r * L::PC + s] * Ps[r * L::PC + s] - dPs[s * L::PC + r] * Ps[s * L::PC + r];
                aa += dAf[r * L::PC + s] * As[r * L::PC + s] - dAf[s * L::PC + r] * As[s * L::PC + r];
            }
            const float dbeta = vdr + gr * wk + akk;
            float dg = gr * (dos + be * wk) + pp + aa - Dr * dD;
            red[r * 8 + 2] = Dr * dD;
            red[r * 8 + 3] = dbeta;
            red[r * 8 + 4] = dg;
        }
        __syncthreads();
        if (tid == 0) {
            // g_C and D depend on the last live token's g (padding tokens
            // have log alpha = 0), so their terms go to token n - 1
            float sdd = 0.f;
            for (int r = 0; r < BC; ++r) sdd += red[r * 8 + 2];
            const float sg = misc[0] + misc[1] + misc[2] + misc[3];
            red[(n - 1) * 8 + 4] += sdd + gCe * sg;
        }
        __syncthreads();
        if (tid < n) {
            pbb[tok(t0 + tid)] = red[tid * 8 + 3];
            pgb[tok(t0 + tid)] = red[tid * 8 + 4];
        }
        // ---- G <- gamma_C G + dO^T diag(gamma) Q - dR^T diag(beta gamma) K
        {
            float acc[2][NC];
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int y = 0; y < NC; ++y) acc[x][y] = gCe * Gs[(i0 + x) * L::PK + j0 + y];
            mm2n<BC, NC>(acc, [&](int x, int r) { return gas[r] * dOs[r * L::PR + i0 + x]; }, Qs, L::PK, j0);
            mm2n<BC, NC>(acc, [&](int x, int r) { return -bes[r] * gas[r] * dRs[r * L::PR + i0 + x]; },
                     Ks, L::PK, j0);
            // each thread rewrites only the G entries it read
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int y = 0; y < NC; ++y) Gs[(i0 + x) * L::PK + j0 + y] = acc[x][y];
        }
    }
    __syncthreads();
    if (p.ds0) {
        for (int e = tid; e < BR * DK; e += BNT) {
            const int i = e / DK, j = e % DK;
            p.ds0[(bh * DV + row0 + i) * DK + j] = Gs[i * L::PK + j];
        }
    }
}

// dq, dk: the sum of the row blocks' partials
template <int DK, int NRB>
__global__ __launch_bounds__(256) void bwd_reduce_qk(int64_t n, const float* __restrict__ pq,
                                                     const float* __restrict__ pk,
                                                     float* __restrict__ dq,
                                                     float* __restrict__ dk) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
        a += pq[r * n + i];
        b += pk[r * n + i];
    }
    dq[i] = a;
    dk[i] = b;
}

// dbeta and dalpha: one thread per (b, h, chunk); dlog alpha is the reverse
// cumulative sum of dg inside the chunk, dalpha = dlog alpha / alpha (alpha
// clamped to FLT_MIN as in the forward's logarithm)
template <int NRB>
__global__ __launch_bounds__(256) void bwd_reduce_gates(int64_t B, int64_t T, int64_t H,
                                                        int64_t BTH, const float* __restrict__ pb,
                                                        const float* __restrict__ pg,
                                                        const float* __restrict__ alpha,
                                                        float* __restrict__ dalpha,
                                                        float* __restrict__ dbeta) {
    const int64_t nch = (T + BC - 1) / BC;
    const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (idx >= B * H * nch) return;
    const int64_t c = idx % nch, bh = idx / nch;
    const int64_t h = bh % H, b = bh / H;
    const int64_t t0 = c * BC, t1 = min(t0 + BC, T);
    float acc = 0.f;
    for (int64_t t = t1 - 1; t >= t0; --t) {
        const int64_t i = (b * T + t) * H + h;
        float g = 0.f, bb = 0.f;
#pragma unroll
        for (int r = 0; r < NRB; ++r) {
            g += pg[r * BTH + i];
            bb += pb[r * BTH + i];
        }
        acc += g;
        dbeta[i] = bb;
        dalpha[i] = acc / fmaxf(alpha[i], 1.17549435e-38f);
    }
}

template <int DK, int DV, typename TIn, typename TD>
hipError_t launch_bwd_t(const BwdArgs& a) {
    constexpr int NRB = DV / BR;
    const int64_t BH = a.B * a.H, BTH = a.B * a.T * a.H;
    const int64_t nch = (a.T + BC - 1) / BC;
    BwdParams p;
    p.T = a.T;
    p.H = a.H;
    p.BH = BH;
    p.BTH = BTH;
    p.q = a.q;
    p.k = a.k;
    p.v = a.v;
    p.dout = a.dout;
    p.alpha = a.alpha;
    p.beta = a.beta;
    p.s0 = a.s0;
    p.dsf = a.ds_final;
    p.dv = a.dv;
    p.ds0 = a.ds0;
    float* ws = reinterpret_cast<float*>(a.workspace);
    p.ck = ws;
    p.pq = p.ck + BH * nch * DV * DK;
    p.pk = p.pq + NRB * BTH * DK;
    p.pb = p.pk + NRB * BTH * DK;
    p.pg = p.pb + NRB * BTH;
    const size_t lds = sizeof(float) * BL<DK>::TOTAL;
    auto fn = chunk_bwd_kernel<DK, DV, TIn, TD>;
    hipError_t e = hipFuncSetAttribute((const void*)fn,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fn, dim3((unsigned)(BH * NRB)), dim3(BNT), lds, a.stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t nqk = BTH * DK;
    hipLaunchKernelGGL((bwd_reduce_qk<DK, NRB>), dim3((unsigned)((nqk + 255) / 256)), dim3(256), 0,
                       a.stream, nqk, p.pq, p.pk, a.dq, a.dk);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t ng = BH * nch;
    hipLaunchKernelGGL((bwd_reduce_gates<NRB>), dim3((unsigned)((ng + 255) / 256)), dim3(256), 0,
                       a.stream, a.B, a.T, a.H, BTH, p.pb, p.pg, a.alpha, a.dalpha, a.dbeta);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_bwd_d(const BwdArgs& a) {
    if (a.in_bf16)
        return a.dout_bf16 ? launch_bwd_t<DK, DV, bf16_t, bf16_t>(a)
                           : launch_bwd_t<DK, DV, bf16_t, float>(a);
    return a.dout_bf16 ? launch_bwd_t<DK, DV, float, bf16_t>(a)
                       : launch_bwd_t<DK, DV, float, float>(a);
}

}  // namespace

size_t bwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv) {
    const int64_t nch = (T + BC - 1) / BC;
    const int64_t nrb = Dv / BR;
    const int64_t BTH = B * T * H;
    return sizeof(float) * (size_t)(B * H * nch * Dv * Dk + 2 * nrb * BTH * Dk + 2 * nrb * BTH);
}

hipError_t launch_chunk_bwd(const BwdArgs& a) {
    if (a.Dk == 128 && a.Dv == 128) return launch_bwd_d<128, 128>(a);
    if (a.Dk == 128 && a.Dv == 64) return launch_bwd_d<128, 64>(a);
    if (a.Dk == 64 && a.Dv == 128) return launch_bwd_d<64, 128>(a);
    return launch_bwd_d<64, 64>(a);
}

}  // namespace gdr
