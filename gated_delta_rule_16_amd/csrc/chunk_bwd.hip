// gdr_chunk_bwd: reverse mode of the gated delta rule with scalar gates
// (alpha_t, beta_t per token and head), chunk by chunk, in fp32.
//
// Per chunk of n <= 16 tokens ("Gated Delta Networks", Method; the chunkwise
// form of the GDN review, section 3.7), with G_r the within-chunk cumulative
// log alpha, lambda_r = e^{G_r}, rho_r = lambda_C / lambda_r (lambda_C of the
// last token) and Gamma_rs = e^{G_r - G_s} (s <= r), the forward is
//
//   A_rs = beta_r Gamma_rs (k_r . k_s) (s < r),   P_rs = Gamma_rs (q_r . k_s) (s <= r)
//   T = (I + A)^{-1},  X = V - diag(lambda) K S^T,  R = diag(beta) X,  U = T R
//   O = diag(lambda) Q S^T + P U,   S' = lambda_C S + (diag(rho) U)^T K.
//
// Every decay is a scalar per token, so the reverse mode needs no table per
// channel: with G' = dL/dS' carried back from the next chunk,
//
//   dU = P^T dO + diag(rho) K G'^T,  dR = T^T dU,  dP = dO U^T (s <= r),
//   dA = -T^T (dU R^T) T^T (s < r),  dv = diag(beta) dR,
//   D_P = dP (.) Gamma,  D_A = dA (.) Gamma,  M_rs = beta_r D_A,rs + beta_s D_A,sr,
//   dq = D_P K + (diag(lambda) dO) S,
//   dk = M K + D_P^T Q + (diag(rho) U) G' - (diag(beta lambda) dR) S,
//   G  = lambda_C G' + (diag(lambda) dO)^T Q - (diag(beta lambda) dR)^T K,
//
// and the gate gradients are sums per token:
//
//   dbeta_r = sum_i dR_ri X_ri + sum_s dA_rs Gamma_rs (k_r . k_s),
//   dlog alpha_t = sum_{r >= t} tau_r + sum_{r < t} kappa_r + lambda_C <G', S>
//                  + sum_{r >= t > s} (dA_rs A_rs + dP_rs P_rs),
//   tau_r = -beta_r sum_i dR_ri (V_ri - X_ri) + sum_c q_rc ((diag(lambda) dO) S)_rc,
//   kappa_r = rho_r sum_i U_ri (K G'^T)_ri,
//
// (lambda_r depends on alpha_t for t <= r, rho_r for r < t, Gamma_rs for
// s < t <= r, lambda_C for every token of the chunk).  The pair sum takes
// each (r, s) once, so nothing cancels.
//
// Work split: one 256-thread workgroup (4 waves) per (b, h, 32 state rows),
// two workgroups per CU (about 78 KB of LDS each).  It runs the forward over
// its rows (chunk-start states to the workspace), then walks the chunks in
// reverse.  dv and dS_0 are final per workgroup.  dq and dk are sums over the
// row blocks (every term is linear in the row block's share of dU, dR, dP
// and dA): each workgroup adds its share by fp32 atomic adds, which the L2
// of the XCD that holds all of a head's row blocks performs, so the order of
// the four additions, and the last bits of dq and dk, vary from run to run.
// dbeta and d log alpha go to per-row-block partials that a second kernel
// adds.  Every product is a
// set of 16 x 16 tiles on the fp32 matrix cores (v_mfma_f32_16x16x4f32),
// the triangular solve and the elementwise terms are vector ALU.  Each wave
// forms the chunk's gate scalars itself (a DPP scan of log2 alpha across the
// 16 lanes of each row), so the gates cost no barrier.
#include "gdr_device.h"
#include "launch.h"
#include "vtile.h"

namespace gdr {

namespace {

constexpr int CB = 16;    // tokens per chunk
constexpr int RBW = 32;   // state rows per workgroup
constexpr int NTB = 256;  // threads per workgroup

struct BwdParams {
    int64_t T, H, BTH;
    const void *q, *k, *v, *dout;
    const float *alpha, *beta, *s0, *dsf;
    float *dv, *ds0;
    float* ck;                     // [BH][nch][Dv][Dk] chunk-start states
    const float* ta;               // [BH][nch][2][16][16]: T and AK of each chunk
    float *aq, *ak;                // [BTH][Dk] dq, dk accumulators (zero on entry)
    float *pb, *pg;                // [NRB][BTH]: dbeta, d log alpha
    bool l2norm;                   // q, k normalised on load (GDR_L2NORM_QK)
};

// LDS tables (floats).  Pitches as in the GDN-2 backward: key-side rows
// PK = 4 (mod 64), n x n PC = 20, n x rows PR = 36, so the row (16-byte) and
// column (4-byte) operand reads of mma16 are free of bank conflicts.
template <int DK>
struct BL {
    static constexpr int PK = DK + 4;
    static constexpr int PC = 20;
    static constexpr int PR = 36;
    static constexpr int NK = CB * PK;           // one token x key-dim table
    static constexpr int NN = CB * PC;           // one n x n tile
    static constexpr int NR = CB * PR;           // one n x rows tile
    static constexpr int K = 0;
    static constexpr int Q = K + NK;
    static constexpr int S = Q + NK;             // [RBW][PK] chunk-start state rows
    static constexpr int G = S + RBW * PK;       // [RBW][PK] dL/dS' rows
    static constexpr int AK = G + RBW * PK;      // Gamma (.) K K^T, s < r
    static constexpr int TM = AK + NN;           // T
    static constexpr int P = TM + NN;
    static constexpr int DP = P + NN;            // D_P
    static constexpr int DA = DP + NN;           // dU R^T, then D_A
    static constexpr int Y = DA + NN;            // (dU R^T) T^T, then M
    static constexpr int V = Y + NN;
    static constexpr int X = V + NR;
    static constexpr int R = X + NR;
    static constexpr int DO = R + NR;            // dL/do
    static constexpr int U = DO + NR;
    static constexpr int UT = U + NR;            // diag(rho) U
    static constexpr int DU = UT + NR;
    static constexpr int KG = DU + NR;           // K G'^T, then diag(lambda) dL/do
    static constexpr int DRB = KG + NR;          // diag(beta lambda) dR
    // per-token partial sums, two sets (chunk parity: a chunk's set is read
    // while the next chunk writes the other), offsets within a set:
    static constexpr int SC = DRB + NR;
    static constexpr int TAUR = 0;               //   [2 row tiles][16] dR terms of tau
    static constexpr int BER = TAUR + 32;        //   [2][16] sum_i dR X
    static constexpr int KAP = BER + 32;         //   [2][16] kappa
    static constexpr int TAUO = KAP + 32;        //   [4 waves][16] dO terms of tau
    static constexpr int BEA = TAUO + 64;        //   [16] A term of dbeta
    static constexpr int PRA = BEA + 16;         //   [16] pair sums of dA (.) A
    static constexpr int PRP = PRA + 16;         //   [16] pair sums of dP (.) P
    static constexpr int GSUM = PRP + 16;        //   [2 row tiles] lambda_C <G', S>
    static constexpr int NSC = GSUM + 4;
    static constexpr int TOTAL = SC + 2 * NSC;
    static_assert(TOTAL * 4 <= 80 * 1024, "two workgroups per CU");
    static_assert(PK % 64 == 4 && NK % 4 == 0 && S % 4 == 0 && G % 4 == 0, "pitches");
    static_assert(AK % 4 == 0 && V % 4 == 0 && SC % 4 == 0, "16-byte rows");
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// inclusive prefix sum over the 16 lanes of each DPP row (row_shr 1, 2, 4, 8;
// lanes shifted in from outside the row add 0)
__device__ __forceinline__ float rscan16(float x) {
    x += dpp<0x111>(x);
    x += dpp<0x112>(x);
    x += dpp<0x114>(x);
    x += dpp<0x118>(x);
    return x;
}

// inclusive suffix sum over the 16 lanes of each DPP row (row_shl 1, 2, 4, 8)
__device__ __forceinline__ float rsuffix16(float x) {
    x += dpp<0x101>(x);
    x += dpp<0x102>(x);
    x += dpp<0x104>(x);
    x += dpp<0x108>(x);
    return x;
}

__device__ __forceinline__ float lane_value(float x, int l) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}

// W 32-bit words at byte offset off of a buffer, in 16-, 8- or 4-byte loads
template <int W>
__device__ __forceinline__ void bld(uint32_t (&w)[W], __amdgpu_buffer_rsrc_t r, int off) {
    if constexpr (W % 4 == 0) {
#pragma unroll
        for (int h = 0; h < W / 4; ++h) {
            const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * h, 0, 0);
            w[4 * h] = x[0];
            w[4 * h + 1] = x[1];
            w[4 * h + 2] = x[2];
            w[4 * h + 3] = x[3];
        }
    } else if constexpr (W == 2) {
        const u32x2w x = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
        w[0] = x[0];
        w[1] = x[1];
    } else {
        static_assert(W == 1, "1, 2 or a multiple of 4 words");
        w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    }
}

// One chunk's global inputs for one thread, as raw words: key-side rows
// (token tid / 16, channels j0 .. j0 + NC), a pair of state rows of v and
// dL/do (token tid / 16, rows 2 (tid % 16), + 1), and the gates of token
// lane % 16.
template <typename TIn, typename TD, int NC>
struct Pre {
    static constexpr int WK = NC / packed<TIn>::PER_WORD;
    static constexpr int WP = 2 / packed<TIn>::PER_WORD;
    static constexpr int WD = 2 / packed<TD>::PER_WORD;
    uint32_t k[WK], q[WK];
    uint32_t v[WP], d[WD];
    float a, b;
};

// The chunk's gate scalars in one wave.  Lane l holds those of token l % 16;
// the r-arrays those of token r = 4 (l / 16) + i, the rows of an
// accumulator tile.
struct Gates {
    float be, G, lam, rho, lamC;
    float br[4], Gr[4], lr[4], rr[4];
};

// The gate scalars of a chunk of n tokens in one wave, from token
// lane % 16's alpha and beta (alpha = 1 past the end): a DPP scan of
// log2 alpha across the 16 lanes of each row, bpermutes for the r-arrays.
__device__ __forceinline__ Gates chunk_gates(float a, float b, int n, int lane) {
    const int l16 = lane & 15, lg = lane >> 4;
    Gates g;
    g.be = b;
    g.G = rscan16(l16 < n ? safe_log2(a) : 0.f);
    const float GC = lane_value(g.G, 15);
    g.lam = ex2(g.G);
    g.rho = ex2(GC - g.G);
    g.lamC = ex2(GC);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * lg + i;
        g.br[i] = __shfl(g.be, r, 64);
        g.Gr[i] = __shfl(g.G, r, 64);
        g.lr[i] = __shfl(g.lam, r, 64);
        g.rr[i] = __shfl(g.rho, r, 64);
    }
    return g;
}

// Gamma at the accumulator entries (r = 4 (lane / 16) + i, s = lane % 16),
// masked to s < r (strict) or s <= r
__device__ __forceinline__ f32x4 gamma_tile(const Gates& g, bool strict, int lane) {
    const int l16 = lane & 15, lg = lane >> 4;
    f32x4 gm;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * lg + i;
        gm[i] = (strict ? l16 < r : l16 <= r) ? ex2(g.Gr[i] - g.G) : 0.f;
    }
    return gm;
}

// T = (I + A)^{-1}, A = diag(beta) AK, by one wave (tables at row pitch PC):
// lane 4 c + q owns column c, rows 4 q .. 4 q + 3; row r of the column is
// delta_rc - beta_r sum_{m < r} AK_rm T_mc (AK's upper part is zero), the
// four partial sums joined by a quad reduction.  The lane's AK entries are
// read before the first row.
template <int PC>
__device__ __forceinline__ void solve_t(const float* AKs, float* Ts, const Gates& g, int lane) {
    const int c = lane >> 2, q = lane & 3;
    f32x4 ak[CB];
#pragma unroll
    for (int r = 0; r < CB; ++r) ak[r] = ld4(AKs + r * PC + 4 * q);
    float tq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < CB; ++r) {
        float part = (ak[r][0] * tq[0] + ak[r][1] * tq[1]) + (ak[r][2] * tq[2] + ak[r][3] * tq[3]);
        part = qsum(part);
        const float t = r < c ? 0.f : (r == c ? 1.f : 0.f) - lane_value(g.be, r) * part;
        if (q == (r >> 2)) tq[r & 3] = t;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) Ts[(4 * q + j) * PC + c] = tq[j];
}

struct SolveParams {
    int64_t T, H, nch, nchunks;    // nchunks = B H nch
    const void* k;
    const float *alpha, *beta;
    float* ta;                     // [B H nch][2][16][16]: T, then AK
    bool l2norm;
};

// T and AK = Gamma (.) K K^T (s < r) of every chunk, one wave per (b, h,
// chunk): they depend on the chunk's keys and gates only, so the main
// kernel's sweeps read them instead of solving one triangle per chunk in
// sequence.  Lane l loads channels DK/4 (l % 4) .. of token l / 4.
template <int DK, typename TIn>
__global__ __launch_bounds__(256) void gdn_bwd_solve(SolveParams p) {
    constexpr int PK = DK + 4, PC = 20, NQK = DK / 16, CW = DK / 4;
    constexpr int PER = CB * PK + 2 * CB * PC;
    __shared__ __align__(16) float sm[4 * PER];
    const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63, l16 = lane & 15, lg = lane >> 4;
    const int64_t ci = (int64_t)blockIdx.x * 4 + wv;
    if (ci >= p.nchunks) return;   // whole waves; no workgroup barrier below
    const int64_t bh = ci / p.nch, c = ci % p.nch;
    const int64_t h = bh % p.H, b = bh / p.H;
    float* Kw = sm + wv * PER;
    float* AKs = Kw + CB * PK;
    float* Ts = AKs + CB * PC;
    const int n = (int)min((int64_t)CB, p.T - c * CB);
    const int64_t tb = (b * p.T + c * CB) * p.H + h;
    const int HDK = (int)(p.H * DK), HI = (int)p.H;
    const int t = lane >> 2, c0 = CW * (lane & 3);
    constexpr int SI = sizeof(TIn);
    uint32_t kw[CW / packed<TIn>::PER_WORD];
    bld(kw, rsrc(reinterpret_cast<const TIn*>(p.k) + tb * DK, n * HDK * SI), (t * HDK + c0) * SI);
    const float a = __uint_as_float(
        __builtin_amdgcn_raw_buffer_load_b32(rsrc(p.alpha + tb, n * HI * 4), l16 * HI * 4, 0, 0));
    const float bt = __uint_as_float(
        __builtin_amdgcn_raw_buffer_load_b32(rsrc(p.beta + tb, n * HI * 4), l16 * HI * 4, 0, 0));
    float kn = 1.f;
    if (p.l2norm) {
        float ss = 0.f;
#pragma unroll
        for (int y = 0; y < CW; ++y) {
            const float kk = packed<TIn>::at(kw, y);
            ss += kk * kk;
        }
        kn = l2_inv(qsum(ss));
    }
#pragma unroll
    for (int y0 = 0; y0 < CW; y0 += 4) {
        f32x4 kv;
#pragma unroll
        for (int e = 0; e < 4; ++e) kv[e] = packed<TIn>::at(kw, y0 + e) * kn;
        *reinterpret_cast<f32x4*>(Kw + t * PK + c0 + y0) = kv;
    }
    const Gates g = chunk_gates(a, bt, n, lane);
    wave_sync();
    const f32x4 kk = mma16<NQK, true, true>(f32x4{0.f, 0.f, 0.f, 0.f}, Kw, PK, Kw, PK, lane);
    const f32x4 gm = gamma_tile(g, true, lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) AKs[(4 * lg + i) * PC + l16] = kk[i] * gm[i];
    wave_sync();
    solve_t<PC>(AKs, Ts, g, lane);
    wave_sync();
    const __amdgpu_buffer_rsrc_t ro = rsrc(p.ta + ci * 512, 512 * 4);
    const int r = lane >> 2, c4 = 4 * (lane & 3);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, ld4(Ts + r * PC + c4)), ro,
                                           (r * 16 + c4) * 4, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, ld4(AKs + r * PC + c4)), ro,
                                           (256 + r * 16 + c4) * 4, 0, 0);
}

template <int DK, int DV, typename TIn, typename TD>
__global__ __launch_bounds__(NTB) __attribute__((amdgpu_waves_per_eu(2)))
void gdn_bwd_kernel(BwdParams p) {
    using L = BL<DK>;
    constexpr int NRB = DV / RBW;
    constexpr int NC = DK / 16;
    constexpr int NQK = DK / 16;                // 16-deep blocks over the key dim
    constexpr int CTW = DK / 64;                // channel tiles per wave
    constexpr int NSV = RBW * DK / 4 / NTB;     // 16-byte state pieces per thread
    constexpr int NSW = RBW * DK / 4 / 64;      // .. per lane of one wave
    extern __shared__ __align__(16) float sm[];
    float* Ks = sm + L::K;
    float* Qs = sm + L::Q;
    float* Ss = sm + L::S;
    float* Gs = sm + L::G;
    float* AKs = sm + L::AK;
    float* Ts = sm + L::TM;
    float* Ps = sm + L::P;
    float* DPs = sm + L::DP;
    float* DAs = sm + L::DA;
    float* Ys = sm + L::Y;
    float* Vs = sm + L::V;
    float* Xs = sm + L::X;
    float* Rs = sm + L::R;
    float* DOs = sm + L::DO;
    float* Us = sm + L::U;
    float* UTs = sm + L::UT;
    float* DUs = sm + L::DU;
    float* KGs = sm + L::KG;
    float* DOLs = KGs;   // diag(lambda) dL/do from the third phase of a chunk on
    float* DRBs = sm + L::DRB;

    const int tid = threadIdx.x;
    const int wv = tid >> 6;
    // lane indices, renewed at the top of every chunk through an opaque copy
    // so that the many LDS addresses formed from them are computed where they
    // are used rather than hoisted out of the chunk loops into registers
    int lane = tid & 63, l16 = lane & 15, lg = lane >> 4;
    auto renew_lane = [&]() {
        asm volatile("" : "+v"(lane));
        l16 = lane & 15;
        lg = lane >> 4;
    };
    // the row blocks of a head on one XCD (blocks are dealt to the 8 XCDs in
    // turn): they read the same key-side rows
    const int64_t nb = gridDim.x;
    const int64_t wid = (nb % (8 * NRB) == 0) ? (blockIdx.x % 8) * (nb / 8) + blockIdx.x / 8
                                              : (int64_t)blockIdx.x;
    const int rb = (int)(wid % NRB);
    const int64_t bh = wid / NRB;
    const int64_t h = bh % p.H;
    const int64_t b = bh / p.H;
    const int64_t T = p.T, H = p.H;
    const int row0 = rb * RBW;
    const int64_t nch = (T + CB - 1) / CB;
    float* ckb = p.ck + bh * nch * DV * DK;
    const float* tab = p.ta + bh * nch * 512;
    auto tok = [&](int64_t t) { return (b * T + t) * H + h; };
    const int tr = tid >> 4;                   // this thread's token for the loads
    const int j0 = NC * (tid & 15);            // .. and its key channels
    const int i2 = 2 * (tid & 15);             // .. and its pair of state rows
    auto chunk_len = [&](int64_t c) { return (int)min((int64_t)CB, T - c * CB); };
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};

    const int HDK = (int)(H * DK), HDV = (int)(H * DV), HI = (int)H;
    using PF = Pre<TIn, TD, NC>;
    // a chunk's rows through buffer resources that end at its last token:
    // rows past it read as zeros (beta = 0; gates() sets alpha to 1 there)
    auto fetch = [&](PF& x, int64_t c, bool bwd) {
        const int n = chunk_len(c);
        const int64_t tb = tok(c * CB);
        constexpr int SI = sizeof(TIn), SD = sizeof(TD);
        bld(x.k, rsrc(reinterpret_cast<const TIn*>(p.k) + tb * DK, n * HDK * SI),
            (tr * HDK + j0) * SI);
        if (bwd)
            bld(x.q, rsrc(reinterpret_cast<const TIn*>(p.q) + tb * DK, n * HDK * SI),
                (tr * HDK + j0) * SI);
        bld(x.v, rsrc(reinterpret_cast<const TIn*>(p.v) + tb * DV, n * HDV * SI),
            (tr * HDV + row0 + i2) * SI);
        if (bwd)
            bld(x.d, rsrc(reinterpret_cast<const TD*>(p.dout) + tb * DV, n * HDV * SD),
                (tr * HDV + row0 + i2) * SD);
        x.a = __uint_as_float(
            __builtin_amdgcn_raw_buffer_load_b32(rsrc(p.alpha + tb, n * HI * 4), l16 * HI * 4, 0, 0));
        x.b = __uint_as_float(
            __builtin_amdgcn_raw_buffer_load_b32(rsrc(p.beta + tb, n * HI * 4), l16 * HI * 4, 0, 0));
    };
    auto commit = [&](const PF& x, int64_t c, bool bwd) {
        const int at = tr * L::PK + j0;
        // GDR_L2NORM_QK: the 16 lanes of a token (one DPP row) hold its row
        float kn = 1.f, qn = 1.f;
        if (p.l2norm) {
            float sk = 0.f, sq = 0.f;
#pragma unroll
            for (int y = 0; y < NC; ++y) {
                const float kk = packed<TIn>::at(x.k, y);
                const float qq = bwd ? packed<TIn>::at(x.q, y) : 0.f;
                sk += kk * kk;
                sq += qq * qq;
            }
            kn = l2_inv(rsum16(sk));
            qn = l2_inv(rsum16(sq));
        }
#pragma unroll
        for (int y0 = 0; y0 < NC; y0 += 4) {
            f32x4 kv, qv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                kv[e] = packed<TIn>::at(x.k, y0 + e) * kn;
                qv[e] = bwd ? packed<TIn>::at(x.q, y0 + e) * qn : 0.f;
            }
            *reinterpret_cast<f32x4*>(Ks + at + y0) = kv;
            if (bwd) *reinterpret_cast<f32x4*>(Qs + at + y0) = qv;
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int o = tr * L::PR + i2 + e;
            Vs[o] = packed<TIn>::at(x.v, e);
            if (bwd) DOs[o] = packed<TD>::at(x.d, e);
        }
    };
    auto gates = [&](const PF& x, int n) { return chunk_gates(x.a, x.b, n, lane); };
    auto gamma = [&](const Gates& g, bool strict) { return gamma_tile(g, strict, lane); };
    // sum over the pairs s < t <= r of W_rs (accumulator layout), for t = l16
    auto straddle = [&](const f32x4& w) {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float e = rscan16(w[i]) - w[i];   // sum over s < l16 of W_rs
            if (4 * lg + i >= l16) acc += e;
        }
        acc += __shfl_xor(acc, 16, 64);
        acc += __shfl_xor(acc, 32, 64);
        return acc;
    };
    // K S^T (or K G'^T) for state-row tile t
    auto ks_tile = [&](const float* M, int t) {
        return mma16<NQK, true, true>(zero4, Ks, L::PK, M + 16 * t * L::PK, L::PK, lane);
    };

    // ======================= forward: chunk-start states =====================
    {
        f32x4 sv[NSV];
#pragma unroll
        for (int it = 0; it < NSV; ++it) {
            const int e4 = tid + it * NTB;
            const int i = e4 / (DK / 4), j = 4 * (e4 % (DK / 4));
            sv[it] = p.s0 ? *reinterpret_cast<const f32x4*>(p.s0 + (bh * DV + row0 + i) * DK + j)
                          : zero4;
            *reinterpret_cast<f32x4*>(Ss + i * L::PK + j) = sv[it];
        }
    }
    // this thread's two entries of a chunk's T and AK (from gdn_bwd_solve)
    u32x2w tv;
    auto fetch_t = [&](int64_t c) {
        tv = __builtin_amdgcn_raw_buffer_load_b64(rsrc(tab + c * 512, 512 * 4), 8 * tid, 0, 0);
    };
    auto commit_t = [&]() {
        const int e = 2 * tid, r = (e & 255) >> 4, col = e & 15;
        float* d = (e < 256 ? Ts : AKs) + r * L::PC + col;
        d[0] = __uint_as_float(tv[0]);
        d[1] = __uint_as_float(tv[1]);
    };
    PF x;
    fetch(x, 0, false);
    fetch_t(0);
    for (int64_t c = 0; c < nch; ++c) {
        renew_lane();
        __syncthreads();
        commit(x, c, false);
        commit_t();
        const Gates g = gates(x, chunk_len(c));
        if (c + 1 < nch) {
            fetch(x, c + 1, false);
            fetch_t(c + 1);
        }
        __syncthreads();
        // waves 0, 1: K S^T, R, then diag(rho) T R on row tile wv;
        // waves 2, 3: S to the workspace, rows 16 (wv - 2) ..
        if (wv < 2) {
            const int t = wv;
            const f32x4 ks = ks_tile(Ss, t);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int o = (4 * lg + i) * L::PR + 16 * t + l16;
                Rs[o] = g.br[i] * (Vs[o] - g.lr[i] * ks[i]);
            }
            wave_sync();
            const f32x4 u = mma16<1, true, false>(zero4, Ts, L::PC, Rs + 16 * t, L::PR, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i) UTs[(4 * lg + i) * L::PR + 16 * t + l16] = g.rr[i] * u[i];
        } else {
            const __amdgpu_buffer_rsrc_t rc = rsrc(ckb + c * DV * DK, DV * DK * 4);
#pragma unroll
            for (int it = 0; it < NSW / 2; ++it) {
                const int e4 = lane + 64 * it + (wv - 2) * (NSW / 2) * 64;
                const int i = e4 / (DK / 4), j = 4 * (e4 % (DK / 4));
                __builtin_amdgcn_raw_buffer_store_b128(
                    __builtin_bit_cast(u32x4, ld4(Ss + i * L::PK + j)), rc,
                    ((row0 + i) * DK + j) * 4, 0, 0);
            }
        }
        __syncthreads();
        // S <- lambda_C S + (diag(rho) U)^T K on this wave's channel tiles
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) {
            const int t = CTW * wv + ct, cc = 16 * t + l16;
#pragma unroll
            for (int a = 0; a < 2; ++a) {
                f32x4 acc;
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[i] = Ss[(16 * a + 4 * lg + i) * L::PK + cc] * g.lamC;
                acc = mma16<1, false, false>(acc, UTs + 16 * a, L::PR, Ks + 16 * t, L::PK, lane);
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
            const int e4 = tid + it * NTB;
            const int i = e4 / (DK / 4), j = 4 * (e4 % (DK / 4));
            gv[it] = p.dsf ? *reinterpret_cast<const f32x4*>(p.dsf + (bh * DV + row0 + i) * DK + j)
                           : zero4;
            *reinterpret_cast<f32x4*>(Gs + i * L::PK + j) = gv[it];
        }
    }
    // a chunk's outputs leave through buffer stores whose range ends at its
    // last token: rows past it are dropped without a branch
    auto bstore = [&](float v, __amdgpu_buffer_rsrc_t r, int off) {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
    };
    auto badd = [&](float v, __amdgpu_buffer_rsrc_t r, int off) {
        __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(v, r, off, 0, 0);
    };
    // the gate gradients of chunk cp from its per-token partial sums (one
    // wave; lane l takes token l % 16, DPP scans over the tokens; the four
    // lane rows store the same values)
    auto finalize = [&](int64_t cp, const float* sc) {
        const int t = l16;
        const float tau = sc[L::TAUR + t] + sc[L::TAUR + 16 + t] + sc[L::TAUO + t] +
                          sc[L::TAUO + 16 + t] + sc[L::TAUO + 32 + t] + sc[L::TAUO + 48 + t];
        const float kap = sc[L::KAP + t] + sc[L::KAP + 16 + t];
        // sum_{r >= t} tau_r + sum_{r < t} kappa_r
        const float dl = rsuffix16(tau) + (rscan16(kap) - kap) + (sc[L::GSUM] + sc[L::GSUM + 1]) +
                         sc[L::PRA + t] + sc[L::PRP + t];
        const float db = sc[L::BER + t] + sc[L::BER + 16 + t] + sc[L::BEA + t];
        const int bytes = chunk_len(cp) * HI * 4;
        const int64_t o = (int64_t)rb * p.BTH + tok(cp * CB);
        bstore(db, rsrc(p.pb + o, bytes), t * HI * 4);
        bstore(dl, rsrc(p.pg + o, bytes), t * HI * 4);
    };
    f32x4 sv[NSV];
    auto fetch_s = [&](int64_t c) {
        const __amdgpu_buffer_rsrc_t rc = rsrc(ckb + c * DV * DK, DV * DK * 4);
#pragma unroll
        for (int it = 0; it < NSV; ++it) {
            const int e4 = tid + it * NTB;
            const int i = e4 / (DK / 4), j = 4 * (e4 % (DK / 4));
            sv[it] = __builtin_bit_cast(
                f32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, ((row0 + i) * DK + j) * 4, 0, 0));
        }
    };
    fetch(x, nch - 1, true);
    fetch_s(nch - 1);
    fetch_t(nch - 1);
    // wait for the first chunk's loads here: entering the loop with nothing
    // in flight lets the compiler count the stores each later chunk issues
    // after its prefetch, instead of waiting for all of them at the top
    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)
    for (int64_t c = nch - 1; c >= 0; --c) {
        const int64_t t0 = c * CB;
        const int n = chunk_len(c);
        const int64_t tb = tok(t0);
        float* scw = sm + L::SC + (int)(c & 1) * L::NSC;                // this chunk's sums
        const float* scr = sm + L::SC + (int)((c + 1) & 1) * L::NSC;    // the later chunk's
        renew_lane();
        __syncthreads();
#pragma unroll
        for (int it = 0; it < NSV; ++it) {
            const int e4 = tid + it * NTB;
            const int i = e4 / (DK / 4), j = 4 * (e4 % (DK / 4));
            *reinterpret_cast<f32x4*>(Ss + i * L::PK + j) = sv[it];
        }
        commit(x, c, true);
        commit_t();
        const Gates g = gates(x, n);
        if (c > 0) {
            fetch(x, c - 1, true);
            fetch_s(c - 1);
            fetch_t(c - 1);
        }
        __syncthreads();
        // ---- (T and AK from gdn_bwd_solve)  waves 0, 3: X, R rows 0..15,
        //      16..31;  wave 0: P;  waves 1, 2: K G'^T rows 0..15, 16..31;
        //      wave 1: the later chunk's gate gradients;  waves 2, 3:
        //      <G', S> over rows 0..15, 16..31
        if (wv == 0 || wv == 3) {
            const int t = wv == 0 ? 0 : 1;
            const f32x4 ks = ks_tile(Ss, t);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int o = (4 * lg + i) * L::PR + 16 * t + l16;
                const float xv = Vs[o] - g.lr[i] * ks[i];
                Xs[o] = xv;
                Rs[o] = g.br[i] * xv;
            }
        } else {
            const int t = wv - 1;
            const f32x4 kg = ks_tile(Gs, t);
#pragma unroll
            for (int i = 0; i < 4; ++i) KGs[(4 * lg + i) * L::PR + 16 * t + l16] = kg[i];
        }
        if (wv == 0) {
            const f32x4 qk = mma16<NQK, true, true>(zero4, Qs, L::PK, Ks, L::PK, lane);
            const f32x4 gm = gamma(g, false);
#pragma unroll
            for (int i = 0; i < 4; ++i) Ps[(4 * lg + i) * L::PC + l16] = qk[i] * gm[i];
        } else if (wv == 1) {
            if (c + 1 < nch) finalize(c + 1, scr);
        } else {
            // lane: 4 channels (16-byte reads), CG / 4 of the 16 rows
            const int t = wv - 2;
            constexpr int CG = DK / 4;
            const int c4 = 4 * (lane % CG), rg = lane / CG;
            float sg = 0.f;
#pragma unroll
            for (int m = 0; m < CG / 4; ++m) {
                const int i = 16 * t + (CG / 4) * rg + m;
                const f32x4 gv = ld4(Gs + i * L::PK + c4), sv4 = ld4(Ss + i * L::PK + c4);
                sg += (gv[0] * sv4[0] + gv[1] * sv4[1]) + (gv[2] * sv4[2] + gv[3] * sv4[3]);
            }
#pragma unroll
            for (int m = 32; m >= 1; m >>= 1) sg += __shfl_xor(sg, m, 64);
            if (lane == 0) scw[L::GSUM + t] = g.lamC * sg;
        }
        __syncthreads();
        // ---- U = T R and kappa (waves 0, 1);
        //      dU = diag(rho) K G'^T + P^T dO (waves 2, 3)
        if (wv < 2) {
            const int t = wv;
            const f32x4 u = mma16<1, true, false>(zero4, Ts, L::PC, Rs + 16 * t, L::PR, lane);
            float kp[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int o = (4 * lg + i) * L::PR + 16 * t + l16;
                const float ut = g.rr[i] * u[i];
                Us[o] = u[i];
                UTs[o] = ut;
                kp[i] = rsum16(ut * KGs[o]);
            }
            if (l16 == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) scw[L::KAP + 16 * t + 4 * lg + i] = kp[i];
            }
        } else {
            const int t = wv - 2;
            f32x4 acc;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = g.rr[i] * KGs[(4 * lg + i) * L::PR + 16 * t + l16];
            acc = mma16<1, false, false>(acc, Ps, L::PC, DOs + 16 * t, L::PR, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i) DUs[(4 * lg + i) * L::PR + 16 * t + l16] = acc[i];
        }
        __syncthreads();
        // ---- dR = T^T dU (waves 0, 1: dv to HBM, dbeta and tau row sums,
        //      then diag(lambda) dO);  dP = dO U^T, D_P, pair sums (wave 2);
        //      dA and M (wave 3)
        if (wv < 2) {
            const int t = wv;
            const f32x4 dr = mma16<1, false, false>(zero4, Ts, L::PC, DUs + 16 * t, L::PR, lane);
            const __amdgpu_buffer_rsrc_t rdv = rsrc(p.dv + tb * DV, n * HDV * 4);
            float sb[4], st[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * lg + i, o = r * L::PR + 16 * t + l16;
                DRBs[o] = g.br[i] * g.lr[i] * dr[i];
                const float xv = Xs[o];
                sb[i] = rsum16(dr[i] * xv);
                st[i] = rsum16(dr[i] * (Vs[o] - xv));
                bstore(g.br[i] * dr[i], rdv, (r * HDV + row0 + 16 * t + l16) * 4);
            }
            if (l16 == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    scw[L::BER + 16 * t + 4 * lg + i] = sb[i];
                    scw[L::TAUR + 16 * t + 4 * lg + i] = -g.br[i] * st[i];
                }
            }
            // diag(lambda) dL/do, tokens 8 t .. 8 t + 7, into K G'^T's place
            // (dead after the last phase): element lane + 64 e is token
            // 8 t + 2 e + lane / 32, row lane % 32
#pragma unroll
            for (int e = 0; e < CB * RBW / 128; ++e) {
                const int r = 8 * t + 2 * e;
                const float lm = lane < 32 ? lane_value(g.lam, r) : lane_value(g.lam, r + 1);
                const int o = (r + (lane >> 5)) * L::PR + (lane & 31);
                DOLs[o] = DOs[o] * lm;
            }
        } else if (wv == 2) {
            const f32x4 dp = mma16<2, true, true>(zero4, DOs, L::PR, Us, L::PR, lane);
            const f32x4 gm = gamma(g, false);
            f32x4 w;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * lg + i;
                const bool m = l16 <= r;
                w[i] = m ? dp[i] * Ps[r * L::PC + l16] : 0.f;
                DPs[r * L::PC + l16] = m ? dp[i] * gm[i] : 0.f;
            }
            const float pr = straddle(w);
            if (lane < 16) scw[L::PRP + lane] = pr;
        } else {
            // dT = dU R^T, Y = dT T^T, dA = -T^T Y (strict), D_A, the A term
            // of dbeta, its pair sums and M
            const f32x4 dt = mma16<2, true, true>(zero4, DUs, L::PR, Rs, L::PR, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * lg + i;
                DAs[r * L::PC + l16] = l16 < r ? dt[i] : 0.f;
            }
            wave_sync();
            const f32x4 y = mma16<1, true, true>(zero4, DAs, L::PC, Ts, L::PC, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i) Ys[(4 * lg + i) * L::PC + l16] = y[i];
            wave_sync();
            const f32x4 da = mma16<1, false, false, true>(zero4, Ts, L::PC, Ys, L::PC, lane);
            const f32x4 gm = gamma(g, true);
            f32x4 w;
            float sb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * lg + i;
                const float dv = l16 < r ? da[i] : 0.f;
                const float ak = dv * AKs[r * L::PC + l16];
                w[i] = g.br[i] * ak;
                sb[i] = rsum16(ak);
                DAs[r * L::PC + l16] = dv * gm[i];
            }
            const float pr = straddle(w);
            if (lane < 16) scw[L::PRA + lane] = pr;
            if (l16 == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) scw[L::BEA + 4 * lg + i] = sb[i];
            }
            wave_sync();
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * lg + i;
                Ys[r * L::PC + l16] = g.br[i] * DAs[r * L::PC + l16] + g.be * DAs[l16 * L::PC + r];
            }
        }
        __syncthreads();
        // ---- this wave's channel tiles, the tiles' chains side by side: dq,
        //      dk, the dO terms of tau; then G' <- lambda_C G' + (lambda dO)^T Q
        //      - (beta lambda dR)^T K (only this wave reads these channels of
        //      G' from here on)
        const __amdgpu_buffer_rsrc_t rq = rsrc(p.aq + tb * DK, n * HDK * 4);
        f32x4 dq[CTW], dk[CTW];
        float tq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct)
            dq[ct] = mma16<2, true, false>(zero4, DOLs, L::PR, Ss + 16 * (CTW * wv + ct), L::PK, lane);
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct)
            dk[ct] = mma16<2, true, false>(zero4, UTs, L::PR, Gs + 16 * (CTW * wv + ct), L::PK, lane);
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) {
            const int cc = 16 * (CTW * wv + ct) + l16;
#pragma unroll
            for (int i = 0; i < 4; ++i) tq[i] += dq[ct][i] * Qs[(4 * lg + i) * L::PK + cc];
        }
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct)
            dq[ct] = mma16<1, true, false>(dq[ct], DPs, L::PC, Ks + 16 * (CTW * wv + ct), L::PK, lane);
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct)
            dk[ct] = mma16<2, true, false, true>(dk[ct], DRBs, L::PR, Ss + 16 * (CTW * wv + ct), L::PK,
                                                 lane);
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) {
            const int cc = 16 * (CTW * wv + ct) + l16;
#pragma unroll
            for (int i = 0; i < 4; ++i) badd(dq[ct][i], rq, ((4 * lg + i) * HDK + cc) * 4);
        }
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct)
            dk[ct] = mma16<1, false, false>(dk[ct], DPs, L::PC, Qs + 16 * (CTW * wv + ct), L::PK, lane);
        const __amdgpu_buffer_rsrc_t rk = rsrc(p.ak + tb * DK, n * HDK * 4);
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) {
            const int t = CTW * wv + ct, cc = 16 * t + l16;
            dk[ct] = mma16<1, true, false>(dk[ct], Ys, L::PC, Ks + 16 * t, L::PK, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i) badd(dk[ct][i], rk, ((4 * lg + i) * HDK + cc) * 4);
        }
        {
            f32x4 gu[2][CTW];
#pragma unroll
            for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
                for (int ct = 0; ct < CTW; ++ct) {
                    const int cc = 16 * (CTW * wv + ct) + l16;
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        gu[a2][ct][i] = Gs[(16 * a2 + 4 * lg + i) * L::PK + cc] * g.lamC;
                    gu[a2][ct] = mma16<1, false, false>(gu[a2][ct], DOLs + 16 * a2, L::PR,
                                                        Qs + 16 * (CTW * wv + ct), L::PK, lane);
                }
#pragma unroll
            for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
                for (int ct = 0; ct < CTW; ++ct) {
                    const int cc = 16 * (CTW * wv + ct) + l16;
                    gu[a2][ct] = mma16<1, false, false, true>(gu[a2][ct], DRBs + 16 * a2, L::PR,
                                                              Ks + 16 * (CTW * wv + ct), L::PK, lane);
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        Gs[(16 * a2 + 4 * lg + i) * L::PK + cc] = gu[a2][ct][i];
                }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) tq[i] = rsum16(tq[i]);
        if (l16 == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) scw[L::TAUO + 16 * wv + 4 * lg + i] = tq[i];
        }
    }
    __syncthreads();
    if (wv == 1) finalize(0, sm + L::SC);
    if (p.ds0) {
#pragma unroll
        for (int it = 0; it < NSV; ++it) {
            const int e4 = tid + it * NTB;
            const int i = e4 / (DK / 4), j = 4 * (e4 % (DK / 4));
            *reinterpret_cast<f32x4*>(p.ds0 + (bh * DV + row0 + i) * DK + j) =
                ld4(Gs + i * L::PK + j);
        }
    }
}

// per token: dbeta and dalpha = d log alpha / alpha (alpha clamped to FLT_MIN
// as in the forward's log) from the row blocks' partials
template <int NRB>
__global__ __launch_bounds__(256) void bwd_reduce_gates(int64_t n, const float* __restrict__ pb,
                                                        const float* __restrict__ pg,
                                                        const float* __restrict__ alpha,
                                                        float* __restrict__ dbeta,
                                                        float* __restrict__ dalpha) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    float b = 0.f, g = 0.f;
#pragma unroll
    for (int r = 0; r < NRB; ++r) {
        b += pb[r * n + i];
        g += pg[r * n + i];
    }
    dbeta[i] = b;
    dalpha[i] = g / fmaxf(alpha[i], 1.17549435e-38f);
}

template <int DK, int DV, typename TIn, typename TD>
hipError_t launch_bwd_t(const BwdArgs& a) {
    constexpr int NRB = DV / RBW;
    const int64_t BH = a.B * a.H, BTH = a.B * a.T * a.H;
    const int64_t nch = (a.T + CB - 1) / CB;
    BwdParams p{};
    p.T = a.T;
    p.H = a.H;
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
    p.ck = reinterpret_cast<float*>(a.workspace);
    float* ta = p.ck + BH * nch * DV * DK;
    p.ta = ta;
    float* wq = ta + BH * nch * 512;           // accumulators of the fused norm's input
    float* wk = wq + BTH * DK;
    p.pb = wk + BTH * DK;
    p.pg = p.pb + NRB * BTH;
    p.l2norm = a.l2norm;
    // dq, dk (or, with the fused norm, the gradients with respect to the
    // normalised q, k) are accumulated in place: zero them first
    p.aq = a.l2norm ? wq : a.dq;
    p.ak = a.l2norm ? wk : a.dk;
    hipError_t e = launch_zero(p.aq, BTH * DK * 4, a.stream);
    if (e == hipSuccess) e = launch_zero(p.ak, BTH * DK * 4, a.stream);
    if (e != hipSuccess) return e;
    const size_t lds = sizeof(float) * BL<DK>::TOTAL;
    auto fn = gdn_bwd_kernel<DK, DV, TIn, TD>;
    // T and AK of every chunk first
    SolveParams sp{};
    sp.T = a.T;
    sp.H = a.H;
    sp.nch = nch;
    sp.nchunks = BH * nch;
    sp.k = a.k;
    sp.alpha = a.alpha;
    sp.beta = a.beta;
    sp.ta = ta;
    sp.l2norm = a.l2norm;
    hipLaunchKernelGGL((gdn_bwd_solve<DK, TIn>), dim3((unsigned)((BH * nch + 3) / 4)), dim3(256), 0,
                       a.stream, sp);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute((const void*)fn,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fn, dim3((unsigned)(BH * NRB)), dim3(NTB), lds, a.stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.l2norm) {
        hipLaunchKernelGGL((bwd_reduce_rows_norm<1, DK, TIn, false>),
                           dim3((unsigned)((BTH + 3) / 4)), dim3(256), 0, a.stream, BTH, wq, wk,
                           nullptr, nullptr, a.q, a.k, nullptr, a.dq, a.dk, nullptr, nullptr);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((bwd_reduce_gates<NRB>), dim3((unsigned)((BTH + 255) / 256)), dim3(256), 0,
                       a.stream, BTH, p.pb, p.pg, a.alpha, a.dbeta, a.dalpha);
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
    const int64_t nch = (T + CB - 1) / CB;
    const int64_t nrb = Dv / RBW;
    const int64_t BTH = B * T * H;
    return sizeof(float) *
           (size_t)(B * H * nch * Dv * Dk + B * H * nch * 512 + 2 * BTH * Dk + 2 * nrb * BTH);
}

hipError_t launch_chunk_bwd(const BwdArgs& a) {
    if (a.Dk == 128 && a.Dv == 128) return launch_bwd_d<128, 128>(a);
    if (a.Dk == 128 && a.Dv == 64) return launch_bwd_d<128, 64>(a);
    if (a.Dk == 64 && a.Dv == 128) return launch_bwd_d<64, 128>(a);
    return launch_bwd_d<64, 64>(a);
}

}  // namespace gdr
