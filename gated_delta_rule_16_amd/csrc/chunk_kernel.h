// The bf16-input kernel of gdr_chunk_fwd (and of its output-gated form):
// the chunkwise UT/WY form of the gated delta rule on gfx950 bf16 matrix
// cores, one fused pass over the sequence.
//
// Chunk algebra (rows of the state S are value channels; within a chunk of
// C = 32 tokens, g_r = sum_{i<=r} log alpha_i, gamma_r = e^{g_r}; this is
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
// The state is carried as S = sigma * S_hat with one scalar sigma per chunk
// (the running product of the chunk decays gamma_C, reset to 1 whenever it
// would drop below 2^-40), so decaying the whole state costs nothing: sigma
// is folded into per-token factors that multiply K S_hat^T and Q S_hat^T
// and divide the update (each at most 2^40 by the reset rule).
//
// Everything that depends only on q, k, alpha, beta of a chunk (A, T, P and
// the per-token factors) is off the sequential path.  The workgroup holds
//
//   team A  RB / 16 waves, wave a owns state rows 16 a .. 16 a + 15 (as S^T
//           tiles in registers) and walks the chunks in order: K S^T and
//           Q S^T, R, V_new = T R, o, and the state update.  Every operand
//           it needs from another wave was written in an earlier period, so
//           it runs without barriers inside a period.
//   team B  four waves, one per SIMD beside the team A waves, running ahead:
//           B3 stages K, scans the gates and computes A for chunk c + 2;
//           for chunk c + 1, B0 computes the per-token factors and sigma, B1
//           solves T = (I + A)^{-1}, and B2 stages Q and V and computes P.
//           Their global loads run two chunks further ahead, in registers.
//
// With GDR_L2NORM_QK (template flag NORM) q and k stay exact bf16 operands:
// k_hat = rho k and q_hat = pi q enter as per-token factors on fp32 results.
// rho_t = 1 / sqrt(|k_t|^2 + eps) comes from the diagonal of B3's Gram
// tiles and multiplies A's rows and columns, FR2, FV and P's columns; pi_t
// from the diagonal of B2's Q Q^T tiles multiplies P's rows and, through
// the factor set, (Q S_hat^T)_t in o.  Both sums are exact bf16 products
// accumulated in fp32 on the matrix cores.
//
// A period ends with one workgroup barrier.  LDS holds two sets of chunk
// tiles (team A reads set c & 1 while team B writes the other), three of K
// and the gate scan (chunk c mod 3), and two copies of A.
//
// Matrix products use v_mfma_f32_16x16x32_bf16 (lane l, g = l / 16,
// m = l % 16: A operand A[m][8 g + e], B operand B[8 g + e][m], C register
// r = C[4 g + r][m]).  A contraction may visit its index in any order as
// long as both operands agree; team A uses kappa(g, e) = 4 g + e for e < 4
// and 16 + 4 g + (e - 4) otherwise, which makes a C tile pair (rows 4 g + r
// of tiles 0 and 1) directly usable as the next product's B operand, so the
// state, R and V_new never leave registers.  Computed operands enter as bf16
// hi/lo pairs (see mfma_common.h).
#pragma once

#include <type_traits>

#include "launch.h"
#include "mfma_common.h"

namespace gdr {

namespace {

constexpr int CH = 32;          // tokens per chunk
constexpr int P36 = 36;         // pitch of the 32-wide fp32 tiles (A, T)
constexpr int P48 = 48;         // pitch of the 32-wide bf16 tiles (T, P hi/lo): 96 bytes
constexpr int NB = 4;           // team B waves
constexpr float kSigmaMin = 9.094947e-13f;   // 2^-40

struct Bf16Params {
    int64_t T, H, BH;
    int64_t bh0;   // first head of this launch (head batches of the gated form)
    const bf16_t *q, *k, *v;
    const float *alpha, *beta;
    const float* s0;
    void* o;       // o, or with the output gate its result y
    float* s_final;
    // output gate (GATE): gate pre-activation [B, T, H, Dv] (bf16 or fp32),
    // RMSNorm weight [Dv] or NULL, epsilon, and the row blocks' exchange of
    // per-token sums of squares ([B H][row blocks][4 chunks][32] words, zero
    // at launch)
    const void* gate;
    bool gate_bf16;
    const float* w;
    float eps;
    unsigned long long* xch;
};

// Per-token factors for team A (token t of the chunk, sigma at chunk start):
//   FR1 = beta_t                 multiplies v_t in R
//   FR2 = beta_t gamma_t sigma   multiplies (K S_hat^T)_t in R
//   FO  = gamma_t sigma          multiplies (Q S_hat^T)_t in o
//   FV  = e^{g_C - g_t} / sigma' scales V_new_t in the update, sigma' the
//                                next chunk's sigma (1 after a reset)
// followed by the reset flag and the factor S_hat is multiplied by on a reset.
// With NORM, FPI = pi_t (1 / |q_t|) follows, written by B2.
enum { FR1 = 0, FR2 = CH, FO = 2 * CH, FV = 3 * CH, FRESET = 4 * CH, FMUL = 4 * CH + 1,
       FPI = 4 * CH + 4 };

template <int DK, int RB, bool NORM, bool GATE = false>
struct Lay {
    static constexpr int PV = RB == 64 ? 80 : 48;   // V row pitch: 8 or 24 banks apart
    // per set (chunk parity)
    static constexpr int Q = 0;                     // Q [32][DK] (swizzled)
    static constexpr int V = Q + CH * DK * 2;       // V [32][PV]
    static constexpr int TH = V + CH * PV * 2;      // T hi, lo [32][P48] (columns kperm'd)
    static constexpr int TL = TH + CH * P48 * 2;
    static constexpr int PH = TL + CH * P48 * 2;    // P hi, lo [32][P48] (columns kperm'd)
    static constexpr int PL = PH + CH * P48 * 2;
    static constexpr int G = PL + CH * P48 * 2;     // per-token factors
    static constexpr int SET = G + (NORM ? 5 * CH + 4 : 4 * CH + 4) * 4;
    // per chunk mod 3: K twice -- in operand order (swizzled) for the
    // products over the key dim, and row-major [32][DK + 16] for the
    // transposed reads -- and the gate scan (g, beta, with NORM rho)
    static constexpr int PKN = DK + 16;
    static constexpr int GRS = (NORM ? 3 : 2) * CH * 4;
    static constexpr int KSLOT = CH * DK * 2 + CH * PKN * 2;
    static constexpr int KR = 2 * SET;
    static constexpr int GR = KR + 3 * KSLOT;
    static constexpr int AF = GR + 3 * GRS;         // A fp32 [32][P36], two copies
    static constexpr int TF = AF + 2 * CH * P36 * 4;   // B1 private: T fp32 [32][P36]
    // output gate: team A's per-token partial sums of squares of o, three
    // chunks [3][RB / 16][32], and w SiLU(gate) of three chunks as B0
    // formed it, token-major fp32 [32][GP] (GP = RB + 8 elements: rows 32
    // bytes apart in banks)
    static constexpr int GP = RB + 8;
    static constexpr int PSQ = TF + CH * P36 * 4;
    static constexpr int GGR = PSQ + (GATE ? 3 * (RB / 16) * CH * 4 : 0);
    static constexpr int GGS = CH * GP * 4;            // one chunk, fp32 gate
    static constexpr int TOTAL = GGR + (GATE ? 3 * GGS : 0);
    static_assert(SET % 16 == 0 && (CH * PV * 2) % 16 == 0, "alignment");
};

// Operand order of a contraction over 32 columns: column 16 h + 4 q + e of
// each block of 32 (h < 2, q < 4, e < 4) is stored at 8 q + 4 h + e, so the
// 8 values that lane group q feeds an MFMA in kappa order are one 16-byte
// read.  K, Q (per 32 key channels), T and P (over their 32 tokens) are
// stored this way.
__device__ __forceinline__ int kperm(int c) {
    return (c & ~31) | ((c & 12) << 1) | ((c & 16) >> 2) | (c & 3);
}

// Element offset of (row, stored column pc) in an operand-order K or Q
// tile: 16-byte unit u of row r is stored at u ^ (r mod DK / 8), so the 16
// rows one lane group reads at one unit fall on distinct banks.
template <int DK>
__device__ __forceinline__ int kq_at(int row, int pc) {
    return row * DK + ((((pc >> 3) ^ (row & (DK / 8 - 1)))) << 3) + (pc & 7);
}

// Orders this wave's earlier LDS writes before its later LDS reads.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ void split44(const f32x4& a, const f32x4& b, bf16x8& h, bf16x8& l) {
    split8(f32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]}, h, l);
}

__device__ __forceinline__ void st8(bf16_t* p, const uint2& x) {
    *reinterpret_cast<uint2*>(p) = x;
}

// NOO: no o at all (the sequence split's state passes want only the final
// state): team A skips Q S^T, P V_new and the stores, B2 stages V only.
template <int DK, int DV, int RB, typename TOut, bool NORM, bool GATE = false, bool NOO = false>
__global__ __launch_bounds__(64 * (RB / 16 + NB)) void chunk_bf16_kernel(Bf16Params p) {
    using L = Lay<DK, RB, NORM, GATE>;
    constexpr int NA = RB / 16;   // team A waves
    constexpr int KJ = DK / 32;   // 32-deep contraction steps over the key dim
    constexpr int NS = DK / 16;   // S^T tiles per team A wave
    constexpr int NRB = DV / RB;
    constexpr int VC = RB / 8;    // 16-byte pieces per value row slice
    constexpr int VL = CH * VC / 64;
    static_assert(VL * 64 == CH * VC, "value load split");
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
    const int64_t bh = p.bh0 + (slot / NRB) * 8 + (blockIdx.x & 7);
    const int rbk = (int)(slot % NRB);
    if (bh >= p.BH) return;
    const int64_t H = p.H, T = p.T;
    const int64_t h = bh % H;
    const int64_t b = bh / H;
    const int row0 = rbk * RB;
    const int64_t nch = (T + CH - 1) / CH;

    auto setp = [&](int64_t c, int off) { return smem + (int)(c & 1) * L::SET + off; };
    auto afp = [&](int64_t c) {
        return reinterpret_cast<float*>(smem + L::AF + (int)(c & 1) * CH * P36 * 4);
    };
    auto kring = [&](int64_t c) {
        return reinterpret_cast<bf16_t*>(smem + L::KR + (int)(c % 3) * L::KSLOT);
    };
    auto gring = [&](int64_t c) {
        return reinterpret_cast<float*>(smem + L::GR + (int)(c % 3) * L::GRS);
    };

    // T and P vanish above their diagonal 16x16 blocks (rows 0..15,
    // columns 16..31); those entries are never written afterwards.
    for (int e = tid; e < 2 * 4 * 256; e += blockDim.x) {
        const int set = e >> 10, arr = (e >> 8) & 3, r = (e >> 4) & 15, s = 16 + (e & 15);
        const int off = arr == 0 ? L::TH : arr == 1 ? L::TL : arr == 2 ? L::PH : L::PL;
        reinterpret_cast<bf16_t*>(smem + set * L::SET + off)[r * P48 + kperm(s)] = 0;
    }

    const int64_t tstride = H * DK;   // elements between tokens of q, k
    const bf16_t* kbase = p.k + (b * T * H + h) * DK;
    const bf16_t* qbase = p.q + (b * T * H + h) * DK;
    const bf16_t* vbase = p.v ? p.v + (b * T * H + h) * DV + row0 : nullptr;
    const float* abase = p.alpha + b * T * H + h;
    const float* bbase = p.beta + b * T * H + h;

    if (wave < NA) {
        // =========================== team A ================================
        const int a = wave;
        const int i = 16 * a + m;   // state row (within the block) of this lane
        // sa[t][r] = S_hat[i][16 t + 4 g + r]
        f32x4 sa[NS];
#pragma unroll
        for (int t = 0; t < NS; ++t) {
            sa[t] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (p.s0)
                sa[t] = *reinterpret_cast<const f32x4*>(p.s0 + ((bh * DV + row0 + i) * DK + 16 * t +
                                                                4 * g));
        }
        // S_hat as hi/lo B operands (contraction index kappa over 32 key
        // channels per step); refreshed at the end of every chunk
        bf16x8 sh[KJ], sl[KJ];
#pragma unroll
        for (int j = 0; j < KJ; ++j) split44(sa[2 * j], sa[2 * j + 1], sh[j], sl[j]);
        // two periods of pipeline fill: A of chunks 0 and 1, then the rest
        // of chunk 0
        lds_barrier();
        lds_barrier();
        // o goes out through buffer stores: a per-chunk resource whose range
        // ends after the chunk's last token (stores past it are dropped) and
        // fixed per-lane byte offsets o[t0 + 16 rt + 4 g + r][row0 + i]
        uint32_t ooff[2][4];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                ooff[rt][r] = (uint32_t)(((16 * rt + 4 * g + r) * (int)(H * DV) + row0 + i) *
                                         (int)sizeof(TOut));
        TOut* obase = reinterpret_cast<TOut*>(p.o) + (b * T * H + h) * DV;

        // ---- output gate (GATE): y = o / sqrt(mean o^2 + eps) w SiLU(gate) ----
        // A token's mean square runs over all DV rows: the wave's 16 rows are
        // summed in registers, the workgroup's waves through LDS at the next
        // barrier, and the row blocks of the head through `xch`, one period
        // later again.  o of a chunk is held (gated) until then.  A row block
        // publishes chunk c - 1 at the top of period c and finishes period c
        // only after the others have published chunk c - 2, so none is more
        // than two periods ahead of another, and a ring of four chunks in
        // `xch` is never overwritten before it is read.
        //   lanes m, m ^ 1 of each 16-lane group own token index
        //   jt = 4 b3 + 2 b2 + b1 (bits of m) of the group's 8 tokens
        const int jt = 4 * ((m >> 3) & 1) + 2 * ((m >> 2) & 1) + ((m >> 1) & 1);
        const int tok = 16 * (jt >> 2) + 4 * g + (jt & 3);
        float* psq = reinterpret_cast<float*>(smem + L::PSQ);   // [3][NA][CH]
        // chunk slots in 32-bit arithmetic (the call keeps T below 2^36)
        auto mod3 = [](int64_t cn) { return (int)((uint32_t)cn % 3u); };
        auto mod4 = [](int64_t cn) { return (int)((uint32_t)cn & 3u); };
        // this lane's token in the head's exchange words
        unsigned long long* xhead = p.xch + bh * NRB * 4 * CH + tok;
        // squares of o summed over the wave's 16 rows (a reduce-scatter over
        // the DPP row: partners lane ^ 15, ^ 7, ^ 3, ^ 1, keeping half each
        // time), written to LDS by the owners of each token
        auto gate_psum = [&](const f32x4 (&ov)[2], int64_t cn) {
            float v[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = ov[e >> 2][e & 3] * ov[e >> 2][e & 3];
            const bool b3 = (m & 8) != 0, b2 = (m & 4) != 0, b1 = (m & 2) != 0;
            float s4[4], s2[2];
#pragma unroll
            for (int k = 0; k < 4; ++k)
                s4[k] = (b3 ? v[4 + k] : v[k]) + dpp_mov<0x140>(b3 ? v[k] : v[4 + k]);
#pragma unroll
            for (int k = 0; k < 2; ++k)
                s2[k] = (b2 ? s4[2 + k] : s4[k]) + dpp_mov<0x141>(b2 ? s4[k] : s4[2 + k]);
            float s1 = (b1 ? s2[1] : s2[0]) + dpp_mov<0x1B>(b1 ? s2[0] : s2[1]);
            s1 += dpp_mov<0xB1>(s1);
            if (!(m & 1)) psq[(mod3(cn) * NA + a) * CH + tok] = s1;
        };
        // the workgroup's sum for the lane's token; wave 0 publishes it to
        // the head's other row blocks, tagged with the chunk
        auto gate_wsum = [&](int64_t cn) {
            float s = 0.f;
#pragma unroll
            for (int aa = 0; aa < NA; ++aa) s += psq[(mod3(cn) * NA + aa) * CH + tok];
            if (NRB > 1 && a == 0 && !(m & 1)) {
                const unsigned long long word =
                    ((unsigned long long)(uint32_t)(cn + 1) << 32) | __float_as_uint(s);
                __hip_atomic_store(xhead + (rbk * 4 + mod4(cn)) * CH, word,
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            return s;
        };
        // o w SiLU(gate) for chunk cn, the gate staged by B0 token-major;
        // SiLU(x) = x / (1 + e^-x).  The lane's gate values (tokens 16 rt +
        // 4 g + r, channel i): bf16 by two transposed reads, fp32 one by one.
        auto gate_apply = [&](const f32x4 (&ov)[2], int64_t cn, f32x4 (&og)[2]) {
            // w SiLU(g) of the chunk, formed by B0 when it staged the gate
            const float* gf = reinterpret_cast<const float*>(smem + L::GGR + mod3(cn) * L::GGS);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int r = 0; r < 4; ++r) og[rt][r] = ov[rt][r] * gf[(16 * rt + 4 * g + r) * L::GP + i];
        };
        // the other row blocks' words for chunk cn, read once early in a
        // period (their round trip overlaps its work)
        constexpr int NP = NRB > 1 ? NRB - 1 : 1;
        auto xsrc = [&](int64_t cn, int k) {   // k-th other row block
            const int rb = k + (k >= rbk ? 1 : 0);
            return xhead + (rb * 4 + mod4(cn)) * CH;
        };
        auto gate_fetch = [&](int64_t cn, unsigned long long (&pw)[NP]) {
#pragma unroll
            for (int k = 0; k < NRB - 1; ++k)
                pw[k] = __hip_atomic_load(xsrc(cn, k), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        };
        // y of chunk cn: the other row blocks' sums (a word not yet tagged
        // with the chunk is read again, with a bounded spin; a sum that never
        // arrives leaves NaN), then 1 / rms of the lane's tokens from their
        // owners in its 16-lane row (token 16 rt + 4 g + r is owned by lane
        // 8 rt + 2 r of the row: a row broadcast), then the stores
        auto gate_out = [&](int64_t cn, const f32x4 (&og)[2], float wsum,
                            unsigned long long (&pw)[NP]) {
            float tot = wsum;
            const uint32_t tag = (uint32_t)(cn + 1);
#pragma unroll
            for (int k = 0; k < NRB - 1; ++k) {
                unsigned long long x = pw[k];
                // the usual case is one uniform test: every word has arrived
                if (__builtin_amdgcn_ballot_w64((uint32_t)(x >> 32) != tag) != 0) {
#pragma nounroll
                    for (int spin = 0; spin < (1 << 18); ++spin) {
                        if ((uint32_t)(x >> 32) == tag) break;
                        __builtin_amdgcn_s_sleep(2);
                        x = __hip_atomic_load(xsrc(cn, k), __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
                    }
                }
                tot += (uint32_t)(x >> 32) == tag ? __uint_as_float((uint32_t)x) : __builtin_nanf("");
            }
            const float rr = rsqrtf(tot * (1.f / DV) + p.eps);
            const f32x4 rv[2] = {f32x4{dpp_mov<0x150>(rr), dpp_mov<0x152>(rr), dpp_mov<0x154>(rr),
                                       dpp_mov<0x156>(rr)},
                                 f32x4{dpp_mov<0x158>(rr), dpp_mov<0x15A>(rr), dpp_mov<0x15C>(rr),
                                       dpp_mov<0x15E>(rr)}};
            const int n = (int)min((int64_t)CH, T - cn * CH);
            const __amdgpu_buffer_rsrc_t ores = __builtin_amdgcn_make_buffer_rsrc(
                obase + cn * CH * H * DV, (short)0, n * (int)(H * DV * sizeof(TOut)), 0x00020000);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const f32x4 y = og[rt] * rv[rt];
                if constexpr (sizeof(TOut) == 4) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y[r]), ores,
                                                              (int)ooff[rt][r], 0, 0);
                } else {
                    store4_bf16(y, ores, ooff[rt]);
                }
            }
        };
        // held across periods: o of the previous chunk, the gated o and
        // workgroup sum of the one before
        f32x4 o_prev[2] = {}, og2[2] = {};
        float ws2 = 0.f;

        for (int64_t c = 0; c < nch; ++c) {
            // output gate, at the top of the period: the other row blocks'
            // words for the chunk whose y this period writes come in, and the
            // previous chunk's workgroup sum (complete since the barrier) goes
            // out to them; both have the period's work to arrive.  The read
            // goes first: a coherent read issued after a coherent write waits
            // for the write to reach memory.
            unsigned long long pw[NP];   // read only for c >= 2
            float ws1 = 0.f;
            if constexpr (GATE) {
                if (c >= 2) gate_fetch(c - 2, pw);
                if (c >= 1) ws1 = gate_wsum(c - 1);
            }
            const bf16_t* Kb = kring(c);
            const bf16_t* Qb = reinterpret_cast<const bf16_t*>(setp(c, L::Q));
            const bf16_t* Vb = reinterpret_cast<const bf16_t*>(setp(c, L::V));
            const bf16_t* Th = reinterpret_cast<const bf16_t*>(setp(c, L::TH));
            const bf16_t* Tl = reinterpret_cast<const bf16_t*>(setp(c, L::TL));
            const bf16_t* Ph = reinterpret_cast<const bf16_t*>(setp(c, L::PH));
            const bf16_t* Pl = reinterpret_cast<const bf16_t*>(setp(c, L::PL));
            const float* G = reinterpret_cast<const float*>(setp(c, L::G));

            // The state chain K S^T -> R -> V_new -> update -> next split
            // runs first in each phase; Q S^T, o and the stores fill the
            // matrix-core and VALU gaps around it.
            // ---- K S_hat^T (state chain) -----------------------------------
            bf16x8 kf[2][KJ], qf[2][KJ];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int j = 0; j < KJ; ++j)
                    kf[tt][j] = *reinterpret_cast<const bf16x8*>(Kb + kq_at<DK>(16 * tt + m, 32 * j + 8 * g));
            if constexpr (!NOO) {
#pragma unroll
                for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                    for (int j = 0; j < KJ; ++j)
                        qf[tt][j] = *reinterpret_cast<const bf16x8*>(Qb + kq_at<DK>(16 * tt + m, 32 * j + 8 * g));
            }
            f32x4 ks[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
            for (int j = 0; j < KJ; ++j)
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    ks[tt] = mfma16(kf[tt][j], sh[j], ks[tt]);
                    ks[tt] = mfma16(kf[tt][j], sl[j], ks[tt]);
                }
            // operands of the rest of the chunk, read while the products run
            f32x4 fr1[2], fr2[2], fo[2], fv[2];
            s16x4 vv[2];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                fr1[tt] = *reinterpret_cast<const f32x4*>(G + FR1 + 16 * tt + 4 * g);
                fr2[tt] = *reinterpret_cast<const f32x4*>(G + FR2 + 16 * tt + 4 * g);
                // V[16 tt + 4 g + r][i], r = 0..3, by a transposed read
                vv[tt] = lds_tr16(Vb + (16 * tt + 4 * g + (m >> 2)) * L::PV + 16 * a + 4 * (m & 3));
            }
            bf16x8 th[2], tl[2];
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                const int at = (16 * rt + m) * P48 + 8 * g;
                th[rt] = *reinterpret_cast<const bf16x8*>(Th + at);
                tl[rt] = *reinterpret_cast<const bf16x8*>(Tl + at);
            }
            __builtin_amdgcn_sched_barrier(0);

            // ---- R = FR1 V - FR2 (K S_hat^T), beside Q S_hat^T -------------
            f32x4 qs[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
            if constexpr (!NOO) {
#pragma unroll
                for (int j = 0; j < KJ; ++j)
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt) {
                        qs[tt] = mfma16(qf[tt][j], sh[j], qs[tt]);
                        qs[tt] = mfma16(qf[tt][j], sl[j], qs[tt]);
                    }
            }
            f32x4 rr[2];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    rr[tt][r] = __builtin_fmaf(-fr2[tt][r], ks[tt][r],
                                               fr1[tt][r] * bf2f((bf16_t)vv[tt][r]));
            bf16x8 rh, rl;
            split44(rr[0], rr[1], rh, rl);
            if constexpr (!NOO) {
#pragma unroll
                for (int u = 0; u < 4 * KJ; ++u) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);   // three VALU
                }
            }
            __builtin_amdgcn_sched_barrier(0);

            // ---- V_new = T R (state chain) ---------------------------------
            f32x4 vn[2];
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                vn[rt] = mfma16(th[rt], rh, f32x4{0.f, 0.f, 0.f, 0.f});
                vn[rt] = mfma16(th[rt], rl, vn[rt]);
                vn[rt] = mfma16(tl[rt], rh, vn[rt]);
            }
            bf16x8 ph[2], pl[2], kt[NS];
#pragma unroll
            for (int rt = 0; rt < 2; ++rt) {
                if constexpr (!NOO) {
                    const int at = (16 * rt + m) * P48 + 8 * g;
                    ph[rt] = *reinterpret_cast<const bf16x8*>(Ph + at);
                    pl[rt] = *reinterpret_cast<const bf16x8*>(Pl + at);
                    fo[rt] = *reinterpret_cast<const f32x4*>(G + FO + 16 * rt + 4 * g);
                    if constexpr (NORM)
                        fo[rt] *= *reinterpret_cast<const f32x4*>(G + FPI + 16 * rt + 4 * g);
                }
                fv[rt] = *reinterpret_cast<const f32x4*>(G + FV + 16 * rt + 4 * g);
            }
#pragma unroll
            for (int t = 0; t < NS; ++t) {
                // K[kappa(g, e)][16 t + m] by two transposed reads
                const bf16_t* kn = Kb + CH * DK + (4 * g + (m >> 2)) * L::PKN + 16 * t + 4 * (m & 3);
                const s16x4 x0 = lds_tr16(kn);
                const s16x4 x1 = lds_tr16(kn + 16 * L::PKN);
                const s16x4 x2[2] = {x0, x1};
                kt[t] = __builtin_bit_cast(bf16x8, x2);
            }
            __builtin_amdgcn_sched_barrier(0);

            // ---- update operands first, then o = FO (Q S_hat^T) + P V_new --
            bf16x8 nh, nl, mh, ml;
            split44(vn[0] * fv[0], vn[1] * fv[1], mh, ml);
            split44(vn[0], vn[1], nh, nl);
            f32x4 o[2];
            if constexpr (!NOO) {
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    o[rt] = qs[rt] * fo[rt];
                    o[rt] = mfma16(ph[rt], nh, o[rt]);
                    o[rt] = mfma16(ph[rt], nl, o[rt]);
                    o[rt] = mfma16(pl[rt], nh, o[rt]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);

            if (__builtin_amdgcn_readfirstlane(__float_as_int(G[FRESET])) != 0) {
                // sigma restarts at 1: S_hat takes the chunk decay now
                const float smul = G[FMUL];
#pragma unroll
                for (int t = 0; t < NS; ++t) sa[t] *= smul;
            }

            // ---- S_hat^T += K^T (FV V_new), next chunk's split beside it ---
#pragma unroll
            for (int t = 0; t < NS; ++t) {
                sa[t] = mfma16(kt[t], mh, sa[t]);
                sa[t] = mfma16(kt[t], ml, sa[t]);
            }
#pragma unroll
            for (int j = 0; j < KJ; ++j) split44(sa[2 * j], sa[2 * j + 1], sh[j], sl[j]);
            if constexpr (!GATE && !NOO) {
                // no o (p.o NULL: a pass that only wants the final state):
                // an empty range drops every store
                const int64_t t0 = c * CH;
                const int n = p.o ? (int)min((int64_t)CH, T - t0) : 0;
                const __amdgpu_buffer_rsrc_t ores = __builtin_amdgcn_make_buffer_rsrc(
                    obase + t0 * H * DV, (short)0, n * (int)(H * DV * sizeof(TOut)), 0x00020000);
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    if constexpr (sizeof(TOut) == 4) {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(o[rt][r]), ores,
                                                                  (int)ooff[rt][r], 0, 0);
                    } else {
                        store4_bf16(o[rt], ores, ooff[rt]);
                    }
                }
            }
            // products of tile pairs 0, 1 first, then each pair's split
            // beside the next pair's products, the stores before the last
            __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
#pragma unroll
            for (int j = 0; j + 2 < KJ; ++j) {
                __builtin_amdgcn_sched_group_barrier(0x002, 24, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x002, 24, 0);
            if constexpr (!NOO) __builtin_amdgcn_sched_group_barrier(0x040, 8, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 24, 0);
            if constexpr (GATE) {
                // this chunk's partial sums and gate; the previous chunk's
                // workgroup sum; y of the chunk before that
                gate_psum(o, c);
                f32x4 og1[2];
                if (c >= 1) gate_apply(o_prev, c - 1, og1);
                if (c >= 2) gate_out(c - 2, og2, ws2, pw);
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    og2[rt] = og1[rt];
                    o_prev[rt] = o[rt];
                }
                ws2 = ws1;
            }
            lds_barrier();
        }
        if constexpr (GATE) {
            // one more period: the last chunk's workgroup sum, then y of the
            // last two chunks
            lds_barrier();
            f32x4 og1[2];
            unsigned long long pw[NP] = {}, pw1[NP] = {};
            if (nch >= 2) gate_fetch(nch - 2, pw);
            const float ws1 = gate_wsum(nch - 1);
            gate_apply(o_prev, nch - 1, og1);
            if (nch >= 2) gate_out(nch - 2, og2, ws2, pw);
            gate_fetch(nch - 1, pw1);
            gate_out(nch - 1, og1, ws1, pw1);
        }
        if (p.s_final) {
            // the last chunk always resets sigma to 1, so S_hat is S here
#pragma unroll
            for (int t = 0; t < NS; ++t)
                *reinterpret_cast<f32x4*>(p.s_final + ((bh * DV + row0 + i) * DK + 16 * t + 4 * g)) =
                    sa[t];
        }
        return;
    }

    // ============================== team B =================================
    const int bw = wave - NA;
    // Team B shares each SIMD with a team A wave; ahead of team A's
    // instructions it finishes its short dependent chains within the period.
    __builtin_amdgcn_s_setprio(2);
    // Global loads: a uniform chunk base plus a 32-bit lane offset.  Rows
    // past the end of the sequence repeat its last token: they only ever
    // meet beta = 0 (rows of A, R and V_new) or are not stored (o).
    auto last_row = [&](int64_t cn) { return (int)min((int64_t)CH - 1, T - 1 - cn * CH); };
    // lane (g, m) gets rows 16 tt + m, elements 32 j + 8 g .. + 7 -- the
    // natural operand layout of the 16x16x32 product
    auto load_k = [&](int64_t cn, u32x4 (&kr)[2][KJ], const bf16_t* base) {
        const int last = last_row(cn);
        const char* cb = reinterpret_cast<const char*>(base + cn * CH * tstride);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const uint32_t off = (uint32_t)(min(16 * tt + m, last) * (int)tstride + 8 * g) * 2u;
#pragma unroll
            for (int j = 0; j < KJ; ++j)
                kr[tt][j] = *reinterpret_cast<const u32x4*>(cb + off + 64 * j);
        }
    };
    // stores rows 16 tt + m, elements 32 j + 8 g .. + 7 into a K or Q tile
    auto stage_kq = [&](bf16_t* dst, const u32x4 (&kr)[2][KJ]) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int j = 0; j < KJ; ++j) {
                const int row = 16 * tt + m;
                st8(dst + kq_at<DK>(row, kperm(32 * j + 8 * g)), uint2{kr[tt][j][0], kr[tt][j][1]});
                st8(dst + kq_at<DK>(row, kperm(32 * j + 8 * g + 4)), uint2{kr[tt][j][2], kr[tt][j][3]});
            }
    };
    // g and beta of the chunk's tokens from the gate ring: gq, bq for tokens
    // 16 rt + m; gk for tokens 16 st + 4 g .. + 3; with NORM rho of the
    // same tokens in rq and rk (1 otherwise)
    struct Gates {
        float gq[2], bq[2], rq[2];
        f32x4 gk[2], rk[2];
    };
    auto read_gates = [&](const float* gr, auto rhoc) {
        constexpr bool RHO = decltype(rhoc)::value;
        Gates z;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            z.gq[u] = gr[16 * u + m];
            z.bq[u] = gr[CH + 16 * u + m];
            z.gk[u] = *reinterpret_cast<const f32x4*>(gr + 16 * u + 4 * g);
            z.rq[u] = 1.f;
            z.rk[u] = f32x4{1.f, 1.f, 1.f, 1.f};
            if constexpr (RHO) {
                z.rq[u] = gr[2 * CH + 16 * u + m];
                z.rk[u] = *reinterpret_cast<const f32x4*>(gr + 2 * CH + 16 * u + 4 * g);
            }
        }
        return z;
    };

    // A role prepares chunk x in period x - lead (periods run from -2 to
    // nch - 1, each closed by the workgroup barrier).  Loading roles keep two
    // chunks in flight in three register buffers (chunk x in buffer x mod 3);
    // loads are unconditional (an index past the end repeats the last chunk)
    // so that the wait before each prepare covers just its buffer.
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
        if constexpr (GATE) lds_barrier();   // team A's output-gate period
    };
    auto run_noload = [&](int lead, auto&& prepare) {
        for (int e = 0; e < 2 - lead; ++e) lds_barrier();
        for (int64_t x = 0; x < nch; ++x) {
            prepare(x);
            lds_barrier();
        }
        for (int e = 0; e < lead; ++e) lds_barrier();
        if constexpr (GATE) lds_barrier();   // team A's output-gate period
    };

    if (bw == 0) {
        // ------------------------ B0: per-token factors ----------------------
        float sigma = 1.f;   // sigma at the start of the chunk being prepared
        auto prepare = [&](int64_t cn) {
            const float* gr = gring(cn);
            float* G = reinterpret_cast<float*>(setp(cn, L::G));
            const float gx = gr[lane & 31], be = gr[CH + (lane & 31)];
            const float rho = NORM ? gr[2 * CH + (lane & 31)] : 1.f;
            const float gC = gr[CH - 1];
            // sigma' = sigma gamma_C; a reset keeps S_hat = S from here on.
            // The last chunk always resets so that the final S_hat is S.
            const float s1 = sigma * __expf(gC);
            const bool reset = s1 < kSigmaMin || cn == nch - 1;
            const float fo = sigma * __expf(gx);
            const float dec = __expf(gC - gx);
            if (lane < CH) {
                G[FR1 + lane] = be;
                G[FR2 + lane] = be * fo * rho;
                G[FO + lane] = fo;
                G[FV + lane] = (reset ? dec : dec / s1) * rho;
            }
            if (lane == 0) {
                G[FRESET] = reset ? 1.f : 0.f;
                G[FMUL] = s1;
            }
            sigma = reset ? 1.f : s1;
        };
        if constexpr (GATE) {
            // and the output gate's factor of the chunk, for team A one period
            // later: w SiLU(g) over 32 tokens x RB channels, token-major fp32
            // in LDS; the gate is read in 16-byte pieces (VPC per token, GPL
            // per lane, EPC elements each), every piece of a lane at the same
            // channels, so the lane's w values are loaded once.  B0 has the
            // slack of the period; team A only multiplies.
            auto stage = [&](auto esz) {
                constexpr int ES = decltype(esz)::value;   // gate element bytes
                constexpr int VPC = RB * ES / 16, NPC = CH * VPC, GPL = (NPC + 63) / 64;
                constexpr int EPC = 16 / ES;
                static_assert(NPC % 64 == 0 && 64 % VPC == 0, "gate pieces");
                struct GBuf {
                    u32x4 v[GPL];
                };
                const int c0 = (lane % VPC) * EPC;   // this lane's first channel
                float wv[EPC];
#pragma unroll
                for (int e = 0; e < EPC; ++e) wv[e] = p.w ? p.w[row0 + c0 + e] : 1.f;
                const char* gbase = reinterpret_cast<const char*>(p.gate);
                auto load = [&](int64_t cn, GBuf& f) {
                    const int last = last_row(cn);
                    const char* cb = gbase + ((b * T * H + h) * DV + row0 + cn * CH * H * DV) * ES;
#pragma unroll
                    for (int u = 0; u < GPL; ++u) {
                        const int pc = lane + 64 * u;
                        if (NPC % 64 == 0 || pc < NPC) {
                            const uint32_t off = (uint32_t)(min(pc / VPC, last) * (int)(H * DV) * ES +
                                                            16 * (pc % VPC));
                            f.v[u] = *reinterpret_cast<const u32x4*>(cb + off);
                        }
                    }
                };
                auto prepare_g = [&](int64_t cn, const GBuf& f) {
                    prepare(cn);
                    float* gs = reinterpret_cast<float*>(smem + L::GGR + (int)(cn % 3) * L::GGS);
#pragma unroll
                    for (int u = 0; u < GPL; ++u) {
                        const int t = (lane + 64 * u) / VPC;
                        float sv[EPC];
#pragma unroll
                        for (int e = 0; e < EPC; ++e) {
                            float x;
                            if constexpr (ES == 2) {
                                const uint32_t wd = f.v[u][e >> 1];
                                x = __uint_as_float((e & 1) ? (wd & 0xffff0000u) : (wd << 16));
                            } else {
                                x = __uint_as_float(f.v[u][e]);
                            }
                            sv[e] = wv[e] * (x * __builtin_amdgcn_rcpf(1.f + __expf(-x)));
                        }
#pragma unroll
                        for (int h4 = 0; h4 < EPC / 4; ++h4)
                            *reinterpret_cast<f32x4*>(gs + t * L::GP + c0 + 4 * h4) =
                                f32x4{sv[4 * h4], sv[4 * h4 + 1], sv[4 * h4 + 2], sv[4 * h4 + 3]};
                    }
                };
                GBuf fa, fb, fc;
                run(1, load, prepare_g, fa, fb, fc);
            };
            if (p.gate_bf16)
                stage(std::integral_constant<int, 2>{});
            else
                stage(std::integral_constant<int, 4>{});
        } else {
            run_noload(1, prepare);
        }
    } else if (bw == 1) {
        // ----------------------- B1: T = (I + A)^{-1} -----------------------
        float* Tf = reinterpret_cast<float*>(smem + L::TF);
        auto prepare = [&](int64_t cn) {
            const float* Af = afp(cn);
            bf16_t* Th = reinterpret_cast<bf16_t*>(setp(cn, L::TH));
            bf16_t* Tl = reinterpret_cast<bf16_t*>(setp(cn, L::TL));
            // Diagonal blocks X = (I + L)^{-1}, L = A's block `blk`: lane pair
            // (blk, rr) builds row rr from X = I - X L, columns right to left,
            // pushing each finished entry into the columns left of it.
            {
                const int blk = lane >> 5, rr = (lane >> 1) & 15, half = lane & 1;
                const float* Lb = Af + 16 * blk * P36 + 16 * blk;
                // all of L's strictly lower part (row cp, columns < cp) in
                // registers first, so the 16 dependent steps wait on nothing
                f32x4 lrow[16][4];
#pragma unroll
                for (int cp = 1; cp < 16; ++cp)
#pragma unroll
                    for (int q4 = 0; q4 < (cp + 3) / 4; ++q4)
                        lrow[cp][q4] = *reinterpret_cast<const f32x4*>(Lb + cp * P36 + 4 * q4);
                __builtin_amdgcn_sched_barrier(0);
                float acc2[16], x[16];
#pragma unroll
                for (int cc = 0; cc < 16; ++cc) acc2[cc] = 0.f;
#pragma unroll
                for (int cp = 15; cp >= 0; --cp) {
                    x[cp] = (rr == cp ? 1.f : 0.f) - acc2[cp];
#pragma unroll
                    for (int q4 = 0; q4 < (cp + 3) / 4; ++q4)
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (4 * q4 + e < cp) acc2[4 * q4 + e] += x[cp] * lrow[cp][q4][e];
                }
                // columns 8 half .. 8 half + 7 of row 16 blk + rr (bitwise
                // select: a conditional here becomes an indexed private array)
                const int row = 16 * blk + rr, col = 16 * blk + 8 * half;
                const uint32_t msk = half ? 0xffffffffu : 0u;
                float xs[8];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    xs[e] = __uint_as_float((__float_as_uint(x[8 + e]) & msk) |
                                            (__float_as_uint(x[e]) & ~msk));
                *reinterpret_cast<f32x4*>(Tf + row * P36 + col) = f32x4{xs[0], xs[1], xs[2], xs[3]};
                *reinterpret_cast<f32x4*>(Tf + row * P36 + col + 4) =
                    f32x4{xs[4], xs[5], xs[6], xs[7]};
                bf16x8 xh, xl;
                split8(f32x8{xs[0], xs[1], xs[2], xs[3], xs[4], xs[5], xs[6], xs[7]}, xh, xl);
                const u32x4 uh = __builtin_bit_cast(u32x4, xh), ul = __builtin_bit_cast(u32x4, xl);
                st8(Th + row * P48 + kperm(col), uint2{uh[0], uh[1]});
                st8(Th + row * P48 + kperm(col + 4), uint2{uh[2], uh[3]});
                st8(Tl + row * P48 + kperm(col), uint2{ul[0], ul[1]});
                st8(Tl + row * P48 + kperm(col + 4), uint2{ul[2], ul[3]});
            }
            wave_lds_sync();
            // T_10 = -T_11 A_10 T_00 on fp32 16x16x4 matrix cores:
            // Y = A_10 T_00 (C layout Y[4 g + r][m]), then -T_10^T = Y^T T_11^T
            // with the contraction order 4 g + kk so that Y's registers are
            // its A operand as they stand.
            float ya[4], yb[4], tb[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                ya[kk] = Af[(16 + m) * P36 + 4 * kk + g];
                yb[kk] = Tf[(4 * kk + g) * P36 + m];
                tb[kk] = Tf[(16 + m) * P36 + 16 + 4 * g + kk];
            }
            __builtin_amdgcn_sched_barrier(0);
            f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) y = mfma_f32(ya[kk], yb[kk], y);
            f32x4 t10 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) t10 = mfma_f32(y[kk], tb[kk], t10);
            uint2 vh, vl;
            split2(-t10[0], -t10[1], vh.x, vl.x);
            split2(-t10[2], -t10[3], vh.y, vl.y);
            st8(Th + (16 + m) * P48 + kperm(4 * g), vh);
            st8(Tl + (16 + m) * P48 + kperm(4 * g), vl);
        };
        run_noload(1, prepare);
    } else if (bw == 2) {
        // ---------------------- B2: Q and V staging, P ----------------------
        struct Buf {
            u32x4 q[2][KJ];
            u32x4 v[VL];
        };
        auto load = [&](int64_t cn, Buf& f) {
            if constexpr (!NOO) load_k(cn, f.q, qbase);
            if (!p.v) {
                // no v: v = 0 (the sequence split's transition pass)
#pragma unroll
                for (int u = 0; u < VL; ++u) f.v[u] = u32x4{0u, 0u, 0u, 0u};
                return;
            }
            const int last = last_row(cn);
            const char* cb = reinterpret_cast<const char*>(vbase + cn * CH * H * DV);
#pragma unroll
            for (int u = 0; u < VL; ++u) {
                const int pc = lane + 64 * u;
                const uint32_t off = (uint32_t)(min(pc / VC, last) * (int)(H * DV) + 8 * (pc % VC)) * 2u;
                f.v[u] = *reinterpret_cast<const u32x4*>(cb + off);
            }
        };
        auto prepare = [&](int64_t cn, const Buf& f) {
            bf16_t* Qb = reinterpret_cast<bf16_t*>(setp(cn, L::Q));
            bf16_t* Vb = reinterpret_cast<bf16_t*>(setp(cn, L::V));
            bf16_t* Ph = reinterpret_cast<bf16_t*>(setp(cn, L::PH));
            bf16_t* Pl = reinterpret_cast<bf16_t*>(setp(cn, L::PL));
            const bf16_t* Kb = kring(cn);
            if constexpr (!NOO) stage_kq(Qb, f.q);
#pragma unroll
            for (int u = 0; u < VL; ++u) {
                const int pc = lane + 64 * u;
                *reinterpret_cast<u32x4*>(Vb + (pc / VC) * L::PV + 8 * (pc % VC)) = f.v[u];
            }
            if constexpr (NOO) return;   // no P without o
            wave_lds_sync();   // this wave's Q tile, read back in operand order
            // C[4 g + r][m] = k_{16 st + 4 g + r} . q_{16 rt + m}
            bf16x8 kf[2][KJ], qf[2][KJ];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int j = 0; j < KJ; ++j) {
                    const int row = 16 * tt + m;
                    kf[tt][j] = *reinterpret_cast<const bf16x8*>(Kb + kq_at<DK>(row, 32 * j + 8 * g));
                    qf[tt][j] = *reinterpret_cast<const bf16x8*>(Qb + kq_at<DK>(row, 32 * j + 8 * g));
                }
            const float* grc = gring(cn);
            const Gates z = read_gates(grc, std::false_type{});
            f32x4 acc[3] = {}, qq[2] = {};
#pragma unroll
            for (int j = 0; j < KJ; ++j) {
                acc[0] = mfma16(kf[0][j], qf[0][j], acc[0]);
                acc[1] = mfma16(kf[0][j], qf[1][j], acc[1]);
                acc[2] = mfma16(kf[1][j], qf[1][j], acc[2]);
                if constexpr (NORM) {
                    // diagonal tiles of Q Q^T: |q|^2 of the chunk's rows
                    qq[0] = mfma16(qf[0][j], qf[0][j], qq[0]);
                    qq[1] = mfma16(qf[1][j], qf[1][j], qq[1]);
                }
            }
            // pi of rows 16 rt + m: |q_{16 rt + m}|^2 sits in register
            // m - 4 g of the diagonal tile on the lane with g = m / 4; one
            // bpermute hands it to the row's other lane groups
            float pq[2] = {1.f, 1.f};
            if constexpr (NORM) {
                const int dr = m & 3;
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    float d = qq[tt][0];
#pragma unroll
                    for (int r = 1; r < 4; ++r) d = dr == r ? qq[tt][r] : d;
                    pq[tt] = l2_inv(__shfl(d, 16 * (m >> 2) + m, 64));
                }
                if (g == 0) {
                    float* G = reinterpret_cast<float*>(setp(cn, L::G));
                    G[FPI + m] = pq[0];
                    G[FPI + 16 + m] = pq[1];
                }
            }
#pragma unroll
            for (int u = 0; u < 3; ++u) {
                const int st = u == 2 ? 1 : 0, rt = u == 0 ? 0 : 1;
                const int rp = 16 * rt + m;
                float pv[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int s = 16 * st + 4 * g + r;
                    pv[r] = s <= rp ? __expf(fminf(z.gq[rt] - z.gk[st][r], 0.f)) * acc[u][r] : 0.f;
                    if constexpr (NORM) pv[r] *= pq[rt] * grc[2 * CH + s];
                }
                uint2 vh, vl;
                split2(pv[0], pv[1], vh.x, vl.x);
                split2(pv[2], pv[3], vh.y, vl.y);
                st8(Ph + rp * P48 + kperm(16 * st + 4 * g), vh);
                st8(Pl + rp * P48 + kperm(16 * st + 4 * g), vl);
            }
        };
        Buf fa, fb, fc;
        run(1, load, prepare, fa, fb, fc);
    } else {
        // --------------------- B3: K staging, gate scan, A -------------------
        struct Buf {
            u32x4 k[2][KJ];
            float al, be;   // alpha, beta of token `lane` (lanes < 32)
        };
        auto load = [&](int64_t cn, Buf& f) {
            load_k(cn, f.k, kbase);
            const uint32_t off = (uint32_t)(min(lane & 31, last_row(cn)) * (int)H);
            f.al = (abase + cn * CH * H)[off];
            f.be = (bbase + cn * CH * H)[off];
        };
        auto prepare = [&](int64_t cn, const Buf& f) {
            float* Af = afp(cn);
            float* gr = gring(cn);
            bf16_t* Kr = kring(cn);
            stage_kq(Kr, f.k);
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int j = 0; j < KJ; ++j)
                    *reinterpret_cast<u32x4*>(Kr + CH * DK + (16 * tt + m) * L::PKN + 32 * j + 8 * g) =
                        f.k[tt][j];
            // Gram tiles (s-tile, r-tile) = (0,0), (0,1), (1,1):
            // C[4 g + r][m] = k_{16 st + 4 g + r} . k_{16 rt + m}
            f32x4 acc[3] = {};
#pragma unroll
            for (int j = 0; j < KJ; ++j) {
                const bf16x8 k0 = __builtin_bit_cast(bf16x8, f.k[0][j]);
                const bf16x8 k1 = __builtin_bit_cast(bf16x8, f.k[1][j]);
                acc[0] = mfma16(k0, k0, acc[0]);
                acc[1] = mfma16(k0, k1, acc[1]);
                acc[2] = mfma16(k1, k1, acc[2]);
            }
            // alpha = 1, beta = 0 past the end of the sequence (and on lanes
            // 32..63); g = within-chunk cumulative log decay
            const bool live = lane < CH && cn * CH + lane < T;
            const float gx = wave_scan(live ? safe_log(f.al) : 0.f);
            if (lane < CH) {
                gr[lane] = gx;
                gr[CH + lane] = live ? f.be : 0.f;
            }
            if constexpr (NORM) {
                // |k_m|^2 and |k_{16 + m}|^2 sit in register m - 4 g of the
                // diagonal tiles on the lanes with g = m / 4
                const int dr = m & 3;
                float d0 = acc[0][0], d1 = acc[2][0];
#pragma unroll
                for (int r = 1; r < 4; ++r) {
                    d0 = dr == r ? acc[0][r] : d0;
                    d1 = dr == r ? acc[2][r] : d1;
                }
                if ((m >> 2) == g) {
                    gr[2 * CH + m] = l2_inv(d0);
                    gr[2 * CH + 16 + m] = l2_inv(d1);
                }
            }
            wave_lds_sync();
            const Gates z = read_gates(gr, std::bool_constant<NORM>{});
#pragma unroll
            for (int u = 0; u < 3; ++u) {
                const int st = u == 2 ? 1 : 0, rt = u == 0 ? 0 : 1;
                const int rp = 16 * rt + m;
                f32x4 av;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int s = 16 * st + 4 * g + r;
                    av[r] = s < rp ? z.bq[rt] * __expf(fminf(z.gq[rt] - z.gk[st][r], 0.f)) * acc[u][r]
                                   : 0.f;
                    if constexpr (NORM) av[r] *= z.rq[rt] * z.rk[st][r];
                }
                *reinterpret_cast<f32x4*>(Af + rp * P36 + 16 * st + 4 * g) = av;
            }
        };
        Buf fa, fb, fc;
        run(2, load, prepare, fa, fb, fc);
    }
}

// Few heads (long single sequences): narrower row blocks (16 state rows per
// workgroup instead of 64) so that more workgroups run side by side.
inline bool narrow_row_blocks(int64_t BH, int64_t Dv) { return BH * (Dv / 64) < 128; }

}  // namespace

}  // namespace gdr
