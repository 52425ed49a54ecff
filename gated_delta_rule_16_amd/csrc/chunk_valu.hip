// fp32-input path of gdr_chunk_fwd and gdr2_chunk_fwd: the chunkwise UT/WY
// form evaluated with fp32 vector ALU arithmetic throughout.
//
// Chunk algebra (derived from the recurrence; the chunkwise equations of
// section 3.7 of the GDN review on meaningful96.github.io, with Gamma read as
// exp of differences of the within-chunk cumulative log decay).  For a chunk
// of n tokens starting from state S (rows = value channels):
//
//   scalar gates (GDN):  g_r = sum_{i<=r} log alpha_i
//     A_rs = beta_r e^{g_r - g_s} k_r.k_s      (s < r)     strict lower
//     P_rs = e^{g_r - g_s} q_r.k_s             (s <= r)    diagonal included
//     R_r  = beta_r (v_r - e^{g_r} S k_r)
//     (I + A) V_new = R                        forward substitution
//     o_r  = e^{g_r} S q_r + sum_{s<=r} P_rs V_new_s
//     S   <- e^{g_n} S + sum_s V_new_s (e^{g_n - g_s} k_s)^T
//
//   channel gates (Gated Delta Rule-2): G_rc = sum_{i<=r} log alpha_ic,
//   e_r = b_r (.) k_r, and every exp(g_r - g_s) above becomes a per-channel
//   factor inside the dot product:
//     A_rs = sum_c e_rc k_sc e^{G_rc - G_sc},  P_rs = sum_c q_rc k_sc e^{G_rc - G_sc}
//     R_r  = w_r (.) v_r - S (e_r (.) e^{G_r}),  o_r = S (q_r (.) e^{G_r}) + ...
//     S   <- S diag(e^{G_n}) + sum_s V_new_s (k_s (.) e^{G_n - G_s})^T
//
// Every exponent is <= 0, so nothing overflows; underflow only drops terms
// that are negligible against the others.
//
// Work split: one 256-thread workgroup per (b, h, block of 32 state rows).
// Rows of S evolve independently given the key-side quantities, so the key
// side (A, P, decays) is recomputed by each row block.  Chunk length 32.
#include "gdr_device.h"
#include "launch.h"

namespace gdr {

namespace {

constexpr int C = 32;    // tokens per chunk
constexpr int RB = 32;   // state rows per workgroup
constexpr int NT = 256;  // threads per workgroup

// q, k, v, and for rule 2 alpha, erase and write, are in the input type
// (fp32 or bf16); the scalar gates of rule 1 are fp32.
struct F32Params {
    int64_t T, H;
    const void *q, *k, *v;
    const void *alpha, *erase, *write;
    const float* beta;
    const float* s0;
    void* o;
    float* s_final;
    bool l2norm;
};

template <int DK>
struct Lds {
    static constexpr int PK = DK + 1;   // padded row pitch, key-side tiles
    static constexpr int PC = C + 1;
    static constexpr int PR = RB + 1;
    static constexpr int S = 0;                    // [RB][PK] state rows
    static constexpr int K = S + RB * PK;          // [C][PK] keys, then decayed keys
    static constexpr int Q = K + C * PK;           // [C][PK] queries
    static constexpr int E = Q + C * PK;           // [C][PK] b.k (rule 2)
    static constexpr int G = E + C * PK;           // [C][PK] cumulative log decay (rule 2)
    static constexpr int A = G + C * PK;           // [C][PC]
    static constexpr int P = A + C * PC;           // [C][PC]
    static constexpr int R = P + C * PC;           // [C][PR] rhs, then V_new
    static constexpr int QS = R + C * PR;          // [C][PR] decayed S q
    static constexpr int V = QS + C * PR;          // [C][PR] values (w.v for rule 2)
    static constexpr int LG = V + C * PR;          // [C] log alpha -> g (scalar rule)
    static constexpr int BE = LG + C;              // [C] beta
    static constexpr int TOTAL = BE + C;
};

template <int DK, int DV, bool G2, typename TIn, typename TOut>
__global__ __launch_bounds__(NT) void chunk_f32_kernel(F32Params p) {
    using L = Lds<DK>;
    auto in = [](const void* x, int64_t off) { return io<TIn>::ld(static_cast<const TIn*>(x) + off); };
    constexpr int NRB = DV / RB;
    extern __shared__ float sm[];
    float* Ss = sm + L::S;
    float* Ks = sm + L::K;
    float* Qs = sm + L::Q;
    float* Es = sm + L::E;
    float* Gs = sm + L::G;
    float* As = sm + L::A;
    float* Ps = sm + L::P;
    float* Rs = sm + L::R;
    float* QSs = sm + L::QS;
    float* Vs = sm + L::V;
    float* lg = sm + L::LG;
    float* be = sm + L::BE;

    const int tid = threadIdx.x;
    const int rb = blockIdx.x % NRB;
    const int64_t bh = blockIdx.x / NRB;
    const int64_t h = bh % p.H;
    const int64_t b = bh / p.H;
    const int64_t T = p.T, H = p.H;
    const int row0 = rb * RB;

    // state rows [row0, row0 + RB) of this (b, h)
    const int64_t sbase = (bh * DV + row0) * DK;
    for (int e = tid; e < RB * DK; e += NT) {
        const int i = e / DK, j = e % DK;
        Ss[i * L::PK + j] = p.s0 ? p.s0[sbase + e] : 0.f;
    }

    for (int64_t t0 = 0; t0 < T; t0 += C) {
        const int n = (int)((T - t0) < C ? (T - t0) : C);
        __syncthreads();  // previous chunk done with every buffer
        // ---- load the chunk (rows >= n are zero / neutral) --------------
        for (int e = tid; e < C * DK; e += NT) {
            const int r = e / DK, j = e % DK;
            float kv = 0.f, qv = 0.f, ev = 0.f, gv = 0.f;
            if (r < n) {
                const int64_t off = ((b * T + t0 + r) * H + h) * DK + j;
                kv = in(p.k, off);
                qv = in(p.q, off);
                if (G2) {
                    ev = in(p.erase, off) * kv;
                    gv = safe_log(in(p.alpha, off));
                }
            }
            Ks[r * L::PK + j] = kv;
            Qs[r * L::PK + j] = qv;
            if (G2) {
                Es[r * L::PK + j] = ev;
                Gs[r * L::PK + j] = gv;
            }
        }
        for (int e = tid; e < C * RB; e += NT) {
            const int r = e / RB, i = e % RB;
            float vv = 0.f;
            if (r < n) {
                const int64_t off = ((b * T + t0 + r) * H + h) * DV + row0 + i;
                vv = in(p.v, off);
                if (G2) vv *= in(p.write, off);
            }
            Vs[r * L::PR + i] = vv;
        }
        if (!G2 && tid < C) {
            const int r = tid;
            const int64_t off = (b * T + t0 + r) * H + h;
            lg[r] = r < n ? safe_log(static_cast<const float*>(p.alpha)[off]) : 0.f;
            be[r] = r < n ? p.beta[off] : 0.f;
        }
        __syncthreads();
        // ---- GDR_L2NORM_QK: unit-norm q and k rows (and e = b k with k) --
        //      eight lanes per row; rows past n stay zero.  Only the rows'
        //      own lanes touch them, and the next reads follow the barrier
        //      after the decay scan.
        if (p.l2norm) {
            static_assert(NT == 8 * C, "eight lanes per row");
            const int r = tid >> 3, part = tid & 7;
            float sk = 0.f, sq = 0.f;
            for (int j = part; j < DK; j += 8) {
                sk += Ks[r * L::PK + j] * Ks[r * L::PK + j];
                sq += Qs[r * L::PK + j] * Qs[r * L::PK + j];
            }
#pragma unroll
            for (int msk = 1; msk < 8; msk <<= 1) {
                sk += __shfl_xor(sk, msk, 64);
                sq += __shfl_xor(sq, msk, 64);
            }
            const float rk = l2_inv(sk), rq = l2_inv(sq);
            for (int j = part; j < DK; j += 8) {
                Ks[r * L::PK + j] *= rk;
                Qs[r * L::PK + j] *= rq;
                if (G2) Es[r * L::PK + j] *= rk;
            }
        }
        // ---- cumulative log decay ----------------------------------------
        if (G2) {
            if (tid < DK) {
                float acc = 0.f;
                for (int r = 0; r < C; ++r) {
                    acc += Gs[r * L::PK + tid];
                    Gs[r * L::PK + tid] = acc;
                }
            }
        } else if (tid == 0) {
            float acc = 0.f;
            for (int r = 0; r < C; ++r) {
                acc += lg[r];
                lg[r] = acc;
            }
        }
        __syncthreads();
        // ---- A (strictly lower) and P (lower incl. diagonal) ------------
        for (int e = tid; e < C * C; e += NT) {
            const int r = e / C, s = e % C;
            float av = 0.f, pv = 0.f;
            if (s <= r) {
                float kk = 0.f, qk = 0.f;
                if (G2) {
                    for (int j = 0; j < DK; ++j) {
                        const float d = __expf(Gs[r * L::PK + j] - Gs[s * L::PK + j]);
                        const float ks = Ks[s * L::PK + j] * d;
                        kk += Es[r * L::PK + j] * ks;
                        qk += Qs[r * L::PK + j] * ks;
                    }
                    av = kk;
                    pv = qk;
                } else {
                    for (int j = 0; j < DK; ++j) {
                        const float ks = Ks[s * L::PK + j];
                        kk += Ks[r * L::PK + j] * ks;
                        qk += Qs[r * L::PK + j] * ks;
                    }
                    const float d = __expf(lg[r] - lg[s]);
                    av = be[r] * d * kk;
                    pv = d * qk;
                }
                if (s == r) av = 0.f;
            }
            As[r * L::PC + s] = av;
            Ps[r * L::PC + s] = pv;
        }
        __syncthreads();
        // ---- decayed queries / erase keys (rule 2: in place) -------------
        if (G2) {
            for (int e = tid; e < C * DK; e += NT) {
                const int r = e / DK, j = e % DK;
                const float d = __expf(Gs[r * L::PK + j]);
                Qs[r * L::PK + j] *= d;
                Es[r * L::PK + j] *= d;
            }
            __syncthreads();
        }
        // ---- R = rhs of the solve, QS = decayed S q ----------------------
        for (int e = tid; e < C * RB; e += NT) {
            const int r = e / RB, i = e % RB;
            float sk = 0.f, sq = 0.f;
            const float* srow = Ss + i * L::PK;
            if (G2) {
                for (int j = 0; j < DK; ++j) {
                    sk += Es[r * L::PK + j] * srow[j];
                    sq += Qs[r * L::PK + j] * srow[j];
                }
                Rs[r * L::PR + i] = Vs[r * L::PR + i] - sk;
                QSs[r * L::PR + i] = sq;
            } else {
                for (int j = 0; j < DK; ++j) {
                    sk += Ks[r * L::PK + j] * srow[j];
                    sq += Qs[r * L::PK + j] * srow[j];
                }
                const float gr = __expf(lg[r]);
                Rs[r * L::PR + i] = be[r] * (Vs[r * L::PR + i] - gr * sk);
                QSs[r * L::PR + i] = gr * sq;
            }
        }
        __syncthreads();
        // ---- (I + A) V_new = R by forward substitution (wave 0) ----------
        //      meanwhile the other waves form the decayed keys for S.
        if (tid < RB) {
            const int i = tid;
            float vn[C];
#pragma unroll
            for (int r = 0; r < C; ++r) {
                float x = Rs[r * L::PR + i];
#pragma unroll
                for (int s = 0; s < r; ++s) x -= As[r * L::PC + s] * vn[s];
                vn[r] = x;
                Rs[r * L::PR + i] = x;
            }
        } else if (tid >= 64) {
            for (int e = tid - 64; e < C * DK; e += NT - 64) {
                const int s = e / DK, j = e % DK;
                float d;
                if (G2)
                    d = __expf(Gs[(C - 1) * L::PK + j] - Gs[s * L::PK + j]);
                else
                    d = __expf(lg[C - 1] - lg[s]);
                Ks[s * L::PK + j] *= d;
            }
        }
        __syncthreads();
        // ---- outputs ----------------------------------------------------
        for (int e = tid; e < C * RB; e += NT) {
            const int r = e / RB, i = e % RB;
            if (r < n) {
                float x = QSs[r * L::PR + i];
                for (int s = 0; s <= r; ++s) x += Ps[r * L::PC + s] * Rs[s * L::PR + i];
                const int64_t off = ((b * T + t0 + r) * H + h) * DV + row0 + i;
                io<TOut>::st(reinterpret_cast<TOut*>(p.o) + off, x);
            }
        }
        // ---- state update ------------------------------------------------
        for (int e = tid; e < RB * DK; e += NT) {
            const int i = e / DK, j = e % DK;
            const float dec = G2 ? __expf(Gs[(C - 1) * L::PK + j]) : __expf(lg[C - 1]);
            float x = dec * Ss[i * L::PK + j];
            for (int s = 0; s < C; ++s) x += Rs[s * L::PR + i] * Ks[s * L::PK + j];
            Ss[i * L::PK + j] = x;
        }
    }
    __syncthreads();
    if (p.s_final) {
        for (int e = tid; e < RB * DK; e += NT) {
            const int i = e / DK, j = e % DK;
            p.s_final[sbase + e] = Ss[i * L::PK + j];
        }
    }
}

template <int DK, int DV, bool G2, typename TIn, typename TOut>
hipError_t launch_f32_t(const ChunkArgs& a) {
    F32Params p;
    p.T = a.T;
    p.H = a.H;
    p.q = a.q;
    p.k = a.k;
    p.v = a.v;
    p.alpha = a.alpha;
    p.beta = (const float*)a.beta;
    p.erase = a.erase;
    p.write = a.write;
    p.s0 = a.s0;
    p.o = a.o;
    p.s_final = a.s_final;
    p.l2norm = a.l2norm;
    const size_t lds = sizeof(float) * Lds<DK>::TOTAL;
    auto fn = chunk_f32_kernel<DK, DV, G2, TIn, TOut>;
    hipError_t e = hipFuncSetAttribute((const void*)fn,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    const unsigned grid = (unsigned)(a.B * a.H * (DV / RB));
    hipLaunchKernelGGL(fn, dim3(grid), dim3(NT), lds, a.stream, p);
    return hipGetLastError();
}

template <int DK, int DV, typename TIn>
hipError_t launch_f32_i(const ChunkArgs& a) {
    if (a.gated2)
        return a.out_bf16 ? launch_f32_t<DK, DV, true, TIn, bf16_t>(a)
                          : launch_f32_t<DK, DV, true, TIn, float>(a);
    return a.out_bf16 ? launch_f32_t<DK, DV, false, TIn, bf16_t>(a)
                      : launch_f32_t<DK, DV, false, TIn, float>(a);
}

// bf16 inputs come here only for rule 2 when full fp32 arithmetic is asked
// for (the sequence-split backward's start states)
template <int DK, int DV>
hipError_t launch_f32_d(const ChunkArgs& a) {
    if (a.in_bf16) {
        if (!a.gated2) return hipErrorNotSupported;
        return launch_f32_i<DK, DV, bf16_t>(a);
    }
    return launch_f32_i<DK, DV, float>(a);
}

}  // namespace

hipError_t launch_chunk_f32(const ChunkArgs& a) {
    if (a.Dk == 128 && a.Dv == 128) return launch_f32_d<128, 128>(a);
    if (a.Dk == 128 && a.Dv == 64) return launch_f32_d<128, 64>(a);
    if (a.Dk == 64 && a.Dv == 128) return launch_f32_d<64, 128>(a);
    return launch_f32_d<64, 64>(a);
}

}  // namespace gdr
