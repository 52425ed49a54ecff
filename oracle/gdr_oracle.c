/*
 * fp64 CPU oracle for the gated delta rule family.  TEST INFRASTRUCTURE ONLY:
 * only the tests, the smoke check and the benchmark's CPU-baseline leg load
 * this library.  It shares no code, header or constant with the HIP kernels.
 *
 * Plain, sequential-in-time recurrences, evaluated token by token in double
 * precision.  Every array is row-major and contiguous:
 *   q, k            [B, T, H, Dk]
 *   v               [B, T, H, Dv]
 *   alpha, beta     [B, T, H]          (GDN, scalar gates)
 *   alpha, erase    [B, T, H, Dk]      (GDN-2, key-axis gates)
 *   write           [B, T, H, Dv]      (GDN-2, value-axis gate)
 *   s0, s_final     [B, H, Dv, Dk]     (state S is Dv x Dk, o = S q)
 *   o               [B, T, H, Dv]
 * s0 == NULL means a zero initial state; s_final == NULL means "not wanted".
 *
 * The state is a Dv x Dk matrix: the review of Gated DeltaNet on
 * meaningful96.github.io ("1. Problem Formulation" and "3.1 Linear Attention
 * as Associative Memory") writes o_t = S_t q_t and the write v_t k_t^T.
 *
 * Row form.  Every rule here right-multiplies S by a Dk x Dk transition and
 * adds an outer product v k^T, so row i of S (the i-th value channel) is
 * updated from its own old value, the scalar v_i, and the shared key-side
 * vectors.  The loops below therefore run row by row inside each token;
 * that is the matrix product written out entry by entry, not a reordering.
 */
#include <stddef.h>
#include <stdlib.h>
#include <math.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_OK 0
#define ORACLE_ERR_ARGS 1
#define ORACLE_ERR_NOMEM 2

static void state_init(double *S, const double *s0, long Dv, long Dk) {
    if (s0)
        memcpy(S, s0, sizeof(double) * (size_t)(Dv * Dk));
    else
        memset(S, 0, sizeof(double) * (size_t)(Dv * Dk));
}

/*
 * One token of the gated delta rule on one (sequence, head) state:
 *
 *   S_t = S_{t-1} . alpha_t (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *   o_t = S_t q_t.
 *
 * This is the update of "Gated Delta Networks" (agihunt.info, both the
 * Chinese summary and the English "Method" section) and equation of section
 * 3.4 of the meaningful96 review; o_t = S_t q_t is from its section 1.
 * Multiplying row s of S_{t-1} into alpha (I - beta k k^T) gives
 * alpha s - alpha beta (s . k) k^T, to which beta v_i k^T is added.
 */
static void gdn_token(double *S, long Dk, long Dv, const double *q,
                      const double *k, const double *v, double alpha,
                      double beta, double *o) {
    for (long i = 0; i < Dv; ++i) {
        double *s = S + i * Dk;
        double sk = 0.0;                     /* (S_{t-1} k_t)_i */
        for (long j = 0; j < Dk; ++j) sk += s[j] * k[j];
        const double c = beta * v[i] - alpha * beta * sk;
        for (long j = 0; j < Dk; ++j) s[j] = alpha * s[j] + c * k[j];
        double oi = 0.0;                     /* (S_t q_t)_i */
        for (long j = 0; j < Dk; ++j) oi += s[j] * q[j];
        o[i] = oi;
    }
}

/* Gated delta rule forward over a whole sequence, for every (b, h). */
int oracle_gdn_fwd(long B, long T, long H, long Dk, long Dv, const double *q,
                   const double *k, const double *v, const double *alpha,
                   const double *beta, const double *s0, double *o,
                   double *s_final) {
    if (B < 0 || T < 0 || H < 0 || Dk <= 0 || Dv <= 0) return ORACLE_ERR_ARGS;
    if (!q || !k || !v || !alpha || !beta || !o) return ORACLE_ERR_ARGS;
    int err = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (long b = 0; b < B; ++b) {
        for (long h = 0; h < H; ++h) {
            double *S = (double *)malloc(sizeof(double) * (size_t)(Dv * Dk));
            if (!S) {
#pragma omp atomic write
                err = 1;
                continue;
            }
            state_init(S, s0 ? s0 + (b * H + h) * Dv * Dk : NULL, Dv, Dk);
            for (long t = 0; t < T; ++t) {
                const long bth = (b * T + t) * H + h;
                gdn_token(S, Dk, Dv, q + bth * Dk, k + bth * Dk, v + bth * Dv,
                          alpha[bth], beta[bth], o + bth * Dv);
            }
            if (s_final)
                memcpy(s_final + (b * H + h) * Dv * Dk, S,
                       sizeof(double) * (size_t)(Dv * Dk));
            free(S);
        }
    }
    return err ? ORACLE_ERR_NOMEM : ORACLE_OK;
}

/*
 * Reverse mode of the gated delta rule (the derivative of oracle_gdn_fwd,
 * written out token by token by the chain rule).  The pages describe the
 * method's throughput as a training workload, and the GDN-2 summary notes
 * that a chunked backward must carry the gates inside its dot products;
 * this is the plain definition such a backward must reproduce.
 *
 * Per token, with u = S_{t-1} k, c = beta v - alpha beta u, the forward is
 * S_t = alpha S_{t-1} + c k^T and o_t = S_t q.  Given G = dL/dS_t (the
 * gradient carried back from later tokens, dL/dS_T at the end) and do_t:
 *
 *   G    += do_t q^T            dq_t  = S_t^T do_t
 *   dc    = G k                 dk_t  = G^T c + S_{t-1}^T du,  du = -alpha beta dc
 *   dv_t  = beta dc             dbeta = dc . (v - alpha u)
 *   dalpha = <G, S_{t-1}>_F - beta (dc . u)
 *   G    <- alpha G + du k^T    (dL/dS_{t-1});  dS_0 = G at the start.
 *
 * dout [B,T,H,Dv]; ds_final [B,H,Dv,Dk] or NULL (zero); outputs dq, dk
 * [B,T,H,Dk], dv [B,T,H,Dv], dalpha, dbeta [B,T,H], ds0 [B,H,Dv,Dk] or NULL.
 * States are kept every SEG tokens and recomputed inside each segment.
 */
#define ORACLE_BWD_SEG 64
static void gdn_step_state(double *S, const double *Sprev, long Dk, long Dv,
                           const double *k, const double *v, double alpha,
                           double beta) {
    for (long i = 0; i < Dv; ++i) {
        const double *sp = Sprev + i * Dk;
        double *s = S + i * Dk;
        double u = 0.0;
        for (long j = 0; j < Dk; ++j) u += sp[j] * k[j];
        const double c = beta * v[i] - alpha * beta * u;
        for (long j = 0; j < Dk; ++j) s[j] = alpha * sp[j] + c * k[j];
    }
}

int oracle_gdn_bwd(long B, long T, long H, long Dk, long Dv, const double *q,
                   const double *k, const double *v, const double *alpha,
                   const double *beta, const double *s0, const double *dout,
                   const double *ds_final, double *dq, double *dk, double *dv,
                   double *dalpha, double *dbeta, double *ds0) {
    if (B < 0 || T < 0 || H < 0 || Dk <= 0 || Dv <= 0) return ORACLE_ERR_ARGS;
    if (!q || !k || !v || !alpha || !beta || !dout || !dq || !dk || !dv || !dalpha || !dbeta)
        return ORACLE_ERR_ARGS;
    const long SEG = ORACLE_BWD_SEG;
    const long nseg = (T + SEG - 1) / SEG;
    int err = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (long b = 0; b < B; ++b) {
        for (long h = 0; h < H; ++h) {
            const size_t SS = (size_t)(Dv * Dk);
            /* segment-start states, the states inside one segment, G, work */
            double *ck = (double *)malloc(sizeof(double) * SS * (size_t)(nseg + 1));
            double *st = (double *)malloc(sizeof(double) * SS * (size_t)(SEG + 1));
            double *G = (double *)malloc(sizeof(double) * SS);
            double *cv = (double *)malloc(sizeof(double) * (size_t)Dv);
            double *uv = (double *)malloc(sizeof(double) * (size_t)Dv);
            double *dcv = (double *)malloc(sizeof(double) * (size_t)Dv);
            if (!ck || !st || !G || !cv || !uv || !dcv) {
#pragma omp atomic write
                err = 1;
                free(ck); free(st); free(G); free(cv); free(uv); free(dcv);
                continue;
            }
            state_init(ck, s0 ? s0 + (b * H + h) * SS : NULL, Dv, Dk);
            for (long sg = 0; sg < nseg; ++sg) {
                memcpy(st, ck + sg * SS, sizeof(double) * SS);
                const long t1 = (sg + 1) * SEG < T ? (sg + 1) * SEG : T;
                for (long t = sg * SEG; t < t1; ++t) {
                    const long bth = (b * T + t) * H + h;
                    gdn_step_state(st, st, Dk, Dv, k + bth * Dk, v + bth * Dv, alpha[bth], beta[bth]);
                }
                memcpy(ck + (sg + 1) * SS, st, sizeof(double) * SS);
            }
            if (ds_final)
                memcpy(G, ds_final + (b * H + h) * SS, sizeof(double) * SS);
            else
                memset(G, 0, sizeof(double) * SS);
            for (long sg = nseg - 1; sg >= 0; --sg) {
                const long t0 = sg * SEG;
                const long t1 = t0 + SEG < T ? t0 + SEG : T;
                /* st[j] = S_{t0 + j}, j = 0 .. t1 - t0 */
                memcpy(st, ck + sg * SS, sizeof(double) * SS);
                for (long t = t0; t < t1; ++t) {
                    const long bth = (b * T + t) * H + h;
                    gdn_step_state(st + (t - t0 + 1) * SS, st + (t - t0) * SS, Dk, Dv,
                                   k + bth * Dk, v + bth * Dv, alpha[bth], beta[bth]);
                }
                for (long t = t1 - 1; t >= t0; --t) {
                    const long bth = (b * T + t) * H + h;
                    const double *Sp = st + (t - t0) * SS;       /* S_{t-1} */
                    const double *Sn = st + (t - t0 + 1) * SS;   /* S_t */
                    const double *qt = q + bth * Dk, *kt = k + bth * Dk, *vt = v + bth * Dv;
                    const double *dot = dout + bth * Dv;
                    const double a = alpha[bth], be = beta[bth];
                    double *dqt = dq + bth * Dk, *dkt = dk + bth * Dk, *dvt = dv + bth * Dv;
                    for (long i = 0; i < Dv; ++i)
                        for (long j = 0; j < Dk; ++j) G[i * Dk + j] += dot[i] * qt[j];
                    for (long j = 0; j < Dk; ++j) {
                        double x = 0.0;
                        for (long i = 0; i < Dv; ++i) x += Sn[i * Dk + j] * dot[i];
                        dqt[j] = x;
                    }
                    double dbt = 0.0, dat = 0.0;
                    for (long i = 0; i < Dv; ++i) {
                        double u = 0.0, dc = 0.0, gs = 0.0;
                        for (long j = 0; j < Dk; ++j) {
                            u += Sp[i * Dk + j] * kt[j];
                            dc += G[i * Dk + j] * kt[j];
                            gs += G[i * Dk + j] * Sp[i * Dk + j];
                        }
                        uv[i] = u;
                        cv[i] = be * vt[i] - a * be * u;
                        dcv[i] = dc;
                        dvt[i] = be * dc;
                        dbt += dc * (vt[i] - a * u);
                        dat += gs - be * dc * u;
                    }
                    dbeta[bth] = dbt;
                    dalpha[bth] = dat;
                    for (long j = 0; j < Dk; ++j) {
                        double x = 0.0;
                        for (long i = 0; i < Dv; ++i)
                            x += G[i * Dk + j] * cv[i] - a * be * dcv[i] * Sp[i * Dk + j];
                        dkt[j] = x;
                    }
                    for (long i = 0; i < Dv; ++i)
                        for (long j = 0; j < Dk; ++j)
                            G[i * Dk + j] = a * G[i * Dk + j] - a * be * dcv[i] * kt[j];
                }
            }
            if (ds0) memcpy(ds0 + (b * H + h) * SS, G, sizeof(double) * SS);
            free(ck); free(st); free(G); free(cv); free(uv); free(dcv);
        }
    }
    return err ? ORACLE_ERR_NOMEM : ORACLE_OK;
}

/*
 * One decode step for N independent sequences: the same single-token update
 * applied in place to state [N, H, Dv, Dk], with q, k [N, H, Dk],
 * v [N, H, Dv], alpha, beta [N, H] and o [N, H, Dv].  A fixed-size state
 * and constant memory per token is how both summaries describe decoding.
 */
int oracle_gdn_step(long N, long H, long Dk, long Dv, const double *q,
                    const double *k, const double *v, const double *alpha,
                    const double *beta, double *state, double *o) {
    if (N < 0 || H < 0 || Dk <= 0 || Dv <= 0) return ORACLE_ERR_ARGS;
    if (!q || !k || !v || !alpha || !beta || !state || !o)
        return ORACLE_ERR_ARGS;
#pragma omp parallel for schedule(static)
    for (long nh = 0; nh < N * H; ++nh)
        gdn_token(state + nh * Dv * Dk, Dk, Dv, q + nh * Dk, k + nh * Dk,
                  v + nh * Dv, alpha[nh], beta[nh], o + nh * Dv);
    return ORACLE_OK;
}

/*
 * One token of Gated Delta Rule-2 ("Gated DeltaNet-2", agihunt.info,
 * paragraph on the update order): decay the old state with the per-channel
 * alpha_t on the key axis, read the old value along b_t (.) k_t, then write
 * the residual between w_t (.) v_t and that read along k_t:
 *
 *   S' = S_{t-1} diag(alpha_t)
 *   S_t = S' + (w_t (.) v_t - S' (b_t (.) k_t)) k_t^T,   o_t = S_t q_t.
 *
 * The equation itself is missing from the page; this is the reading its
 * wording gives, and collapsing the gates (alpha = a 1, b = w = beta 1)
 * returns the scalar rule above, as the page states.
 */
static void gdn2_token(double *S, long Dk, long Dv, const double *q,
                       const double *k, const double *v, const double *alpha,
                       const double *erase, const double *write, double *o) {
    for (long i = 0; i < Dv; ++i) {
        double *s = S + i * Dk;
        for (long j = 0; j < Dk; ++j) s[j] *= alpha[j];      /* S' */
        double rd = 0.0;                                     /* S'(b.k) */
        for (long j = 0; j < Dk; ++j) rd += s[j] * (erase[j] * k[j]);
        const double c = write[i] * v[i] - rd;
        for (long j = 0; j < Dk; ++j) s[j] += c * k[j];
        double oi = 0.0;
        for (long j = 0; j < Dk; ++j) oi += s[j] * q[j];
        o[i] = oi;
    }
}

int oracle_gdn2_fwd(long B, long T, long H, long Dk, long Dv, const double *q,
                    const double *k, const double *v, const double *alpha,
                    const double *erase, const double *write,
                    const double *s0, double *o, double *s_final) {
    if (B < 0 || T < 0 || H < 0 || Dk <= 0 || Dv <= 0) return ORACLE_ERR_ARGS;
    if (!q || !k || !v || !alpha || !erase || !write || !o)
        return ORACLE_ERR_ARGS;
    int err = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (long b = 0; b < B; ++b) {
        for (long h = 0; h < H; ++h) {
            double *S = (double *)malloc(sizeof(double) * (size_t)(Dv * Dk));
            if (!S) {
#pragma omp atomic write
                err = 1;
                continue;
            }
            state_init(S, s0 ? s0 + (b * H + h) * Dv * Dk : NULL, Dv, Dk);
            for (long t = 0; t < T; ++t) {
                const long bth = (b * T + t) * H + h;
                gdn2_token(S, Dk, Dv, q + bth * Dk, k + bth * Dk,
                           v + bth * Dv, alpha + bth * Dk, erase + bth * Dk,
                           write + bth * Dv, o + bth * Dv);
            }
            if (s_final)
                memcpy(s_final + (b * H + h) * Dv * Dk, S,
                       sizeof(double) * (size_t)(Dv * Dk));
            free(S);
        }
    }
    return err ? ORACLE_ERR_NOMEM : ORACLE_OK;
}

/*
 * L2 normalisation of the rows of x [n, d] into out [n, d]:
 *
 *   out_r = x_r / sqrt(sum_c x_rc^2 + eps).
 *
 * The Gated DeltaNet block ends the q and k paths with an L2 normalisation
 * before the rule (review on meaningful96.github.io, section 3.8, the block
 * diagram of q and k; the Gated DeltaNet-2 page keeps that block design).
 * The pages give no guard for a zero row: eps inside the square root is the
 * reading taken here (the library fixes eps = 1e-6).
 */
int oracle_l2norm_rows(long n, long d, const double *x, double eps, double *out) {
    if (n < 0 || d < 0 || !(eps >= 0.0)) return 1;
    for (long r = 0; r < n; ++r) {
        const double *xr = x + r * d;
        double ss = 0.0;
        for (long c = 0; c < d; ++c) ss += xr[c] * xr[c];
        const double inv = 1.0 / sqrt(ss + eps);
        for (long c = 0; c < d; ++c) out[r * d + c] = xr[c] * inv;
    }
    return 0;
}

/*
 * Reverse mode of oracle_l2norm_rows: given the rows x and the gradient dy
 * with respect to y = x / n, n = sqrt(sum_c x_c^2 + eps), the gradient with
 * respect to x is the transposed Jacobian of the map applied to dy,
 *
 *   dx_j = sum_i dy_i (delta_ij / n - x_i x_j / n^3).
 */
int oracle_l2norm_rows_bwd(long n, long d, const double *x, const double *dy, double eps,
                           double *dx) {
    if (n < 0 || d < 0 || !(eps >= 0.0)) return 1;
    for (long r = 0; r < n; ++r) {
        const double *xr = x + r * d, *gr = dy + r * d;
        double ss = 0.0, xg = 0.0;
        for (long c = 0; c < d; ++c) {
            ss += xr[c] * xr[c];
            xg += xr[c] * gr[c];
        }
        const double nn = sqrt(ss + eps);
        for (long j = 0; j < d; ++j) dx[r * d + j] = gr[j] / nn - xr[j] * xg / (nn * nn * nn);
    }
    return 0;
}

/*
 * Output gate of the block on each row of d values (one token and head):
 *
 *   y_i = o_i / sqrt(mean_j o_j^2 + eps) * w_i * g_i * sigmoid(g_i),
 *
 * an RMS normalisation of the recurrent output followed by a SiLU output
 * gate (the Gated DeltaNet-2 page: the recurrent output passes an RMSNorm
 * and a SiLU output gate; review on meaningful96.github.io, section 3.8:
 * normalisation and gating on the output before the output projection).
 * w (d values, shared by every row) is the norm's per-channel weight, NULL
 * meaning all ones; g is the gate branch's pre-activation.  The mean runs
 * over the d channels of the row.
 */
int oracle_rmsnorm_gate_rows(long n, long d, const double *o, const double *g,
                             const double *w, double eps, double *y) {
    if (n < 0 || d <= 0 || !(eps >= 0.0)) return 1;
    for (long r = 0; r < n; ++r) {
        const double *orow = o + r * d, *grow = g + r * d;
        double ss = 0.0;
        for (long c = 0; c < d; ++c) ss += orow[c] * orow[c];
        const double inv = 1.0 / sqrt(ss / (double)d + eps);
        for (long c = 0; c < d; ++c) {
            const double gate = grow[c] / (1.0 + exp(-grow[c]));
            y[r * d + c] = orow[c] * inv * (w ? w[c] : 1.0) * gate;
        }
    }
    return 0;
}

/*
 * Reverse mode of oracle_rmsnorm_gate_rows by the chain rule, per row with
 * r = 1 / sqrt(mean_j o_j^2 + eps), n = r o, s(g) = g sigmoid(g):
 *
 *   y_i = n_i w_i s(g_i)
 *   dn_i = dy_i w_i s(g_i)
 *   do_j = sum_i dn_i dn_i/do_j = sum_i dn_i (r delta_ij - o_i o_j r^3 / d)
 *   dg_i = dy_i n_i w_i s'(g_i),  s'(g) = sigmoid(g) (1 + g (1 - sigmoid(g)))
 *   dw_i = sum over rows of dy_i n_i s(g_i)   (when w is given; dw may be
 *          NULL; w NULL means ones)
 */
int oracle_rmsnorm_gate_rows_bwd(long n, long d, const double *o, const double *g,
                                 const double *w, double eps, const double *dy, double *dout,
                                 double *dg, double *dw) {
    if (n < 0 || d <= 0 || !(eps >= 0.0)) return 1;
    if (dw)
        for (long c = 0; c < d; ++c) dw[c] = 0.0;
    for (long rr = 0; rr < n; ++rr) {
        const double *orow = o + rr * d, *grow = g + rr * d, *dyr = dy + rr * d;
        double ss = 0.0;
        for (long c = 0; c < d; ++c) ss += orow[c] * orow[c];
        const double r = 1.0 / sqrt(ss / (double)d + eps);
        double on = 0.0;   /* sum_i dn_i o_i */
        for (long i = 0; i < d; ++i) {
            const double sg = 1.0 / (1.0 + exp(-grow[i]));
            const double wi = w ? w[i] : 1.0;
            const double dn = dyr[i] * wi * grow[i] * sg;
            on += dn * orow[i];
            dg[rr * d + i] = dyr[i] * orow[i] * r * wi * sg * (1.0 + grow[i] * (1.0 - sg));
            if (dw) dw[i] += dyr[i] * orow[i] * r * grow[i] * sg;
        }
        for (long j = 0; j < d; ++j) {
            const double sg = 1.0 / (1.0 + exp(-grow[j]));
            const double dn = dyr[j] * (w ? w[j] : 1.0) * grow[j] * sg;
            dout[rr * d + j] = dn * r - orow[j] * on * r * r * r / (double)d;
        }
    }
    return 0;
}

/*
 * Reverse mode of Gated Delta Rule-2 (the derivative of oracle_gdn2_fwd,
 * token by token by the chain rule; the GDN-2 summary notes that its
 * chunked backward must carry the gates inside the dot products).  Per
 * token and value row i, with S' = S_{t-1} diag(alpha), e = b (.) k,
 * u_i = s'_i . e, c_i = w_i v_i - u_i, s_i <- s'_i + c_i k, o_i = s_i . q.
 * Given G = dL/dS_t and do_t:
 *
 *   g_i += do_i q           dq   = sum_i do_i s_i (new state)
 *   dc_i = g_i . k          dk   = sum_i c_i g_i + b (.) de
 *   dw_i = dc_i v_i         dv_i = dc_i w_i
 *   ds'_i = g_i - dc_i e    de   = -sum_i dc_i s'_i,  db = k (.) de
 *   dalpha = sum_i ds'_i (.) s_i (old state)
 *   G <- ds' diag(alpha)    (dL/dS_{t-1})
 *
 * Layouts as oracle_gdn2_fwd; dalpha, derase [B,T,H,Dk], dwrite
 * [B,T,H,Dv].  States are kept every SEG tokens and recomputed.
 */
static void gdn2_step_state(double *S, const double *Sprev, long Dk, long Dv,
                            const double *k, const double *v, const double *alpha,
                            const double *erase, const double *write) {
    for (long i = 0; i < Dv; ++i) {
        const double *sp = Sprev + i * Dk;
        double *s = S + i * Dk;
        double u = 0.0;
        for (long j = 0; j < Dk; ++j) u += sp[j] * alpha[j] * erase[j] * k[j];
        const double c = write[i] * v[i] - u;
        for (long j = 0; j < Dk; ++j) s[j] = sp[j] * alpha[j] + c * k[j];
    }
}

int oracle_gdn2_bwd(long B, long T, long H, long Dk, long Dv, const double *q,
                    const double *k, const double *v, const double *alpha,
                    const double *erase, const double *write, const double *s0,
                    const double *dout, const double *ds_final, double *dq, double *dk,
                    double *dv, double *dalpha, double *derase, double *dwrite,
                    double *ds0) {
    if (B < 0 || T < 0 || H < 0 || Dk <= 0 || Dv <= 0) return ORACLE_ERR_ARGS;
    if (!q || !k || !v || !alpha || !erase || !write || !dout || !dq || !dk || !dv || !dalpha ||
        !derase || !dwrite)
        return ORACLE_ERR_ARGS;
    const long SEG = ORACLE_BWD_SEG;
    const long nseg = (T + SEG - 1) / SEG;
    int err = 0;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (long b = 0; b < B; ++b) {
        for (long h = 0; h < H; ++h) {
            const size_t SS = (size_t)(Dv * Dk);
            double *ck = (double *)malloc(sizeof(double) * SS * (size_t)(nseg + 1));
            double *st = (double *)malloc(sizeof(double) * SS * (size_t)(SEG + 1));
            double *G = (double *)malloc(sizeof(double) * SS);
            double *cv = (double *)malloc(sizeof(double) * (size_t)Dv);
            double *dcv = (double *)malloc(sizeof(double) * (size_t)Dv);
            double *ev = (double *)malloc(sizeof(double) * (size_t)Dk);
            double *dev = (double *)malloc(sizeof(double) * (size_t)Dk);
            if (!ck || !st || !G || !cv || !dcv || !ev || !dev) {
#pragma omp atomic write
                err = 1;
                free(ck); free(st); free(G); free(cv); free(dcv); free(ev); free(dev);
                continue;
            }
            state_init(ck, s0 ? s0 + (b * H + h) * SS : NULL, Dv, Dk);
            for (long sg = 0; sg < nseg; ++sg) {
                memcpy(st, ck + sg * SS, sizeof(double) * SS);
                const long t1 = (sg + 1) * SEG < T ? (sg + 1) * SEG : T;
                for (long t = sg * SEG; t < t1; ++t) {
                    const long bth = (b * T + t) * H + h;
                    gdn2_step_state(st, st, Dk, Dv, k + bth * Dk, v + bth * Dv, alpha + bth * Dk,
                                    erase + bth * Dk, write + bth * Dv);
                }
                memcpy(ck + (sg + 1) * SS, st, sizeof(double) * SS);
            }
            if (ds_final)
                memcpy(G, ds_final + (b * H + h) * SS, sizeof(double) * SS);
            else
                memset(G, 0, sizeof(double) * SS);
            for (long sg = nseg - 1; sg >= 0; --sg) {
                const long t0 = sg * SEG;
                const long t1 = t0 + SEG < T ? t0 + SEG : T;
                memcpy(st, ck + sg * SS, sizeof(double) * SS);
                for (long t = t0; t < t1; ++t) {
                    const long bth = (b * T + t) * H + h;
                    gdn2_step_state(st + (t - t0 + 1) * SS, st + (t - t0) * SS, Dk, Dv,
                                    k + bth * Dk, v + bth * Dv, alpha + bth * Dk,
                                    erase + bth * Dk, write + bth * Dv);
                }
                for (long t = t1 - 1; t >= t0; --t) {
                    const long bth = (b * T + t) * H + h;
                    const double *Sp = st + (t - t0) * SS;       /* S_{t-1} */
                    const double *Sn = st + (t - t0 + 1) * SS;   /* S_t */
                    const double *qt = q + bth * Dk, *kt = k + bth * Dk, *vt = v + bth * Dv;
                    const double *at = alpha + bth * Dk, *bt = erase + bth * Dk, *wt = write + bth * Dv;
                    const double *dot = dout + bth * Dv;
                    double *dqt = dq + bth * Dk, *dkt = dk + bth * Dk, *dvt = dv + bth * Dv;
                    double *dat = dalpha + bth * Dk, *dbt = derase + bth * Dk, *dwt = dwrite + bth * Dv;
                    for (long j = 0; j < Dk; ++j) {
                        ev[j] = bt[j] * kt[j];
                        dev[j] = 0.0;
                        dat[j] = 0.0;
                        dkt[j] = 0.0;
                    }
                    for (long i = 0; i < Dv; ++i)
                        for (long j = 0; j < Dk; ++j) G[i * Dk + j] += dot[i] * qt[j];
                    for (long j = 0; j < Dk; ++j) {
                        double x = 0.0;
                        for (long i = 0; i < Dv; ++i) x += Sn[i * Dk + j] * dot[i];
                        dqt[j] = x;
                    }
                    for (long i = 0; i < Dv; ++i) {
                        double u = 0.0, dc = 0.0;
                        for (long j = 0; j < Dk; ++j) {
                            u += Sp[i * Dk + j] * at[j] * ev[j];
                            dc += G[i * Dk + j] * kt[j];
                        }
                        cv[i] = wt[i] * vt[i] - u;
                        dcv[i] = dc;
                        dwt[i] = dc * vt[i];
                        dvt[i] = dc * wt[i];
                    }
                    for (long i = 0; i < Dv; ++i)
                        for (long j = 0; j < Dk; ++j) {
                            const double sprime = Sp[i * Dk + j] * at[j];
                            const double dsp = G[i * Dk + j] - dcv[i] * ev[j];
                            dkt[j] += cv[i] * G[i * Dk + j];
                            dev[j] -= dcv[i] * sprime;
                            dat[j] += dsp * Sp[i * Dk + j];
                            G[i * Dk + j] = dsp * at[j];
                        }
                    for (long j = 0; j < Dk; ++j) {
                        dbt[j] = dev[j] * kt[j];
                        dkt[j] += dev[j] * bt[j];
                    }
                }
            }
            if (ds0) memcpy(ds0 + (b * H + h) * SS, G, sizeof(double) * SS);
            free(ck); free(st); free(G); free(cv); free(dcv); free(ev); free(dev);
        }
    }
    return err ? ORACLE_ERR_NOMEM : ORACLE_OK;
}

/* Threads the oracle's parallel loops use (reported with CPU timings). */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
