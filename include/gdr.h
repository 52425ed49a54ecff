/*
 * gdr.h — C ABI of the MI355X (gfx950) gated delta rule library, libgdr.so.
 *
 * Three operations, each evaluated by hand-written HIP kernels:
 *
 *   gdr_chunk_fwd       chunkwise-parallel forward of the gated delta rule
 *   gdr_recurrent_step  one decode token of the same rule, state in place
 *   gdr2_chunk_fwd      chunkwise forward of Gated Delta Rule-2 (channel gates)
 *
 * plus their _ex variants (q, k L2-normalised on load), the block's output
 * gate on their result (gdr_output_gate, and fused on the forward's stores:
 * gdr_chunk_fwd_gate), the reverse modes of the two
 * chunkwise forwards and of the gate (gdr_chunk_bwd, gdr2_chunk_bwd,
 * gdr_output_gate_bwd), and sequence-split forms of both chunkwise
 * directions for few long sequences (gdr_chunk_fwd_split,
 * gdr_chunk_bwd_split, gdr2_chunk_fwd_split, gdr2_chunk_bwd_split).
 * gdr_output_gate_bwd_noalloc is the gate's reverse mode without a caller
 * workspace, for callers that cannot allocate.
 *
 * The rule ("Gated Delta Networks", agihunt.info, "Method"; review of GDN on
 * meaningful96.github.io, section 3.4; inputs and outputs from its
 * section 1 "Problem Formulation"):
 *
 *   S_t = S_{t-1} alpha_t (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *   o_t = S_t q_t,
 *
 * with the state S a d_v x d_k fp32 matrix per (sequence, head).  No scale
 * is applied to q (o_t = S_t q_t exactly).  The block L2-normalises q and
 * k before the mixer (review section 3.8): the plain calls take them as
 * given (nothing here depends on the normalisation for correctness), and
 * the _ex variants at the end of this header can apply it on load.
 *
 * Conventions shared by every call
 *   - Every tensor pointer is a DEVICE pointer owned by the caller; tensors
 *     are contiguous and row-major in the layouts given per argument.  The
 *     library calls no allocator and keeps no state between calls, with one
 *     exception: gdr_output_gate_bwd_noalloc writes its partial sums to a
 *     1 MiB array the library holds per GPU (see there).
 *   - Calls are asynchronous on `stream` (0 = the null stream) and return
 *     after the kernels are enqueued.
 *   - Arguments are validated on the host before anything is launched; on
 *     any error nothing is written.  Status codes:
 *       GDR_ERR_INVALID      a required pointer is NULL, a size is negative,
 *                            H exceeds GDR_MAX_HEADS in a chunkwise call
 *                            (forward, split or backward), a launch would
 *                            exceed the 2^32 - 1 work-items of one dispatch
 *                            (more than 2^21 - 8 heads B H -- B nseg H in a
 *                            split call -- in a chunkwise call, 2^24 - 1
 *                            N H in a decode step, or 2^32 - 256 elements
 *                            B T H Dk in a backward), or a pointer is
 *                            misaligned: q, k, v, the
 *                            channel gates, s0, s_final and the decode
 *                            state need 16-byte alignment; the scalar gates
 *                            and o need element alignment;
 *       GDR_ERR_UNSUPPORTED  (Dk, Dv) not in {64, 128} x {64, 128}, an
 *                            unsupported dtype, or an unknown flag bit;
 *       GDR_ERR_DEVICE       the HIP runtime reported a launch error.
 *     No C++ exception crosses this interface.
 *   - Values are not checked on the device: NaN/Inf propagate.  A decay gate
 *     of exactly 0 acts as a full reset without producing NaN (gates are
 *     clamped to FLT_MIN wherever a logarithm is taken).
 *   - Gate ranges: alpha in (0, 1]; write in [0, 1]; beta and erase in
 *     [0, 2] -- above 1 the per-token transition has a negative eigenvalue
 *     along k, down to the reflection I - 2 k k^T at 2.
 *   - T, B, H, N may be 0 (nothing is launched; s_final receives s0 or zeros
 *     when T == 0 and B*H > 0).  Any T >= 1 is accepted: the sequence is cut
 *     into internal chunks and the last one is partial.  The chunk length is
 *     not a parameter; results do not depend on it beyond rounding.
 *   - s0 == NULL means a zero initial state; s_final == NULL means the final
 *     state is not written.  s0 and s_final may be the same buffer.  q, k, v
 *     and the gates must not overlap o or s_final.
 *   - Thread safety: calls carry no shared mutable state and may be issued
 *     from several host threads on different streams, except that
 *     overlapping gdr_output_gate_bwd_noalloc calls on one GPU share its
 *     array.
 */
#ifndef GDR_H
#define GDR_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GDR_OK = 0,
    GDR_ERR_INVALID = 1,
    GDR_ERR_UNSUPPORTED = 2,
    GDR_ERR_DEVICE = 3
} gdr_status_t;

/* Largest head count the chunkwise calls accept: their kernels address one
 * chunk of tokens (H heads x d channels per token) with 32-bit byte offsets
 * from a 64-bit chunk base. */
#define GDR_MAX_HEADS 65536

typedef enum {
    GDR_F32 = 0,   /* IEEE binary32 */
    GDR_BF16 = 1   /* bfloat16, round-to-nearest-even on every store */
} gdr_dtype_t;

/*
 * Chunkwise forward of the gated delta rule over whole sequences.
 *
 * Algorithm: the chunkwise UT/WY form of the rule ("Gated Delta Networks",
 * "Method": chunkwise algorithm via the UT transform; review section 3.7,
 * the equations for U^g, S_[t+1] and O_[t]).  Within a chunk the scalar
 * gates enter through Gamma_rs = exp(g_r - g_s), g the within-chunk
 * cumulative log alpha; chunks are chained through the fp32 state.
 *
 *   B, T, H     batch, sequence length, heads (each >= 0)
 *   Dk, Dv      key and value head dims, each 64 or 128
 *   in_dt       dtype of q, k, v (GDR_F32 or GDR_BF16)
 *   q, k        [B, T, H, Dk] in_dt
 *   v           [B, T, H, Dv] in_dt
 *   alpha, beta [B, T, H] fp32 (scalar gates per token and head)
 *   s0          [B, H, Dv, Dk] fp32 or NULL (zero initial state)
 *   out_dt      dtype of o (GDR_F32 or GDR_BF16)
 *   o           [B, T, H, Dv] out_dt  (output, o_t = S_t q_t)
 *   s_final     [B, H, Dv, Dk] fp32 or NULL; may alias s0
 *
 * Precision: fp32 inputs are computed in fp32.  bf16 inputs run on bf16
 * matrix cores with fp32 accumulation; every product whose operand is a
 * computed (not input) value uses a two-term bf16 split of that operand, so
 * products carry ~16 significant bits.  Output rounding to bf16 (out_dt =
 * GDR_BF16) adds up to half a bf16 ulp of each output.
 */
gdr_status_t gdr_chunk_fwd(int64_t B, int64_t T, int64_t H, int64_t Dk,
                           int64_t Dv, gdr_dtype_t in_dt, const void *q,
                           const void *k, const void *v, const float *alpha,
                           const float *beta, const float *s0,
                           gdr_dtype_t out_dt, void *o, float *s_final,
                           hipStream_t stream);

/*
 * One decode token for N independent sequences, the state updated in place.
 *
 * For each (n, h) and each row i of S (value channel i), in one pass over
 * the old row: a_i = s_i . k, c_i = s_i . q; d_i = beta (v_i - alpha a_i);
 * s_i <- alpha s_i + d_i k; o_i = alpha c_i + d_i (k . q).  This is the rule
 * above for a single token with a fixed-size state (constant memory per
 * decoded token, as both GDN summaries describe decoding).
 *
 *   N, H        sequences, heads (each >= 0)
 *   Dk, Dv      64 or 128
 *   in_dt       dtype of q, k, v
 *   q, k        [N, H, Dk] in_dt
 *   v           [N, H, Dv] in_dt
 *   alpha, beta [N, H] fp32
 *   state       [N, H, Dv, Dk] fp32, read and overwritten
 *   out_dt      dtype of o
 *   o           [N, H, Dv] out_dt
 */
gdr_status_t gdr_recurrent_step(int64_t N, int64_t H, int64_t Dk, int64_t Dv,
                                gdr_dtype_t in_dt, const void *q,
                                const void *k, const void *v,
                                const float *alpha, const float *beta,
                                float *state, gdr_dtype_t out_dt, void *o,
                                hipStream_t stream);

/*
 * Chunkwise forward of Gated Delta Rule-2 ("Gated DeltaNet-2",
 * agihunt.info: per token, decay the state with the per-channel alpha_t on
 * the key axis, read the old value along b_t (.) k_t, write the residual of
 * w_t (.) v_t against that read along k_t; in chunks, the channel decay is
 * absorbed into an asymmetric rank-1 erase factor and solved in WY form):
 *
 *   S' = S_{t-1} diag(alpha_t),
 *   S_t = S' + (w_t (.) v_t - S' (b_t (.) k_t)) k_t^T,   o_t = S_t q_t.
 *
 *   q, k        [B, T, H, Dk] in_dt
 *   v           [B, T, H, Dv] in_dt
 *   alpha       [B, T, H, Dk] in_dt, per-key-channel decay in (0, 1]
 *   erase       [B, T, H, Dk] in_dt, b in [0, 2]
 *   write       [B, T, H, Dv] in_dt, w in [0, 1]
 *   s0, s_final, o, out_dt as for gdr_chunk_fwd.
 */
gdr_status_t gdr2_chunk_fwd(int64_t B, int64_t T, int64_t H, int64_t Dk,
                            int64_t Dv, gdr_dtype_t in_dt, const void *q,
                            const void *k, const void *v, const void *alpha,
                            const void *erase, const void *write,
                            const float *s0, gdr_dtype_t out_dt, void *o,
                            float *s_final, hipStream_t stream);

/*
 * Fused prologue: the _ex variants below take the same arguments as the
 * three calls above plus a `flags` word, an OR of
 *
 *   GDR_L2NORM_QK  normalise q_t and k_t to unit L2 norm per token and head
 *                  as they are loaded, the step the Gated DeltaNet block
 *                  applies to q and k right before the rule (review on
 *                  meaningful96.github.io, section 3.8, the q and k paths of
 *                  the block; the Gated DeltaNet-2 page keeps that block
 *                  design):
 *
 *                    x_hat = x / sqrt(sum_c x_c^2 + GDR_L2NORM_EPS)
 *
 *                  over the Dk channels, the sum taken in fp32 over the
 *                  input values.  The rule then runs on q_hat, k_hat
 *                  exactly as documented above (for Gated Delta Rule-2 the
 *                  erase direction becomes b (.) k_hat).  q and k in memory
 *                  are not modified.
 *
 * flags == 0 is the plain call.  A set bit not listed here returns
 * GDR_ERR_UNSUPPORTED and launches nothing.  Precision and every other
 * convention are those of the plain call; on the bf16 paths q_hat and k_hat
 * are never rounded back to bf16: the 1 / norm factors are applied to fp32
 * intermediate results or to operands that are split into hi/lo pairs.
 */
#define GDR_L2NORM_QK 1u

#define GDR_L2NORM_EPS 1e-6f

/*
 * Accepted by gdr2_chunk_bwd_split only (other calls return
 * GDR_ERR_UNSUPPORTED for it): skip the sequence split and run the plain
 * gdr2_chunk_bwd_ex over the whole sequence, whose states are fp32
 * throughout (nseg is then only range-checked; the split's workspace size
 * covers the plain call's).  Without the bit the split builds the
 * segments' start states with a matrix-core forward whose computed
 * operands all enter as hi/lo bf16 pairs, which keeps the gradients within
 * 1e-3 of rms of the oracle on the B1 H16 T32768 d128 long-context
 * workload (4 segments).
 */
#define GDR_SPLIT_FP32_STATES 2u

gdr_status_t gdr_chunk_fwd_ex(int64_t B, int64_t T, int64_t H, int64_t Dk,
                              int64_t Dv, gdr_dtype_t in_dt, const void *q,
                              const void *k, const void *v,
                              const float *alpha, const float *beta,
                              const float *s0, gdr_dtype_t out_dt, void *o,
                              float *s_final, uint32_t flags,
                              hipStream_t stream);

gdr_status_t gdr_recurrent_step_ex(int64_t N, int64_t H, int64_t Dk,
                                   int64_t Dv, gdr_dtype_t in_dt,
                                   const void *q, const void *k,
                                   const void *v, const float *alpha,
                                   const float *beta, float *state,
                                   gdr_dtype_t out_dt, void *o,
                                   uint32_t flags, hipStream_t stream);

gdr_status_t gdr2_chunk_fwd_ex(int64_t B, int64_t T, int64_t H, int64_t Dk,
                               int64_t Dv, gdr_dtype_t in_dt, const void *q,
                               const void *k, const void *v,
                               const void *alpha, const void *erase,
                               const void *write, const float *s0,
                               gdr_dtype_t out_dt, void *o, float *s_final,
                               uint32_t flags, hipStream_t stream);

/*
 * Sequence-split form of gdr_chunk_fwd_ex, for few long sequences (few
 * (b, h) pairs leave most compute units idle when each sequence runs as one
 * chain).  The rule maps a segment's start state affinely, S -> S P + R,
 * with R the segment's final state from a zero start and
 * P = prod_t alpha_t (I - beta_t k_t k_t^T) (the chunkwise form of the rule,
 * "Gated Delta Networks", agihunt.info, "Method"; GDN review on
 * meaningful96.github.io, section 3.4).  The call splits each sequence into
 * nseg segments of T / nseg tokens and runs the chunk kernels three times
 * over all segments side by side: for R, for P (v = 0 from the identity),
 * and, after a scan S_in(p) = S_in(p - 1) P_{p-1} + R_{p-1} with
 * S_in(0) = s0, for o and the final states.
 *
 *   arguments as for gdr_chunk_fwd_ex, plus
 *   nseg       segments per sequence, >= 1, dividing T; 1 is the plain call
 *              (no workspace needed)
 *   workspace  device memory of at least
 *              gdr_chunk_fwd_split_workspace_size(B, T, H, Dk, Dv, in_dt,
 *              nseg) bytes, 16-byte aligned, owned by the caller, contents
 *              irrelevant on entry and unspecified on return: R, P and the
 *              start states (fp32, B nseg H Dv Dk, B nseg H Dk Dk and
 *              B nseg H Dv Dk floats) and, for fp32 inputs only, a zero
 *              v for the P pass (B T H Dk floats) and, when Dk != Dv, that
 *              pass's discarded output (B T H Dk bf16)
 *
 * The results equal the plain call's up to rounding (the segments' states
 * are composed in fp32).  With fp32 inputs o is written three times (the
 * first two are overwritten); with bf16 inputs once.  The workspace size is 0 for arguments the call rejects
 * and when no workspace is needed.  Calls on one workspace must not overlap.
 */
size_t gdr_chunk_fwd_split_workspace_size(int64_t B, int64_t T, int64_t H,
                                          int64_t Dk, int64_t Dv,
                                          gdr_dtype_t in_dt, int64_t nseg);

gdr_status_t gdr_chunk_fwd_split(int64_t B, int64_t T, int64_t H, int64_t Dk,
                                 int64_t Dv, gdr_dtype_t in_dt, const void *q,
                                 const void *k, const void *v,
                                 const float *alpha, const float *beta,
                                 const float *s0, gdr_dtype_t out_dt, void *o,
                                 float *s_final, int64_t nseg, uint32_t flags,
                                 void *workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/*
 * Sequence-split form of gdr_chunk_bwd_ex, for few long sequences.  The
 * backward's carry composes like the state: dL/dS_in(p) = G_end(p) P_p^T +
 * N_p, where P_p is segment p's transition (as in gdr_chunk_fwd_split) and
 * N_p its own contribution (its backward from G_end = 0).  The call forms
 * every segment's start state and P_p with the split forward's passes,
 * runs the backward over all segments side by side from a zero end
 * gradient (N_p), scans the end gradients from the last segment to the
 * first, and runs the backward over all segments once more with them.
 *
 *   arguments as for gdr_chunk_bwd_ex, plus nseg (>= 1, dividing T; 1 is
 *   the plain call) and a workspace of at least
 *   gdr_chunk_bwd_split_workspace_size(B, T, H, Dk, Dv, in_dt, nseg) bytes
 *   (for nseg = 1 the plain call's), 16-byte aligned, owned by the caller
 *
 * Results equal the plain call's up to rounding.  The gradient outputs are
 * written twice (the first pass's values are overwritten).
 */
size_t gdr_chunk_bwd_split_workspace_size(int64_t B, int64_t T, int64_t H,
                                          int64_t Dk, int64_t Dv,
                                          gdr_dtype_t in_dt, int64_t nseg);

gdr_status_t gdr_chunk_bwd_split(int64_t B, int64_t T, int64_t H, int64_t Dk,
                                 int64_t Dv, gdr_dtype_t in_dt, const void *q,
                                 const void *k, const void *v,
                                 const float *alpha, const float *beta,
                                 const float *s0, gdr_dtype_t dout_dt,
                                 const void *dout, const float *ds_final,
                                 float *dq, float *dk, float *dv,
                                 float *dalpha, float *dbeta, float *ds0,
                                 int64_t nseg, uint32_t flags,
                                 void *workspace, size_t workspace_bytes,
                                 hipStream_t stream);

/*
 * The same two sequence-split calls for Gated Delta Rule-2: the rule maps a
 * segment's start state affinely as well (per token S -> S diag(alpha)
 * (I - e k^T) + ...), so P_p is again the segment run with v = 0 from the
 * identity (the P pass uses a zero write gate too).  Arguments as for
 * gdr2_chunk_fwd_ex and gdr2_chunk_bwd_ex plus nseg, flags and the
 * workspace; gdr2_chunk_fwd_split takes gdr_chunk_fwd_split_workspace_size
 * bytes (the same layout), gdr2_chunk_bwd_split its own size below.  The
 * backward's start-state passes split every computed operand into hi/lo
 * bf16 terms (the forward's own passes round E (.) lambda, A and T once,
 * which its o and S tolerate but the gradients through S would inherit);
 * GDR_SPLIT_FP32_STATES in flags runs the plain backward instead.
 */
gdr_status_t gdr2_chunk_fwd_split(int64_t B, int64_t T, int64_t H, int64_t Dk,
                                  int64_t Dv, gdr_dtype_t in_dt, const void *q,
                                  const void *k, const void *v,
                                  const void *alpha, const void *erase,
                                  const void *write, const float *s0,
                                  gdr_dtype_t out_dt, void *o, float *s_final,
                                  int64_t nseg, uint32_t flags,
                                  void *workspace, size_t workspace_bytes,
                                  hipStream_t stream);

size_t gdr2_chunk_bwd_split_workspace_size(int64_t B, int64_t T, int64_t H,
                                           int64_t Dk, int64_t Dv,
                                           gdr_dtype_t in_dt, int64_t nseg);

gdr_status_t gdr2_chunk_bwd_split(int64_t B, int64_t T, int64_t H, int64_t Dk,
                                  int64_t Dv, gdr_dtype_t in_dt, const void *q,
                                  const void *k, const void *v,
                                  const void *alpha, const void *erase,
                                  const void *write, const float *s0,
                                  gdr_dtype_t dout_dt, const void *dout,
                                  const float *ds_final, float *dq, float *dk,
                                  float *dv, float *dalpha, float *derase,
                                  float *dwrite, float *ds0, int64_t nseg,
                                  uint32_t flags, void *workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/*
 * Output gate of the block, applied to the rule's output o per token and
 * head over the Dv channels ("Gated DeltaNet-2", agihunt.info: the
 * recurrent output passes an RMSNorm and a SiLU output gate; GDN review on
 * meaningful96.github.io, section 3.8: normalisation and gating before the
 * output projection):
 *
 *   y = o / sqrt(mean_c o_c^2 + eps) * w * g * sigmoid(g)
 *
 *   N, H        tokens (B * T), heads (each >= 0)
 *   Dv          64 or 128
 *   o_dt, o     [N, H, Dv] (the output of the calls above)
 *   g_dt, g     [N, H, Dv], the gate branch's pre-activation
 *   w           [Dv] fp32, the norm's per-channel weight, or NULL (ones)
 *   eps         >= 0, added to the mean square inside the root
 *   out_dt, y   [N, H, Dv]; y may be o itself when out_dt == o_dt
 *
 * One pass over HBM (o, g in, y out).  gdr_chunk_fwd_gate below fuses the
 * same gate onto the stores of the scalar-gate forward.  o, g and y need
 * 16-byte alignment, w too when given.  Arithmetic in fp32; a bf16 y is
 * rounded to nearest even.
 */
gdr_status_t gdr_output_gate(int64_t N, int64_t H, int64_t Dv, gdr_dtype_t o_dt,
                             const void *o, gdr_dtype_t g_dt, const void *g,
                             const float *w, float eps, gdr_dtype_t out_dt,
                             void *y, hipStream_t stream);

/*
 * gdr_chunk_fwd followed by gdr_output_gate, with the gate fused on the
 * forward's stores: o is never written, y = o / sqrt(mean_c o_c^2 + eps) *
 * w * g * sigmoid(g) is (the block's RMSNorm and SiLU output gate after the
 * recurrence: "Gated DeltaNet-2", agihunt.info, block paragraph; GDN review
 * on meaningful96.github.io, section 3.8).
 *
 *   B, T, H, Dk, Dv, in_dt, q, k, v, alpha, beta, s0, s_final, flags
 *                 as for gdr_chunk_fwd_ex
 *   g_dt, g       [B, T, H, Dv] the gate branch's pre-activation
 *   w             [Dv] fp32 norm weight, or NULL (ones)
 *   eps           >= 0, inside the root
 *   out_dt, y     [B, T, H, Dv] (written)
 *   workspace     device memory of at least
 *                 gdr_chunk_fwd_gate_workspace_size(B, T, H, Dk, Dv, in_dt)
 *                 bytes, 16-byte aligned, owned by the caller: for bf16
 *                 inputs the row blocks' exchange of per-token sums of
 *                 squares (a few KB per head), for fp32 inputs an fp32 o
 *                 between the forward and the gate
 *
 * With bf16 inputs one kernel pass computes and gates o: a head's Dv rows
 * are split over workgroups, which trade per-token sums of squares through
 * the workspace.  The heads go out in cooperative launches of as many
 * workgroups as the GPU holds at once, so the call is not for HIP graph
 * capture.  Equals gdr_output_gate(gdr_chunk_fwd(...)) up to fp32 rounding;
 * GDR_ERR_DEVICE if a cooperative launch is refused.  q, k, v, g, y need
 * 16-byte alignment; alpha, beta element alignment; w 16 bytes when given.
 * T must stay below 2^36 (the kernel keeps chunk slots in 32 bits;
 * GDR_ERR_INVALID otherwise).
 */
size_t gdr_chunk_fwd_gate_workspace_size(int64_t B, int64_t T, int64_t H, int64_t Dk,
                                         int64_t Dv, gdr_dtype_t in_dt);

gdr_status_t gdr_chunk_fwd_gate(int64_t B, int64_t T, int64_t H, int64_t Dk,
                                int64_t Dv, gdr_dtype_t in_dt, const void *q,
                                const void *k, const void *v, const float *alpha,
                                const float *beta, const float *s0,
                                gdr_dtype_t g_dt, const void *g, const float *w,
                                float eps, gdr_dtype_t out_dt, void *y,
                                float *s_final, uint32_t flags, void *workspace,
                                size_t workspace_bytes, hipStream_t stream);

/*
 * Reverse mode of gdr_output_gate: with r = 1 / sqrt(mean o^2 + eps),
 * n = r o and s(g) = g sigmoid(g) per row, given dy = dL/dy,
 *
 *   dout = r (dn - n mean(n dn)),   dn = dy w s(g)
 *   dg   = dy n w sigmoid(g) (1 + g (1 - sigmoid(g)))
 *   dw   = sum over all rows of dy n s(g)
 *
 *   N, H, Dv, o_dt, o, g_dt, g, w, eps  as for gdr_output_gate (w NULL: ones)
 *   dy_dt, dy   [N, H, Dv] dL/dy
 *   dout, dg    [N, H, Dv] fp32 (written)
 *   dw          [Dv] fp32 (written), or NULL: not computed, no workspace
 *   workspace   when dw is given: device memory of at least
 *               gdr_output_gate_bwd_workspace_size(N, H, Dv) bytes (the
 *               workgroups' partial sums of dw, at most 2048 x Dv floats),
 *               16-byte aligned, owned by the caller
 *
 * One pass over o, g and dy plus a small reduction for dw.  All tensors
 * 16-byte aligned.  fp32 arithmetic; N H == 0 writes dw = 0.
 */
size_t gdr_output_gate_bwd_workspace_size(int64_t N, int64_t H, int64_t Dv);

gdr_status_t gdr_output_gate_bwd(int64_t N, int64_t H, int64_t Dv,
                                 gdr_dtype_t o_dt, const void *o,
                                 gdr_dtype_t g_dt, const void *g,
                                 const float *w, float eps, gdr_dtype_t dy_dt,
                                 const void *dy, float *dout, float *dg,
                                 float *dw, void *workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/*
 * gdr_output_gate_bwd without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving or training
 * loops, harnesses that forbid hipMalloc.  Same arguments and results as
 * gdr_output_gate_bwd minus workspace and workspace_bytes.
 *
 * The workgroups' dw partials go to an array the library holds in device
 * memory, GDR_GATE_BWD_SCRATCH_BYTES (1 MiB) per GPU, kept until the process
 * ends.  The partial count is capped at 2048 x Dv floats, so every valid
 * (N, H, Dv) fits; a call that would not fit returns GDR_ERR_INVALID.
 * The call allocates nothing: it enqueues the same kernels as
 * gdr_output_gate_bwd on `stream`.  `stream` must belong to the current
 * device (GDR_ERR_INVALID otherwise).  Every call on one GPU uses that GPU's
 * one array, and each call rewrites every partial it reads, so calls that
 * run one after another need no clearing; calls on one GPU that may
 * overlap (other streams, other host threads) race on the array and must be
 * ordered by the caller.  With dw NULL the array is not used.
 */
#define GDR_GATE_BWD_SCRATCH_BYTES (2048u * 128u * 4u)

gdr_status_t gdr_output_gate_bwd_noalloc(int64_t N, int64_t H, int64_t Dv,
                                         gdr_dtype_t o_dt, const void *o,
                                         gdr_dtype_t g_dt, const void *g,
                                         const float *w, float eps,
                                         gdr_dtype_t dy_dt, const void *dy,
                                         float *dout, float *dg, float *dw,
                                         hipStream_t stream);

/*
 * Reverse mode of gdr_chunk_fwd (the scalar-gate rule): the gradients of a
 * loss L through o and the final state, given dL/do and dL/dS_T.  It is the
 * chain rule through the chunkwise form of the rule ("Gated Delta
 * Networks", agihunt.info, "Method"; GDN review on meaningful96.github.io,
 * section 3.7), evaluated chunk by chunk in fp32: the pages' throughput
 * figures are for training, and the GDN-2 summary notes that a chunked
 * backward carries the gates inside its dot products.  With one decay per
 * token, every decay factor is a scalar per token or token pair, so the
 * gate gradients are formed per token (no per-channel decay tables).
 *
 *   q, k, v, alpha, beta, s0, in_dt  the forward's inputs, as for gdr_chunk_fwd
 *   dout_dt, dout  [B, T, H, Dv] dL/do (GDR_F32 or GDR_BF16)
 *   ds_final       [B, H, Dv, Dk] fp32 dL/dS_T, or NULL (zero)
 *   dq, dk         [B, T, H, Dk] fp32 (written).  Each is a sum over the
 *                  Dv/32 blocks of state rows, which the kernel adds with
 *                  fp32 atomic adds: the order of those additions varies,
 *                  so dq and dk can differ from run to run in the last
 *                  bits (every other output is the same bit for bit)
 *   dv             [B, T, H, Dv] fp32 (written)
 *   dalpha, dbeta  [B, T, H] fp32 (written).  dalpha is dL/d(log alpha)
 *                  divided by alpha, alpha clamped to FLT_MIN as in the
 *                  forward's logarithm
 *   ds0            [B, H, Dv, Dk] fp32 dL/dS_0, or NULL (not written)
 *   workspace      device memory of at least
 *                  gdr_chunk_bwd_workspace_size(B, T, H, Dk, Dv) bytes,
 *                  16-byte aligned, owned by the caller; its contents on
 *                  entry do not matter and on return are unspecified.
 *                  It holds the chunk-start states (B H ceil(T/16) Dv Dk
 *                  floats), every chunk's T and decayed Gram matrix
 *                  (512 floats per (b, h, chunk)), dq and
 *                  dk accumulators for GDR_L2NORM_QK (2 B T H Dk floats) and
 *                  per-row-block partial sums of the gate gradients
 *                  (2 (Dv/32) B T H floats).  A smaller workspace_bytes is
 *                  GDR_ERR_INVALID.
 *
 * Calls on one workspace must not overlap.  T == 0 copies ds_final (or
 * zeros) into ds0.  Alignment: as for gdr_chunk_fwd, plus dq, dk, dv,
 * dout and the workspace 16 bytes, dalpha and dbeta 4 bytes.
 */
size_t gdr_chunk_bwd_workspace_size(int64_t B, int64_t T, int64_t H,
                                    int64_t Dk, int64_t Dv);

gdr_status_t gdr_chunk_bwd(int64_t B, int64_t T, int64_t H, int64_t Dk,
                           int64_t Dv, gdr_dtype_t in_dt, const void *q,
                           const void *k, const void *v, const float *alpha,
                           const float *beta, const float *s0,
                           gdr_dtype_t dout_dt, const void *dout,
                           const float *ds_final, float *dq, float *dk,
                           float *dv, float *dalpha, float *dbeta, float *ds0,
                           void *workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * Reverse mode of gdr2_chunk_fwd (Gated Delta Rule-2): the gradients of a
 * loss L through o and the final state, given dL/do and dL/dS_T, by the
 * chain rule through the chunkwise form ("Gated DeltaNet-2", agihunt.info:
 * the chunked WY form with the channel decay absorbed into the erase
 * factor; the summary's remark that the backward keeps the gates inside
 * its dot products).  Chunks of 16 tokens, fp32 throughout.
 *
 *   q, k, v, alpha, erase, write, s0, in_dt  the forward's inputs, as for
 *                  gdr2_chunk_fwd
 *   dout_dt, dout  [B, T, H, Dv] dL/do (GDR_F32 or GDR_BF16)
 *   ds_final       [B, H, Dv, Dk] fp32 dL/dS_T, or NULL (zero)
 *   dq, dk         [B, T, H, Dk] fp32 (written)
 *   dv             [B, T, H, Dv] fp32 (written)
 *   dalpha         [B, T, H, Dk] fp32 (written): dL/d(log alpha) divided
 *                  by alpha, alpha clamped to FLT_MIN as in the forward
 *   derase         [B, T, H, Dk] fp32 dL/db (written)
 *   dwrite         [B, T, H, Dv] fp32 dL/dw (written)
 *   ds0            [B, H, Dv, Dk] fp32 dL/dS_0, or NULL (not written)
 *                  dq, dk, dalpha and derase are sums over the Dv/32
 *                  blocks of state rows, added by fp32 atomic adds whose
 *                  order varies: they can differ from run to run in the
 *                  last bits (dv, dwrite and ds0 are the same bit for bit)
 *   workspace      device memory of at least
 *                  gdr2_chunk_bwd_workspace_size(B, T, H, Dk, Dv) bytes,
 *                  16-byte aligned, owned by the caller, contents on entry
 *                  irrelevant and on return unspecified: the chunk-start
 *                  states (B H ceil(T/16) Dv Dk floats), every chunk's
 *                  T = (I + A)^{-1} (256 floats per (b, h, chunk)) and four
 *                  accumulators of B T H Dk floats.  A smaller
 *                  workspace_bytes is GDR_ERR_INVALID.
 *
 * Calls on one workspace must not overlap.  T == 0 copies ds_final (or
 * zeros) into ds0.  Every tensor argument needs 16-byte alignment.
 * gdr2_chunk_bwd_workspace_size returns 0 for arguments the call rejects.
 */
size_t gdr2_chunk_bwd_workspace_size(int64_t B, int64_t T, int64_t H,
                                     int64_t Dk, int64_t Dv);

gdr_status_t gdr2_chunk_bwd(int64_t B, int64_t T, int64_t H, int64_t Dk,
                            int64_t Dv, gdr_dtype_t in_dt, const void *q,
                            const void *k, const void *v, const void *alpha,
                            const void *erase, const void *write,
                            const float *s0, gdr_dtype_t dout_dt,
                            const void *dout, const float *ds_final,
                            float *dq, float *dk, float *dv, float *dalpha,
                            float *derase, float *dwrite, float *ds0,
                            void *workspace, size_t workspace_bytes,
                            hipStream_t stream);

/*
 * Backward of the _ex forwards: the same arguments as gdr_chunk_bwd and
 * gdr2_chunk_bwd plus `flags` (before the stream).  With GDR_L2NORM_QK the
 * forward normalised q and k on load; q and k here are the same raw
 * tensors, the kernels normalise them the same way, and dq, dk are the
 * gradients with respect to the raw q and k: the rule's gradients with
 * respect to q_hat, k_hat taken through the normalisation,
 *
 *   dx = (dx_hat - x_hat (x_hat . dx_hat)) / sqrt(|x|^2 + GDR_L2NORM_EPS)
 *
 * per token and head.  derase (GDN-2) is then with respect to b given
 * k_hat.  flags == 0 is the plain call; another bit is GDR_ERR_UNSUPPORTED.
 */
gdr_status_t gdr_chunk_bwd_ex(int64_t B, int64_t T, int64_t H, int64_t Dk,
                              int64_t Dv, gdr_dtype_t in_dt, const void *q,
                              const void *k, const void *v, const float *alpha,
                              const float *beta, const float *s0,
                              gdr_dtype_t dout_dt, const void *dout,
                              const float *ds_final, float *dq, float *dk,
                              float *dv, float *dalpha, float *dbeta,
                              float *ds0, void *workspace,
                              size_t workspace_bytes, uint32_t flags,
                              hipStream_t stream);

gdr_status_t gdr2_chunk_bwd_ex(int64_t B, int64_t T, int64_t H, int64_t Dk,
                               int64_t Dv, gdr_dtype_t in_dt, const void *q,
                               const void *k, const void *v, const void *alpha,
                               const void *erase, const void *write,
                               const float *s0, gdr_dtype_t dout_dt,
                               const void *dout, const float *ds_final,
                               float *dq, float *dk, float *dv, float *dalpha,
                               float *derase, float *dwrite, float *ds0,
                               void *workspace, size_t workspace_bytes,
                               uint32_t flags, hipStream_t stream);

/* Static, NUL-terminated description of a status code. */
const char *gdr_status_string(gdr_status_t s);

/* Library version as MAJOR * 10000 + MINOR * 100 + PATCH. */
int gdr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H */
