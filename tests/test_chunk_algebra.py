"""Chunkwise (UT/WY) form of the gated delta rules against the token-by-token
oracle, in fp64 NumPy (CPU only).

This pins the chunk algebra the HIP kernels evaluate — the readings of the
undefined or garbled symbols in the chunkwise equations of section 3.7 of the
meaningful96.github.io GDN review — before any kernel is trusted:

* Gamma_rs = exp(g_r - g_s) with g the within-chunk cumulative log alpha;
* the output mask M carries that decay and includes the diagonal;
* left arrow X = diag(gamma) X; right arrow K = diag(gamma_C / gamma) K;
  right arrow S = gamma_C S;  W = T diag(beta gamma) K,  U = T diag(beta) V.

For Gated DeltaNet-2 (agihunt.info summary: channel decay absorbed into an
asymmetric rank-1 erase factor, WY solve plus dense products, chunk 64) the
decayed products A and P are formed per 16-token block with the block's
left boundary as reference point, so every exponent on the operands is
bounded (see ``gdn2_chunk``).

Nothing here is shared with the HIP code; it is an independent derivation
checked against the oracle at every chunk size.
"""
import numpy as np
import pytest

import oracle
from oracle_pins import rand_gdn, rand_gdn2


def gdn_chunk(q, k, v, a, b, s0, C):
    """Scalar-gated chunkwise forward for one (b, h): q, k [T,Dk], v [T,Dv],
    a, b [T]; s0 [Dv,Dk].  Returns o [T,Dv], S [Dv,Dk]."""
    T, Dk = q.shape
    Dv = v.shape[1]
    S = s0.copy()
    o = np.zeros((T, Dv))
    for c0 in range(0, T, C):
        sl = slice(c0, min(c0 + C, T))
        Q, K, V, al, be = q[sl], k[sl], v[sl], a[sl], b[sl]
        n = Q.shape[0]
        g = np.cumsum(np.log(al))                       # g_r
        ge = np.tril(np.ones((n, n), dtype=bool))       # r >= s
        # Gamma_rs = exp(g_r - g_s) on r >= s; the exponent is masked before
        # exp so the (unused) upper part cannot overflow.
        Gam = np.exp(np.where(ge, g[:, None] - g[None, :], -np.inf))
        gt = np.tril(np.ones((n, n), dtype=bool), -1)
        A = np.where(gt, be[:, None] * Gam * (K @ K.T), 0.0)  # strictLower
        Tm = np.linalg.inv(np.eye(n) + A)               # T = (I + A)^-1
        W = Tm @ ((be * np.exp(g))[:, None] * K)   # left-arrow W
        U = Tm @ (be[:, None] * V)                      # U^g
        Vn = U - W @ S.T                                # U^g - W S^T
        P = np.where(ge, (Q @ K.T) * Gam, 0.0)          # mask incl. diagonal
        o[sl] = (np.exp(g)[:, None] * Q) @ S.T + P @ Vn
        S = np.exp(g[-1]) * S + Vn.T @ (np.exp(g[-1] - g)[:, None] * K)
    return o, S


def gdn2_chunk(q, k, v, a, e, w, s0, C, sub=16):
    """Channel-gated chunkwise forward for one (b, h).

    Within a chunk, G[r] = cumsum log alpha (per channel).  The decayed
    products A_sj = sum_c e_sc k_jc exp(G_sc - G_jc) (j < s) and
    P_rs = sum_c q_rc k_sc exp(G_rc - G_sc) (s <= r) are formed per block of
    ``sub`` rows: with m the position just before the block,
    exp(G_s - G_j) = exp(G_s - G_m) exp(G_m - G_j), the first factor <= 1
    and the second <= 1 for every earlier block; on the block's own diagonal
    the second factor is >= 1, bounded by the block's decay range.  When that
    range is too wide for fp32 (> 80 in natural-log units) the diagonal block
    is formed entry by entry instead.
    """
    T, Dk = q.shape
    Dv = v.shape[1]
    S = s0.copy()
    o = np.zeros((T, Dv))
    for c0 in range(0, T, C):
        sl = slice(c0, min(c0 + C, T))
        Q, K, V, Al, E, Wg = q[sl], k[sl], v[sl], a[sl], e[sl] * k[sl], w[sl]
        n = Q.shape[0]
        G = np.cumsum(np.log(Al), axis=0)               # [n, Dk]
        A = np.zeros((n, n))
        P = np.zeros((n, n))
        for r0 in range(0, n, sub):
            r1 = min(r0 + sub, n)
            Gm = G[r0 - 1] if r0 > 0 else np.zeros(Dk)
            Et = E[r0:r1] * np.exp(G[r0:r1] - Gm)       # <= |e|
            Qt = Q[r0:r1] * np.exp(G[r0:r1] - Gm)
            Kt = K[:r1] * np.exp(Gm - G[:r1])            # <= |k| for j < r0
            rng = np.max(Gm - G[r1 - 1])
            A[r0:r1, :r1] = Et @ Kt.T
            P[r0:r1, :r1] = Qt @ Kt.T
            if rng > 80.0:                               # exact diagonal block
                for s in range(r0, r1):
                    for j in range(r0, s + 1):
                        d = np.exp(G[s] - G[j])
                        A[s, j] = np.sum(E[s] * K[j] * d)
                        P[s, j] = np.sum(Q[s] * K[j] * d)
        A = np.where(np.tril(np.ones((n, n), dtype=bool), -1), A, 0.0)
        P = np.where(np.tril(np.ones((n, n), dtype=bool)), P, 0.0)
        Tm = np.linalg.inv(np.eye(n) + A)
        W2 = Tm @ (E * np.exp(G))
        U2 = Tm @ (Wg * V)
        Vn = U2 - W2 @ S.T
        o[sl] = (Q * np.exp(G)) @ S.T + P @ Vn
        S = S * np.exp(G[-1])[None, :] + Vn.T @ (K * np.exp(G[-1] - G))
    return o, S


@pytest.mark.parametrize("C", [1, 4, 16, 64, 200])
def test_gdn_chunk_form(C):
    q, k, v, a, b, S0 = rand_gdn(40, B=1, T=200, H=2, Dk=16, Dv=12)
    o_ref, s_ref = oracle.gdn_fwd(q, k, v, a, b, S0)
    for h in range(2):
        o, S = gdn_chunk(q[0, :, h], k[0, :, h], v[0, :, h], a[0, :, h],
                         b[0, :, h], S0[0, h], C)
        np.testing.assert_allclose(o, o_ref[0, :, h], rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(S, s_ref[0, h], rtol=1e-11, atol=1e-11)


def test_gdn_chunk_form_strong_decay():
    """Workload-like decay (alpha ~ exp(-softplus(N + 2))): the product of
    alphas over a 64-chunk underflows, exp of differences does not."""
    q, k, v, a, b, S0 = rand_gdn(41, B=1, T=160, H=1, Dk=16, Dv=16)
    g = np.random.Generator(np.random.PCG64(1))
    a = np.exp(-np.logaddexp(0, g.standard_normal(a.shape) + 2.0))
    a[0, 70, 0] = 1e-300                                 # near-total reset
    o_ref, s_ref = oracle.gdn_fwd(q, k, v, a, b, S0)
    o, S = gdn_chunk(q[0, :, 0], k[0, :, 0], v[0, :, 0], a[0, :, 0],
                     b[0, :, 0], S0[0, 0], 64)
    np.testing.assert_allclose(o, o_ref[0, :, 0], rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(S, s_ref[0, 0], rtol=1e-10, atol=1e-11)


@pytest.mark.parametrize("C", [1, 4, 16, 64, 150])
def test_gdn2_chunk_form(C):
    q, k, v, a, e, w, S0 = rand_gdn2(42, B=1, T=150, H=2, Dk=16, Dv=12)
    o_ref, s_ref = oracle.gdn2_fwd(q, k, v, a, e, w, S0)
    for h in range(2):
        o, S = gdn2_chunk(q[0, :, h], k[0, :, h], v[0, :, h], a[0, :, h],
                          e[0, :, h], w[0, :, h], S0[0, h], C)
        np.testing.assert_allclose(o, o_ref[0, :, h], rtol=1e-11, atol=1e-11)
        np.testing.assert_allclose(S, s_ref[0, h], rtol=1e-11, atol=1e-11)


def test_gdn2_chunk_form_wide_decay_range():
    """Per-channel alphas small enough that a 16-block's decay range passes
    the fp32 limit: the diagonal blocks take the entry-by-entry path."""
    q, k, v, a, e, w, S0 = rand_gdn2(43, B=1, T=128, H=1, Dk=16, Dv=8)
    g = np.random.Generator(np.random.PCG64(2))
    a = np.exp(-np.logaddexp(0, g.standard_normal(a.shape) + 2.0))
    a[0, 20:24, 0, 3] = 1e-12                            # range > 80
    o_ref, s_ref = oracle.gdn2_fwd(q, k, v, a, e, w, S0)
    o, S = gdn2_chunk(q[0, :, 0], k[0, :, 0], v[0, :, 0], a[0, :, 0],
                      e[0, :, 0], w[0, :, 0], S0[0, 0], 64)
    np.testing.assert_allclose(o, o_ref[0, :, 0], rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(S, s_ref[0, 0], rtol=1e-9, atol=1e-10)


def gdn_chunk_bwd(q, k, v, a, b, s0, dO, dSf, C):
    """Chunkwise reverse mode of the scalar-gated rule for one (b, h): the
    algebra the backward kernels evaluate.  Per chunk (n tokens, g the
    within-chunk cumulative log alpha, gamma = e^g, D_r = e^{g_C - g_r}):

      forward  A = diag(beta) (K K^T o Gamma) strict,  T = (I + A)^{-1},
               W = diag(beta gamma) K,  R = diag(beta) V - W S^T,  U = T R,
               P = (Q K^T o Gamma) incl. diagonal,
               O = diag(gamma) Q S^T + P U,  S' = gamma_C S + U^T diag(D) K
      reverse  dU = P^T dO + diag(D) K G^T,  dR = T^T dU,
               dP = dO U^T (masked),  dT = dU R^T,  dA = -T^T dT T^T (strict),
               dS = gamma_C G + dO^T diag(gamma) Q - dR^T W,  dV = diag(beta) dR,
               dW = -dR S,  dQ = diag(gamma) dO S + (dP o Gamma) K,
               dK = diag(D) U G + (dP o Gamma)^T Q + diag(beta gamma) dW
                    + diag(beta) dA~ K + (diag(beta) dA~)^T K   (dA~ = dA o Gamma),
               dbeta, dg from every place beta, gamma, Gamma, D, gamma_C enter,
               dlog alpha = reverse cumulative sum of dg inside the chunk,
    with G = dL/dS' carried from the next chunk.  Returns
    (dq, dk, dv, dalpha, dbeta, ds0)."""
    T, Dk = q.shape
    Dv = v.shape[1]
    chunks = [slice(c0, min(c0 + C, T)) for c0 in range(0, T, C)]
    S = s0.copy()
    starts = []
    for sl in chunks:                                   # forward: chunk-start states
        starts.append(S.copy())
        _, S = gdn_chunk(q[sl], k[sl], v[sl], a[sl], b[sl], S, C)
    G = dSf.copy()
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dla, db = np.zeros_like(a), np.zeros_like(b)
    for sl, S in zip(reversed(chunks), reversed(starts)):
        Q, K, V, al, be, dOc = q[sl], k[sl], v[sl], a[sl], b[sl], dO[sl]
        n = Q.shape[0]
        g = np.cumsum(np.log(al))
        gam, gC = np.exp(g), np.exp(g[-1])
        D = np.exp(g[-1] - g)
        ge = np.tril(np.ones((n, n), dtype=bool))
        gt = np.tril(np.ones((n, n), dtype=bool), -1)
        Gam = np.exp(np.where(ge, g[:, None] - g[None, :], -np.inf))
        KK = K @ K.T
        A = np.where(gt, be[:, None] * Gam * KK, 0.0)
        Tm = np.linalg.inv(np.eye(n) + A)
        W = (be * gam)[:, None] * K
        R = be[:, None] * V - W @ S.T
        U = Tm @ R
        P = np.where(ge, (Q @ K.T) * Gam, 0.0)
        QS = Q @ S.T
        UG = U @ G                                       # n x Dk
        dU = P.T @ dOc + D[:, None] * (K @ G.T)
        dR = Tm.T @ dU
        dP = np.where(ge, dOc @ U.T, 0.0)
        dT = dU @ R.T
        dA = np.where(gt, -(Tm.T @ dT @ Tm.T), 0.0)
        dW = -dR @ S
        dPG = dP * Gam
        dAG = dA * Gam
        dq[sl] = gam[:, None] * (dOc @ S) + dPG @ K
        dk[sl] = (D[:, None] * UG + dPG.T @ Q + (be * gam)[:, None] * dW
                  + be[:, None] * (dAG @ K) + (be[:, None] * dAG).T @ K)
        dv[sl] = be[:, None] * dR
        wk = np.sum(dW * K, axis=1)
        db[sl] = np.sum(V * dR, axis=1) + gam * wk + np.sum(dAG * KK, axis=1)
        dgam = np.sum(dOc * QS, axis=1) + be * wk
        dD = np.sum(K * UG, axis=1)
        PP, AA = dP * P, dA * A
        dg = gam * dgam + PP.sum(1) - PP.sum(0) + AA.sum(1) - AA.sum(0) - D * dD
        dg[-1] += np.sum(D * dD) + gC * np.sum(S * G)
        dla[sl] = np.cumsum(dg[::-1])[::-1]
        G = gC * G + dOc.T @ (gam[:, None] * Q) - dR.T @ W
    return dq, dk, dv, dla / a, db, G


@pytest.mark.parametrize("C", [1, 4, 16, 32, 64])
def test_gdn_chunk_bwd_matches_oracle(C):
    q, k, v, a, b, S0 = rand_gdn(36, B=1, T=77, H=2, Dk=6, Dv=5)
    g = np.random.Generator(np.random.PCG64(37))
    do = g.standard_normal(v.shape)
    dsf = g.standard_normal(S0.shape)
    ref = oracle.gdn_bwd(q, k, v, a, b, S0, do, dsf)
    for h in range(2):
        got = gdn_chunk_bwd(q[0, :, h], k[0, :, h], v[0, :, h], a[0, :, h], b[0, :, h],
                            S0[0, h], do[0, :, h], dsf[0, h], C)
        want = [ref[0][0, :, h], ref[1][0, :, h], ref[2][0, :, h], ref[3][0, :, h],
                ref[4][0, :, h], ref[5][0, h]]
        for name, x, y in zip(("dq", "dk", "dv", "dalpha", "dbeta", "ds0"), got, want):
            np.testing.assert_allclose(x, y, rtol=1e-9, atol=1e-10 * max(1.0, np.abs(y).max()),
                                       err_msg=f"{name} C={C} h={h}")


def test_gdn_chunk_bwd_small_gates():
    """Gates near zero (alpha down to 1e-6) keep the chunk backward finite and
    equal to the oracle's."""
    q, k, v, a, b, S0 = rand_gdn(38, B=1, T=40, H=1, Dk=4, Dv=3)
    a = a.copy()
    a[0, 5, 0] = 1e-6
    a[0, 20:23, 0] = 1e-3
    g = np.random.Generator(np.random.PCG64(39))
    do = g.standard_normal(v.shape)
    dsf = g.standard_normal(S0.shape)
    ref = oracle.gdn_bwd(q, k, v, a, b, S0, do, dsf)
    got = gdn_chunk_bwd(q[0, :, 0], k[0, :, 0], v[0, :, 0], a[0, :, 0], b[0, :, 0], S0[0, 0],
                        do[0, :, 0], dsf[0, 0], 16)
    want = [ref[0][0, :, 0], ref[1][0, :, 0], ref[2][0, :, 0], ref[3][0, :, 0], ref[4][0, :, 0],
            ref[5][0, 0]]
    for x, y in zip(got, want):
        np.testing.assert_allclose(x, y, rtol=1e-8, atol=1e-9 * max(1.0, np.abs(y).max()))


def gdn_chunk_bwd_tokens(q, k, v, a, b, s0, dO, dSf, C, nrb):
    """The scalar-gate reverse mode in the form gdr_chunk_bwd's kernel
    evaluates: the state rows in nrb blocks, each block's share of every
    gradient summed, and the gate gradients formed per token.  Per chunk
    (lam = e^g, rho = lam_C / lam, Gamma_rs = e^{g_r - g_s}) and row block:

      X = V - diag(lam) K S^T,  R = diag(beta) X,  U = T R,  KG = K G^T,
      dU = P^T dO + diag(rho) KG,  dR = T^T dU,  dP = dO U^T,  dA = -T^T (dU R^T) T^T,
      D_P = dP o Gamma,  D_A = dA o Gamma,  M = diag(beta) D_A + D_A^T diag(beta),
      dq += D_P K + (diag(lam) dO) S,
      dk += M K + D_P^T Q + (diag(rho) U) G - (diag(beta lam) dR) S,
      dbeta += rowsum(dR o X) + rowsum(dA o AK)            (AK = Gamma o K K^T, s < r)
      tau = -beta rowsum(dR o (V - X)) + rowsum(Q o (diag(lam) dO) S)
      kappa = rho rowsum(U o KG),  W = dA o A + dP o P,
      dlog alpha_t += sum_{r >= t} tau_r + sum_{r < t} kappa_r
                      + lam_C <G, S> + sum_{r >= t > s} W_rs,
      G <- lam_C G + (diag(lam) dO)^T Q - (diag(beta lam) dR)^T K."""
    T, Dk = q.shape
    Dv = v.shape[1]
    blocks = np.array_split(np.arange(Dv), nrb)
    chunks = [slice(c0, min(c0 + C, T)) for c0 in range(0, T, C)]
    S = s0.copy()
    starts = []
    for sl in chunks:
        starts.append(S.copy())
        _, S = gdn_chunk(q[sl], k[sl], v[sl], a[sl], b[sl], S, C)
    G = dSf.copy()
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dla, db = np.zeros_like(a), np.zeros_like(b)
    for sl, S in zip(reversed(chunks), reversed(starts)):
        Q, K, al, be = q[sl], k[sl], a[sl], b[sl]
        n = Q.shape[0]
        g = np.cumsum(np.log(al))
        lam, lC = np.exp(g), np.exp(g[-1])
        rho = np.exp(g[-1] - g)
        ge = np.tril(np.ones((n, n), dtype=bool))
        gt = np.tril(np.ones((n, n), dtype=bool), -1)
        Gam = np.exp(np.where(ge, g[:, None] - g[None, :], -np.inf))
        AK = np.where(gt, Gam * (K @ K.T), 0.0)
        A = be[:, None] * AK
        Tm = np.linalg.inv(np.eye(n) + A)
        P = np.where(ge, Gam * (Q @ K.T), 0.0)
        Gn = np.empty_like(G)
        for rows in blocks:
            Sb, Gb, V, dOb = S[rows], G[rows], v[sl][:, rows], dO[sl][:, rows]
            X = V - lam[:, None] * (K @ Sb.T)
            R = be[:, None] * X
            U = Tm @ R
            KG = K @ Gb.T
            dU = P.T @ dOb + rho[:, None] * KG
            dR = Tm.T @ dU
            dP = np.where(ge, dOb @ U.T, 0.0)
            dA = np.where(gt, -(Tm.T @ (dU @ R.T) @ Tm.T), 0.0)
            DP, DA = dP * Gam, dA * Gam
            M = be[:, None] * DA + DA.T * be[None, :]
            dOl = lam[:, None] * dOb
            dRbl = (be * lam)[:, None] * dR
            dOlS = dOl @ Sb
            dq[sl] += DP @ K + dOlS
            dk[sl] += M @ K + DP.T @ Q + (rho[:, None] * U) @ Gb - dRbl @ Sb
            dv[sl][:, rows] = be[:, None] * dR
            db[sl] += np.sum(dR * X, axis=1) + np.sum(dA * AK, axis=1)
            tau = -be * np.sum(dR * (V - X), axis=1) + np.sum(Q * dOlS, axis=1)
            kap = rho * np.sum(U * KG, axis=1)
            W = dA * A + dP * P
            gs = lC * np.sum(Gb * Sb)
            for t in range(n):
                dla[sl][t] += (tau[t:].sum() + kap[:t].sum() + gs + W[t:, :t].sum())
            Gn[rows] = lC * Gb + dOl.T @ Q - dRbl.T @ K
        G = Gn
    return dq, dk, dv, dla / a, db, G


@pytest.mark.parametrize("C,nrb", [(1, 1), (4, 2), (16, 1), (16, 2), (16, 5)])
def test_gdn_chunk_bwd_token_form_matches_oracle(C, nrb):
    """The kernel's per-token gate gradients (suffix sums of tau, prefix sums
    of kappa, pair sums across t, lam_C <G, S>) and its row-block split of
    every gradient give the oracle's backward."""
    q, k, v, a, b, S0 = rand_gdn(40, B=1, T=53, H=1, Dk=6, Dv=5)
    g = np.random.Generator(np.random.PCG64(41))
    do = g.standard_normal(v.shape)
    dsf = g.standard_normal(S0.shape)
    ref = oracle.gdn_bwd(q, k, v, a, b, S0, do, dsf)
    got = gdn_chunk_bwd_tokens(q[0, :, 0], k[0, :, 0], v[0, :, 0], a[0, :, 0], b[0, :, 0],
                               S0[0, 0], do[0, :, 0], dsf[0, 0], C, nrb)
    want = [ref[0][0, :, 0], ref[1][0, :, 0], ref[2][0, :, 0], ref[3][0, :, 0], ref[4][0, :, 0],
            ref[5][0, 0]]
    for name, x, y in zip(("dq", "dk", "dv", "dalpha", "dbeta", "ds0"), got, want):
        np.testing.assert_allclose(x, y, rtol=1e-9, atol=1e-10 * max(1.0, np.abs(y).max()),
                                   err_msg=f"{name} C={C} nrb={nrb}")


def gdn2_chunk_bwd(q, k, v, a, e, w, s0, dO, dSf, C):
    """Chunkwise reverse mode of Gated Delta Rule-2 for one (b, h).  Per chunk
    (G the within-chunk cumulative log alpha per channel, E = b (.) k,
    Gamma_rsc = e^{G_rc - G_sc}, E~ = E (.) e^G, Q~ = Q (.) e^G,
    K~ = K (.) e^{G_C - G}, lambda_C = e^{G_C}):

      forward  A_rs = sum_c E_rc K_sc Gamma_rsc (s < r),
               P_rs = sum_c Q_rc K_sc Gamma_rsc (s <= r),  T = (I + A)^{-1},
               R = w (.) v - E~ S^T,  U = T R,  O = Q~ S^T + P U,
               S' = S diag(lambda_C) + U^T K~
      reverse  dU = P^T dO + K~ G^T,  dR = T^T dU,  dP = dO U^T (masked),
               dA = -T^T (dU R^T) T^T (strict),  dw = dR (.) v,  dv = dR (.) w,
               dE~ = -dR S,  dQ~ = dO S,  dK~ = U G,
               dS = G diag(lambda_C) + dO^T Q~ - dR^T E~,
               and the A, P, E~, Q~, K~, lambda_C terms into dE, dQ, dK, dG
               (the decay inside the dot products: a per-channel dG),
               db = dE (.) K,  dK += dE (.) b,
               dlog alpha = reverse cumulative sum of dG inside the chunk.
    Returns (dq, dk, dv, dalpha, derase, dwrite, ds0)."""
    T, Dk = q.shape
    chunks = [slice(c0, min(c0 + C, T)) for c0 in range(0, T, C)]
    S = s0.copy()
    starts = []
    for sl in chunks:
        starts.append(S.copy())
        _, S = gdn2_chunk(q[sl], k[sl], v[sl], a[sl], e[sl], w[sl], S, C)
    Gr = dSf.copy()
    out = [np.zeros_like(q), np.zeros_like(k), np.zeros_like(v), np.zeros_like(a),
           np.zeros_like(e), np.zeros_like(w)]
    for sl, S in zip(reversed(chunks), reversed(starts)):
        Q, K, V, Al, B_, W_ = q[sl], k[sl], v[sl], a[sl], e[sl], w[sl]
        dOc = dO[sl]
        n = Q.shape[0]
        E = B_ * K
        G = np.cumsum(np.log(Al), axis=0)
        Gam = np.exp(np.minimum(G[:, None, :] - G[None, :, :], 0.0))    # [r, s, c]
        lt = np.tril(np.ones((n, n)), -1)
        le = np.tril(np.ones((n, n)))
        A = np.einsum('rc,sc,rsc->rs', E, K, Gam) * lt
        P = np.einsum('rc,sc,rsc->rs', Q, K, Gam) * le
        Tm = np.linalg.inv(np.eye(n) + A)
        eG = np.exp(G)
        Et, Qt, Kt = E * eG, Q * eG, K * np.exp(G[-1] - G)
        lC = np.exp(G[-1])
        R = W_ * V - Et @ S.T
        U = Tm @ R
        dU = P.T @ dOc + Kt @ Gr.T
        dR = Tm.T @ dU
        dP = (dOc @ U.T) * le
        dA = -(Tm.T @ (dU @ R.T) @ Tm.T) * lt
        dEt, dQt, dKt = -dR @ S, dOc @ S, U @ Gr
        dlC = np.sum(Gr * S, axis=0)
        dE = np.einsum('rs,sc,rsc->rc', dA, K, Gam) + dEt * eG
        dQ = np.einsum('rs,sc,rsc->rc', dP, K, Gam) + dQt * eG
        dK = (np.einsum('rs,rc,rsc->sc', dA, E, Gam) + np.einsum('rs,rc,rsc->sc', dP, Q, Gam)
              + dKt * np.exp(G[-1] - G))
        tA = np.einsum('rs,rc,sc,rsc->rsc', dA, E, K, Gam)
        tP = np.einsum('rs,rc,sc,rsc->rsc', dP, Q, K, Gam)
        dG = (tA.sum(1) - tA.sum(0) + tP.sum(1) - tP.sum(0) + dEt * Et + dQt * Qt
              - dKt * Kt)
        dG[-1] += np.sum(dKt * Kt, axis=0) + dlC * lC
        out[0][sl] = dQ
        out[1][sl] = dK + dE * B_
        out[2][sl] = dR * W_
        out[3][sl] = np.cumsum(dG[::-1], axis=0)[::-1] / Al
        out[4][sl] = dE * K
        out[5][sl] = dR * V
        Gr = Gr * lC[None, :] + dOc.T @ Qt - dR.T @ Et
    return tuple(out) + (Gr,)


def gdn2_dlog_alpha_split(Gr_S, Kt_, dKt, Et_, dEt, Qt_, dQt, E, dEa, Q, dQa, K, dKa, lC, n):
    """d log alpha of one chunk without the cancelling cumulative sum:
    suffix sums of dE~ (.) E~ + dQ~ (.) Q~, prefix sums of dK~ (.) K~, the
    lambda_C term on every token, and the pair terms (which sum to zero over
    the chunk) as a suffix sum for the later half of the chunk and minus a
    prefix sum for the earlier half."""
    pr = E * dEa + Q * dQa - K * dKa
    tl = dEt * Et_ + dQt * Qt_
    kk = dKt * Kt_
    out = np.zeros_like(pr)
    for t in range(n):
        pair = pr[t:].sum(0) if t >= n // 2 else -pr[:t].sum(0)
        out[t] = tl[t:].sum(0) + kk[:t].sum(0) + Gr_S * lC + pair
    return out


def test_gdn2_dlog_alpha_split_form():
    """The split form equals the reverse cumulative sum of dG (the chunk's
    pair terms cancel exactly) on random chunk quantities."""
    g = np.random.Generator(np.random.PCG64(46))
    n, d = 16, 7
    E, K, Q = (g.standard_normal((n, d)) for _ in range(3))
    Gm = np.cumsum(-np.abs(g.standard_normal((n, d))), axis=0)
    Gam = np.exp(np.minimum(Gm[:, None, :] - Gm[None, :, :], 0.0))
    dA = np.tril(g.standard_normal((n, n)), -1)
    dP = np.tril(g.standard_normal((n, n)))
    dEa = np.einsum('rs,sc,rsc->rc', dA, K, Gam)
    dQa = np.einsum('rs,sc,rsc->rc', dP, K, Gam)
    dKa = np.einsum('rs,rc,rsc->sc', dA, E, Gam) + np.einsum('rs,rc,rsc->sc', dP, Q, Gam)
    Et_, Qt_, Kt_ = E * np.exp(Gm), Q * np.exp(Gm), K * np.exp(Gm[-1] - Gm)
    dEt, dQt, dKt = (g.standard_normal((n, d)) for _ in range(3))
    GS, lC = g.standard_normal(d), np.exp(Gm[-1])
    dG = E * dEa + Q * dQa - K * dKa + dEt * Et_ + dQt * Qt_ - dKt * Kt_
    dG[-1] += np.sum(dKt * Kt_, axis=0) + GS * lC
    want = np.cumsum(dG[::-1], axis=0)[::-1]
    got = gdn2_dlog_alpha_split(GS, Kt_, dKt, Et_, dEt, Qt_, dQt, E, dEa, Q, dQa, K, dKa, lC, n)
    np.testing.assert_allclose(got, want, rtol=1e-10, atol=1e-10 * np.abs(want).max())


@pytest.mark.parametrize("C", [1, 4, 16, 32])
def test_gdn2_chunk_bwd_matches_oracle(C):
    q, k, v, a, e, w, S0 = rand_gdn2(44, B=1, T=45, H=2, Dk=6, Dv=5)
    g = np.random.Generator(np.random.PCG64(45))
    do = g.standard_normal(v.shape)
    dsf = g.standard_normal(S0.shape)
    ref = oracle.gdn2_bwd(q, k, v, a, e, w, S0, do, dsf)
    names = ("dq", "dk", "dv", "dalpha", "derase", "dwrite", "ds0")
    for h in range(2):
        got = gdn2_chunk_bwd(q[0, :, h], k[0, :, h], v[0, :, h], a[0, :, h], e[0, :, h],
                             w[0, :, h], S0[0, h], do[0, :, h], dsf[0, h], C)
        want = [x[0, :, h] for x in ref[:6]] + [ref[6][0, h]]
        for name, x, y in zip(names, got, want):
            np.testing.assert_allclose(x, y, rtol=1e-9, atol=1e-10 * max(1.0, np.abs(y).max()),
                                       err_msg=f"{name} C={C} h={h}")


@pytest.mark.parametrize("nseg", [2, 3, 6])
def test_segment_split_composes_to_the_recurrence(nseg):
    """The sequence-split forward's identity, with the oracle only: each
    segment maps its start state affinely, S -> S P + R, where R is the
    segment run from zero and P the run with v = 0 from the identity; the
    scan S_in(p) = S_in(p-1) P_{p-1} + R_{p-1} from S_0 gives every
    segment's start state, and re-running each segment from it gives the
    whole sequence's o and final state."""
    T, H, Dk, Dv = 36, 2, 6, 5
    q, k, v, a, b, S0 = rand_gdn(47 + nseg, T=T, H=H, Dk=Dk, Dv=Dv)
    o_ref, s_ref = oracle.gdn_fwd(q, k, v, a, b, S0)
    L = T // nseg
    seg = lambda x, p: x[:, p * L:(p + 1) * L]
    eye = np.broadcast_to(np.eye(Dk), (1, H, Dk, Dk)).copy()
    Sin = S0.copy()
    o = np.empty_like(o_ref)
    s_last = None
    for p in range(nseg):
        qs, ks, vs, as_, bs = (seg(x, p) for x in (q, k, v, a, b))
        _, R = oracle.gdn_fwd(qs, ks, vs, as_, bs, None)
        _, P = oracle.gdn_fwd(qs, ks, np.zeros((1, L, H, Dk)), as_, bs, eye)
        op, s_last = oracle.gdn_fwd(qs, ks, vs, as_, bs, Sin)
        o[:, p * L:(p + 1) * L] = op
        np.testing.assert_allclose(s_last, Sin @ P + R, rtol=1e-11, atol=1e-11)
        Sin = Sin @ P + R
    np.testing.assert_allclose(o, o_ref, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(s_last, s_ref, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("nseg", [2, 3])
def test_segment_split_backward_composes(nseg):
    """The sequence-split backward's identity, with the oracle only: a
    segment's dL/dS_in is G_end P^T + N, N its backward from G_end = 0 and P
    its transition; scanning G_end from the last segment and re-running each
    segment's backward from its start state gives the whole sequence's
    gradients."""
    T, H, Dk, Dv = 24, 2, 5, 4
    q, k, v, a, b, S0 = rand_gdn(60 + nseg, T=T, H=H, Dk=Dk, Dv=Dv)
    g = np.random.Generator(np.random.PCG64(61))
    do = g.standard_normal(v.shape)
    dsf = g.standard_normal(S0.shape)
    ref = oracle.gdn_bwd(q, k, v, a, b, S0, do, dsf)
    L = T // nseg
    seg = lambda x, p: x[:, p * L:(p + 1) * L]
    eye = np.broadcast_to(np.eye(Dk), (1, H, Dk, Dk)).copy()
    Sin, P, N = [], [], []
    S = S0.copy()
    for p in range(nseg):
        qs, ks, vs, as_, bs = (seg(x, p) for x in (q, k, v, a, b))
        Sin.append(S)
        _, Pp = oracle.gdn_fwd(qs, ks, np.zeros((1, L, H, Dk)), as_, bs, eye)
        _, S = oracle.gdn_fwd(qs, ks, vs, as_, bs, S)
        P.append(Pp)
        N.append(oracle.gdn_bwd(qs, ks, vs, as_, bs, Sin[p], seg(do, p), None)[5])
    G = dsf.copy()
    got = [np.zeros_like(x) for x in ref[:5]]
    for p in reversed(range(nseg)):
        qs, ks, vs, as_, bs = (seg(x, p) for x in (q, k, v, a, b))
        gp = oracle.gdn_bwd(qs, ks, vs, as_, bs, Sin[p], seg(do, p), G)
        np.testing.assert_allclose(gp[5], G @ np.swapaxes(P[p], -1, -2) + N[p], rtol=1e-10,
                                   atol=1e-10)
        for i in range(5):
            got[i][:, p * L:(p + 1) * L] = gp[i]
        G = gp[5]
    for i in range(5):
        np.testing.assert_allclose(got[i], ref[i], rtol=1e-9, atol=1e-10)
    np.testing.assert_allclose(G, ref[5], rtol=1e-9, atol=1e-10)
