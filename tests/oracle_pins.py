"""Pins that tie the fp64 oracle to facts the pages and the mathematics fix.

Each ``pin_*`` takes an ``oracle.OracleLib`` and raises AssertionError when
the oracle disagrees.  ``test_oracle.py`` runs them on the real oracle and
``test_oracle_mutants.py`` runs them on deliberately broken copies to show
that each plausible slip (a dropped term, a wrong sign, a shifted index, a
transposed operand) trips at least one of them.

None of them re-types the oracle's loop: they use exact worked examples,
closed forms, invariants, independent formulations (the DeltaNet delta
form, the SGD gradient computed by autograd, the literal transition-matrix
product in exact rationals) and special cases that reduce to a library
routine.
"""
from __future__ import annotations

import json
import os
from fractions import Fraction

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def rand_gdn(seed, B=1, T=12, H=2, Dk=6, Dv=5, s0=True, alpha=None,
             beta=None):
    g = _rng(seed)
    q = _unit(g.standard_normal((B, T, H, Dk)))
    k = _unit(g.standard_normal((B, T, H, Dk)))
    v = g.standard_normal((B, T, H, Dv))
    a = g.uniform(0.3, 1.0, (B, T, H)) if alpha is None else \
        np.full((B, T, H), float(alpha))
    b = g.uniform(0.0, 1.0, (B, T, H)) if beta is None else \
        np.full((B, T, H), float(beta))
    S0 = g.standard_normal((B, H, Dv, Dk)) if s0 else None
    return q, k, v, a, b, S0


def rand_gdn2(seed, B=1, T=10, H=2, Dk=6, Dv=5, s0=True):
    g = _rng(seed)
    q = _unit(g.standard_normal((B, T, H, Dk)))
    k = _unit(g.standard_normal((B, T, H, Dk)))
    v = g.standard_normal((B, T, H, Dv))
    a = g.uniform(0.3, 1.0, (B, T, H, Dk))
    e = g.uniform(0.0, 1.0, (B, T, H, Dk))
    w = g.uniform(0.0, 1.0, (B, T, H, Dv))
    S0 = g.standard_normal((B, H, Dv, Dk)) if s0 else None
    return q, k, v, a, e, w, S0


def _frac_arr(x):
    return np.array([[float(Fraction(c)) for c in row] for row in x])


def _load_golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --- exact worked examples --------------------------------------------------

def pin_golden_gdn(orc):
    for name in ("gdn_d2_t2.json", "gdn_dk3_dv2_t1.json"):
        g = _load_golden(name)
        sh = g["shape"]
        T, Dk, Dv = sh["T"], sh["Dk"], sh["Dv"]
        q = _frac_arr(g["q"]).reshape(1, T, 1, Dk)
        k = _frac_arr(g["k"]).reshape(1, T, 1, Dk)
        v = _frac_arr(g["v"]).reshape(1, T, 1, Dv)
        a = np.array([float(Fraction(x)) for x in g["alpha"]]).reshape(1, T, 1)
        b = np.array([float(Fraction(x)) for x in g["beta"]]).reshape(1, T, 1)
        s0 = None if g["s0"] is None else \
            _frac_arr(g["s0"]).reshape(1, 1, Dv, Dk)
        o, sf = orc.gdn_fwd(q, k, v, a, b, s0)
        np.testing.assert_allclose(o.reshape(T, Dv), _frac_arr(g["o"]),
                                   rtol=0, atol=1e-14, err_msg=name)
        np.testing.assert_allclose(sf.reshape(Dv, Dk),
                                   _frac_arr(g["s_final"]), rtol=0,
                                   atol=1e-14, err_msg=name)


def pin_golden_step(orc):
    g = _load_golden("gdn_dk3_dv2_t1.json")
    q = _frac_arr(g["q"]).reshape(1, 1, 3)
    k = _frac_arr(g["k"]).reshape(1, 1, 3)
    v = _frac_arr(g["v"]).reshape(1, 1, 2)
    a = np.array([[0.5]])
    b = np.array([[0.25]])
    st = np.ascontiguousarray(_frac_arr(g["s0"]).reshape(1, 1, 2, 3))
    o = orc.gdn_step(q, k, v, a, b, st)
    np.testing.assert_allclose(o.reshape(2), _frac_arr(g["o"]).reshape(2),
                               rtol=0, atol=1e-14)
    np.testing.assert_allclose(st.reshape(2, 3), _frac_arr(g["s_final"]),
                               rtol=0, atol=1e-14)


def pin_golden_gdn2(orc):
    g = _load_golden("gdn2_d2_t2.json")
    T, Dk, Dv = 2, 2, 2
    f = lambda key, d: _frac_arr(g[key]).reshape(1, T, 1, d)  # noqa: E731
    o, sf = orc.gdn2_fwd(f("q", Dk), f("k", Dk), f("v", Dv), f("alpha", Dk),
                         f("erase", Dk), f("write", Dv),
                         _frac_arr(g["s0"]).reshape(1, 1, Dv, Dk))
    np.testing.assert_allclose(o.reshape(T, Dv), _frac_arr(g["o"]), rtol=0,
                               atol=1e-14)
    np.testing.assert_allclose(sf.reshape(Dv, Dk), _frac_arr(g["s_final"]),
                               rtol=0, atol=1e-14)


# --- brute force in exact rationals: the literal transition-matrix product --

def _rat_vec(g, n, lo=-4, hi=5, den=4):
    return [Fraction(int(g.integers(lo, hi)), den) for _ in range(n)]


def _mat_mul(A, B):
    return [[sum(A[i][l] * B[l][j] for l in range(len(B)))
             for j in range(len(B[0]))] for i in range(len(A))]


def pin_exact_matrix_form_gdn(orc):
    """S_t = S_{t-1} M_t + beta v k^T with M_t = alpha (I - beta k k^T) formed
    as a d_k x d_k matrix, in exact rational arithmetic."""
    g = _rng(7)
    T, Dk, Dv = 4, 3, 2
    S = [[Fraction(int(g.integers(-3, 4)), 2) for _ in range(Dk)]
         for _ in range(Dv)]
    s0 = np.array([[float(x) for x in r] for r in S]).reshape(1, 1, Dv, Dk)
    qs, ks, vs, al, be, outs = [], [], [], [], [], []
    for _ in range(T):
        q, k, v = _rat_vec(g, Dk), _rat_vec(g, Dk), _rat_vec(g, Dv)
        a = Fraction(int(g.integers(1, 9)), 8)
        b = Fraction(int(g.integers(0, 9)), 8)
        M = [[a * ((1 if i == j else 0) - b * k[i] * k[j]) for j in range(Dk)]
             for i in range(Dk)]
        SM = _mat_mul(S, M)
        S = [[SM[i][j] + b * v[i] * k[j] for j in range(Dk)]
             for i in range(Dv)]
        outs.append([sum(S[i][j] * q[j] for j in range(Dk))
                     for i in range(Dv)])
        qs.append(q); ks.append(k); vs.append(v); al.append(a); be.append(b)
    arr = lambda x, d: np.array(x, dtype=float).reshape(1, T, 1, d)  # noqa
    o, sf = orc.gdn_fwd(arr([[float(c) for c in r] for r in qs], Dk),
                        arr([[float(c) for c in r] for r in ks], Dk),
                        arr([[float(c) for c in r] for r in vs], Dv),
                        np.array([float(x) for x in al]).reshape(1, T, 1),
                        np.array([float(x) for x in be]).reshape(1, T, 1), s0)
    np.testing.assert_allclose(o.reshape(T, Dv),
                               np.array(outs, dtype=float), rtol=1e-13,
                               atol=1e-13)
    np.testing.assert_allclose(sf.reshape(Dv, Dk), np.array(S, dtype=float),
                               rtol=1e-13, atol=1e-13)


def pin_exact_matrix_form_gdn2(orc):
    """S_t = S_{t-1} diag(alpha)(I - (b.k) k^T) + (w.v) k^T in exact
    rationals, the matrix form of decay, read along b.k, write along k."""
    g = _rng(8)
    T, Dk, Dv = 4, 3, 2
    S = [[Fraction(int(g.integers(-3, 4)), 2) for _ in range(Dk)]
         for _ in range(Dv)]
    s0 = np.array([[float(x) for x in r] for r in S]).reshape(1, 1, Dv, Dk)
    rec = {n: [] for n in "qkvaew"}
    outs = []
    for _ in range(T):
        q, k, v = _rat_vec(g, Dk), _rat_vec(g, Dk), _rat_vec(g, Dv)
        a = [Fraction(int(g.integers(1, 9)), 8) for _ in range(Dk)]
        e = [Fraction(int(g.integers(0, 9)), 8) for _ in range(Dk)]
        w = [Fraction(int(g.integers(0, 9)), 8) for _ in range(Dv)]
        M = [[a[i] * ((1 if i == j else 0) - e[i] * k[i] * k[j])
              for j in range(Dk)] for i in range(Dk)]
        SM = _mat_mul(S, M)
        S = [[SM[i][j] + w[i] * v[i] * k[j] for j in range(Dk)]
             for i in range(Dv)]
        outs.append([sum(S[i][j] * q[j] for j in range(Dk))
                     for i in range(Dv)])
        for n, x in zip("qkvaew", (q, k, v, a, e, w)):
            rec[n].append([float(c) for c in x])
    arr = lambda n, d: np.array(rec[n]).reshape(1, T, 1, d)  # noqa: E731
    o, sf = orc.gdn2_fwd(arr("q", Dk), arr("k", Dk), arr("v", Dv),
                         arr("a", Dk), arr("e", Dk), arr("w", Dv), s0)
    np.testing.assert_allclose(o.reshape(T, Dv), np.array(outs, dtype=float),
                               rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(sf.reshape(Dv, Dk), np.array(S, dtype=float),
                               rtol=1e-13, atol=1e-13)


# --- special cases and invariants -------------------------------------------

def pin_a_deltanet(orc):
    """alpha = 1: DeltaNet in its delta form S + beta (v - S k) k^T
    (review section 3.3)."""
    q, k, v, a, b, S0 = rand_gdn(11, alpha=1.0)
    o, sf = orc.gdn_fwd(q, k, v, a, b, S0)
    B, T, H, _ = q.shape
    for bb in range(B):
        for h in range(H):
            S = S0[bb, h].copy()
            for t in range(T):
                kt = k[bb, t, h]
                S = S + b[bb, t, h] * np.outer(v[bb, t, h] - S @ kt, kt)
                np.testing.assert_allclose(o[bb, t, h], S @ q[bb, t, h],
                                           rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(sf[bb, h], S, rtol=1e-12, atol=1e-12)


def pin_b_pure_decay(orc):
    """beta = 0: S_t = alpha_t S_{t-1}; closed form with the product of
    alphas taken in log space."""
    q, k, v, a, b, S0 = rand_gdn(12, T=40, beta=0.0)
    a = np.exp(-np.abs(_rng(3).standard_normal(a.shape)) * 2)
    o, sf = orc.gdn_fwd(q, k, v, a, b, S0)
    cum = np.exp(np.cumsum(np.log(a), axis=1))           # [B,T,H]
    ref_o = np.einsum("bth,bhij,bthj->bthi", cum, S0, q)
    np.testing.assert_allclose(o, ref_o, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(sf, cum[:, -1][:, :, None, None] * S0,
                               rtol=1e-12, atol=1e-14)


def pin_c_unit_key_write(orc):
    """beta = 1, |k| = 1: after the write, S_t k_t = v_t exactly (the
    delta rule replaces the value stored under k_t)."""
    q, k, v, a, b, S0 = rand_gdn(13, T=6, beta=1.0)
    for t in range(1, 7):
        _, sf = orc.gdn_fwd(q[:, :t], k[:, :t], v[:, :t], a[:, :t],
                            b[:, :t], S0)
        got = np.einsum("bhij,bhj->bhi", sf, k[:, t - 1])
        np.testing.assert_allclose(got, v[:, t - 1], rtol=0, atol=1e-13)


def pin_d_orthonormal_retrieval(orc):
    """n <= d_k orthonormal keys, alpha = beta = 1, zero state: every v_i is
    retrieved by its key (brute force at d in {8, 16, 64})."""
    for d in (8, 16, 64):
        g = _rng(d)
        n = d if d < 64 else 40
        Qm, _ = np.linalg.qr(g.standard_normal((d, d)))
        keys = Qm[:, :n].T.reshape(1, n, 1, d)
        vals = g.standard_normal((1, n, 1, d))
        q = _unit(g.standard_normal((1, n, 1, d)))
        one = np.ones((1, n, 1))
        _, sf = orc.gdn_fwd(q, keys, vals, one, one, None)
        got = sf[0, 0] @ keys[0, :, 0].T                 # [Dv, n]
        np.testing.assert_allclose(got.T, vals[0, :, 0], rtol=0, atol=1e-12)


def pin_e_gdn2_collapse(orc):
    """GDN-2 with alpha = a 1, b = w = beta 1 is the scalar gated rule."""
    q, k, v, a, b, S0 = rand_gdn(14, T=15, Dk=7, Dv=4)
    Dk, Dv = 7, 4
    o1, s1 = orc.gdn_fwd(q, k, v, a, b, S0)
    o2, s2 = orc.gdn2_fwd(q, k, v, np.repeat(a[..., None], Dk, -1),
                          np.repeat(b[..., None], Dk, -1),
                          np.repeat(b[..., None], Dv, -1), S0)
    np.testing.assert_allclose(o2, o1, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(s2, s1, rtol=1e-13, atol=1e-13)


def pin_f_first_token(orc):
    """T = 1: S_1 = alpha S_0 (I - beta k k^T) + beta v k^T as numpy matrix
    products; with S_0 = 0, o_1 = beta (k . q) v."""
    q, k, v, a, b, S0 = rand_gdn(15, T=1, Dk=5, Dv=3)
    o, sf = orc.gdn_fwd(q, k, v, a, b, S0)
    for h in range(q.shape[2]):
        kk = k[0, 0, h]
        M = a[0, 0, h] * (np.eye(5) - b[0, 0, h] * np.outer(kk, kk))
        S1 = S0[0, h] @ M + b[0, 0, h] * np.outer(v[0, 0, h], kk)
        np.testing.assert_allclose(sf[0, h], S1, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(o[0, 0, h], S1 @ q[0, 0, h], rtol=1e-13,
                                   atol=1e-13)
    o, _ = orc.gdn_fwd(q, k, v, a, b, None)
    ref = (b[0, 0, :, None] * np.sum(k[0, 0] * q[0, 0], -1)[:, None]
           * v[0, 0])
    np.testing.assert_allclose(o[0, 0], ref, rtol=1e-13, atol=1e-14)


def pin_g_read_only(orc):
    """alpha = 1, beta = 0: the state never changes and O = Q S_0^T is a
    single GEMM."""
    q, k, v, a, b, S0 = rand_gdn(16, T=9, alpha=1.0, beta=0.0)
    o, sf = orc.gdn_fwd(q, k, v, a, b, S0)
    for h in range(q.shape[2]):
        np.testing.assert_allclose(o[0, :, h], q[0, :, h] @ S0[0, h].T,
                                   rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(sf, S0)


def pin_h_split(orc):
    """Running T tokens equals running T1 then T - T1 from the handed-over
    state (the chunk-to-chunk state recurrence)."""
    q, k, v, a, b, S0 = rand_gdn(17, T=29)
    o, sf = orc.gdn_fwd(q, k, v, a, b, S0)
    T1 = 11
    oa, sa = orc.gdn_fwd(q[:, :T1], k[:, :T1], v[:, :T1], a[:, :T1],
                         b[:, :T1], S0)
    ob, sb = orc.gdn_fwd(q[:, T1:], k[:, T1:], v[:, T1:], a[:, T1:],
                         b[:, T1:], sa)
    np.testing.assert_allclose(np.concatenate([oa, ob], 1), o, rtol=1e-13,
                               atol=1e-13)
    np.testing.assert_allclose(sb, sf, rtol=1e-13, atol=1e-13)


def pin_h_step_chain(orc):
    """T decode steps carried through the state equal one T-token forward."""
    q, k, v, a, b, S0 = rand_gdn(18, B=3, T=7, H=2)
    o, sf = orc.gdn_fwd(q, k, v, a, b, S0)
    st = np.ascontiguousarray(S0.copy())
    for t in range(q.shape[1]):
        ot = orc.gdn_step(q[:, t], k[:, t], v[:, t], a[:, t], b[:, t], st)
        np.testing.assert_allclose(ot, o[:, t], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(st, sf, rtol=1e-13, atol=1e-13)


def pin_i_sgd(orc):
    """One SGD step of L(S) = 1/2 |S k - v|^2 with learning rate beta, taken
    at the decayed state alpha S_{t-1} (review section 3.5, alpha as weight
    decay); the gradient comes from torch autograd in float64."""
    q, k, v, a, b, S0 = rand_gdn(19, T=5, H=1)
    o, sf = orc.gdn_fwd(q, k, v, a, b, S0)
    S = torch.tensor(S0[0, 0])
    for t in range(5):
        Sp = (float(a[0, t, 0]) * S).detach().requires_grad_(True)
        kt = torch.tensor(k[0, t, 0])
        vt = torch.tensor(v[0, t, 0])
        loss = 0.5 * torch.sum((Sp @ kt - vt) ** 2)
        (grad,) = torch.autograd.grad(loss, Sp)
        S = (Sp - float(b[0, t, 0]) * grad).detach()
        np.testing.assert_allclose(o[0, t, 0], (S @ torch.tensor(
            q[0, t, 0])).numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(sf[0, 0], S.numpy(), rtol=1e-12, atol=1e-12)


def pin_j_contraction(orc):
    """|k| = 1, beta in [0,1], alpha <= 1: |I - beta k k^T|_2 = 1, so
    |S_t|_2 <= alpha |S_{t-1}|_2 + beta |v| along a long run."""
    q, k, v, a, b, S0 = rand_gdn(20, T=64, H=1, Dk=8, Dv=8)
    prev = np.linalg.norm(S0[0, 0], 2)
    for t in range(64):
        _, st = orc.gdn_fwd(q[:, :t + 1], k[:, :t + 1], v[:, :t + 1],
                            a[:, :t + 1], b[:, :t + 1], S0)
        cur = np.linalg.norm(st[0, 0], 2)
        bound = a[0, t, 0] * prev + b[0, t, 0] * np.linalg.norm(v[0, t, 0])
        assert cur <= bound * (1 + 1e-12), (t, cur, bound)
        prev = cur


def pin_k_kda(orc):
    """b = w = beta 1 with per-channel alpha: the KDA loop
    S <- S diag(a) + beta (v - S diag(a) k) k^T, written independently."""
    q, k, v, a, e, w, S0 = rand_gdn2(21, T=9)
    beta = _rng(5).uniform(0, 1, q.shape[:3])
    Dk, Dv = q.shape[-1], v.shape[-1]
    o, sf = orc.gdn2_fwd(q, k, v, a, np.repeat(beta[..., None], Dk, -1),
                         np.repeat(beta[..., None], Dv, -1), S0)
    for h in range(q.shape[2]):
        S = S0[0, h].copy()
        for t in range(q.shape[1]):
            Sd = S * a[0, t, h][None, :]
            kt = k[0, t, h]
            S = Sd + beta[0, t, h] * np.outer(v[0, t, h] - Sd @ kt, kt)
            np.testing.assert_allclose(o[0, t, h], S @ q[0, t, h],
                                       rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(sf[0, h], S, rtol=1e-12, atol=1e-12)


def pin_gdn2_pure_decay(orc):
    """GDN-2 with b = w = 0: S_t = S_0 diag(prod alpha) per channel, so
    o_t = S_0 (lambda_t . q_t) with lambda taken in log space."""
    q, k, v, a, e, w, S0 = rand_gdn2(22, T=30)
    o, sf = orc.gdn2_fwd(q, k, v, a, np.zeros_like(e), np.zeros_like(w), S0)
    lam = np.exp(np.cumsum(np.log(a), axis=1))           # [B,T,H,Dk]
    ref_o = np.einsum("bhij,bthj->bthi", S0, lam * q)
    np.testing.assert_allclose(o, ref_o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(sf, S0 * lam[:, -1][:, :, None, :],
                               rtol=1e-12, atol=1e-13)


def pin_gdn2_write_only(orc):
    """GDN-2 with alpha = 1 and b = 0: nothing is erased, so
    S_t = S_0 + sum_{s<=t} (w_s . v_s) k_s^T (linear attention, review 3.1)."""
    q, k, v, a, e, w, S0 = rand_gdn2(23, T=11)
    o, sf = orc.gdn2_fwd(q, k, v, np.ones_like(a), np.zeros_like(e), w, S0)
    cum = np.cumsum(np.einsum("bthi,bthj->bthij", w * v, k), axis=1)
    St = S0[:, None] + cum                               # [B,T,H,Dv,Dk]
    np.testing.assert_allclose(o, np.einsum("bthij,bthj->bthi", St, q),
                               rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(sf, St[:, -1], rtol=1e-12, atol=1e-12)


def pin_gdn2_erase_axis(orc):
    """The erase gate acts on the key axis only: with per-channel alpha = 1,
    w = 1, a unit key k = e_j and b_j = 1, column j of S becomes v (the old
    value is fully replaced) and the other columns are untouched."""
    g = _rng(24)
    Dk, Dv = 5, 4
    S0 = g.standard_normal((1, 1, Dv, Dk))
    for j in range(Dk):
        k = np.zeros((1, 1, 1, Dk)); k[..., j] = 1.0
        e = g.uniform(0, 1, (1, 1, 1, Dk)); e[..., j] = 1.0
        v = g.standard_normal((1, 1, 1, Dv))
        q = g.standard_normal((1, 1, 1, Dk))
        _, sf = orc.gdn2_fwd(q, k, v, np.ones((1, 1, 1, Dk)), e,
                             np.ones((1, 1, 1, Dv)), S0)
        ref = S0[0, 0].copy(); ref[:, j] = v[0, 0, 0]
        np.testing.assert_allclose(sf[0, 0], ref, rtol=0, atol=1e-15)


def pin_gdn2_householder(orc):
    """Negative eigenvalue range: per-channel alpha = 1, erase b = 2 on every
    channel, w = 0 and unit keys make each step S <- S (I - 2 k k^T), a
    reflection.  The Frobenius norm of S is kept at every step, and the same
    key twice in a row gives back the state it started from."""
    g = _rng(25)
    T, Dk, Dv = 12, 6, 5
    k = _unit(g.standard_normal((1, T, 1, Dk)))
    k[0, 7] = k[0, 6]                                    # tokens 6 and 7 repeat
    q = g.standard_normal((1, T, 1, Dk))
    v = g.standard_normal((1, T, 1, Dv))
    S0 = g.standard_normal((1, 1, Dv, Dk))
    ones, twos = np.ones((1, T, 1, Dk)), np.full((1, T, 1, Dk), 2.0)
    n0 = np.linalg.norm(S0[0, 0])
    states = []
    for t in range(T):
        _, st = orc.gdn2_fwd(q[:, :t + 1], k[:, :t + 1], v[:, :t + 1], ones[:, :t + 1],
                             twos[:, :t + 1], np.zeros((1, t + 1, 1, Dv)), S0)
        states.append(st[0, 0])
        assert abs(np.linalg.norm(st[0, 0]) - n0) <= 1e-12 * n0, t
    np.testing.assert_allclose(states[7], states[5], rtol=0, atol=1e-12)


def pin_gdn_negative_beta(orc):
    """Scalar rule with beta = 2, alpha = 1, v = 0 and unit keys: each step is
    the reflection S (I - 2 k k^T), so |S|_F is kept and a repeated key undoes
    itself; with v != 0 the step adds 2 v k^T after the reflection."""
    g = _rng(26)
    T, Dk, Dv = 10, 6, 4
    k = _unit(g.standard_normal((1, T, 1, Dk)))
    k[0, 4] = k[0, 3]
    q = g.standard_normal((1, T, 1, Dk))
    S0 = g.standard_normal((1, 1, Dv, Dk))
    a, b = np.ones((1, T, 1)), np.full((1, T, 1), 2.0)
    n0 = np.linalg.norm(S0[0, 0])
    _, s3 = orc.gdn_fwd(q[:, :3], k[:, :3], np.zeros((1, 3, 1, Dv)), a[:, :3], b[:, :3], S0)
    _, s5 = orc.gdn_fwd(q[:, :5], k[:, :5], np.zeros((1, 5, 1, Dv)), a[:, :5], b[:, :5], S0)
    _, sT = orc.gdn_fwd(q, k, np.zeros((1, T, 1, Dv)), a, b, S0)
    assert abs(np.linalg.norm(sT[0, 0]) - n0) <= 1e-12 * n0
    np.testing.assert_allclose(s5[0, 0], s3[0, 0], rtol=0, atol=1e-12)
    v = g.standard_normal((1, 1, 1, Dv))
    _, s1 = orc.gdn_fwd(q[:, :1], k[:, :1], v, a[:, :1], b[:, :1], S0)
    kk = k[0, 0, 0]
    ref = S0[0, 0] @ (np.eye(Dk) - 2 * np.outer(kk, kk)) + 2 * np.outer(v[0, 0, 0], kk)
    np.testing.assert_allclose(s1[0, 0], ref, rtol=0, atol=1e-12)


# --- reverse mode of the scalar-gate rule ------------------------------------
def _gdn_loss(orc, q, k, v, a, b, S0, do, dsf):
    o, sf = orc.gdn_fwd(q, k, v, a, b, S0)
    return float(np.sum(o * do) + np.sum(sf * dsf))


def pin_bwd_finite_differences(orc):
    """Every gradient of L = sum(o * dout) + sum(S_T * dS_T) against central
    differences of the forward oracle, element by element on a tiny case
    (T = 6, H = 2, d_k = 4, d_v = 3, with S_0); step 1e-5, so the error is
    ~1e-10 of the gradient scale."""
    q, k, v, a, b, S0 = rand_gdn(30, B=1, T=6, H=2, Dk=4, Dv=3)
    g = _rng(31)
    do = g.standard_normal((1, 6, 2, 3))
    dsf = g.standard_normal((1, 2, 3, 4))
    grads = orc.gdn_bwd(q, k, v, a, b, S0, do, dsf)
    args = [q, k, v, a, b, S0]
    h = 1e-5
    for idx, x in enumerate(args):
        num = np.zeros_like(x)
        for pos in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[pos] += h
            xm[pos] -= h
            ap, am = list(args), list(args)
            ap[idx], am[idx] = xp, xm
            num[pos] = (_gdn_loss(orc, *ap, do, dsf) - _gdn_loss(orc, *am, do, dsf)) / (2 * h)
        scale = max(1.0, np.abs(num).max())
        assert np.abs(grads[idx] - num).max() <= 1e-7 * scale, (idx, np.abs(grads[idx] - num).max())


def pin_bwd_directional(orc):
    """Directional derivatives along random directions on a case that crosses
    the oracle's 64-token recompute segments (T = 150) and has no S_T
    gradient and no S_0."""
    q, k, v, a, b, _ = rand_gdn(32, B=2, T=150, H=1, Dk=5, Dv=4, s0=False)
    g = _rng(33)
    do = g.standard_normal(v.shape)
    zs = np.zeros((2, 1, 4, 5))
    dq, dk, dv, da, db, ds0 = orc.gdn_bwd(q, k, v, a, b, None, do, None)
    S0 = np.zeros((2, 1, 4, 5))
    for d in range(3):
        dirs = [g.standard_normal(x.shape) for x in (q, k, v, a, b, S0)]
        h = 1e-5
        xp = [x + h * e for x, e in zip((q, k, v, a, b, S0), dirs)]
        xm = [x - h * e for x, e in zip((q, k, v, a, b, S0), dirs)]
        num = (_gdn_loss(orc, *xp, do, zs) - _gdn_loss(orc, *xm, do, zs)) / (2 * h)
        ana = sum(float(np.sum(gr * e)) for gr, e in zip((dq, dk, dv, da, db, ds0), dirs))
        assert abs(num - ana) <= 1e-7 * max(1.0, abs(ana)), (d, num, ana)


def pin_bwd_autograd_matrix_form(orc):
    """The gradients equal autograd's through the literal matrix form
    S_t = alpha S_{t-1} (I - beta k k^T) + beta v k^T, o_t = S_t q_t in
    torch fp64 (a different formulation from the oracle's row loops)."""
    q, k, v, a, b, S0 = rand_gdn(34, B=1, T=20, H=2, Dk=6, Dv=5)
    g = _rng(35)
    do = g.standard_normal(v.shape)
    dsf = g.standard_normal(S0.shape)
    t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, a, b, S0)]
    tq, tk, tv, ta, tb, tS = t
    loss = 0.0
    for h in range(2):
        S = tS[0, h]
        for s in range(20):
            kk = tk[0, s, h]
            S = ta[0, s, h] * S @ (torch.eye(6, dtype=torch.float64) - tb[0, s, h] * torch.outer(kk, kk)) \
                + tb[0, s, h] * torch.outer(tv[0, s, h], kk)
            loss = loss + (S @ tq[0, s, h] * torch.tensor(do[0, s, h])).sum()
        loss = loss + (S * torch.tensor(dsf[0, h])).sum()
    loss.backward()
    grads = orc.gdn_bwd(q, k, v, a, b, S0, do, dsf)
    for x, gr in zip(t, grads):
        np.testing.assert_allclose(gr, x.grad.numpy(), rtol=1e-10, atol=1e-12)


# --- reverse mode of Gated Delta Rule-2 -------------------------------------
def _gdn2_loss(orc, q, k, v, a, e, w, S0, do, dsf):
    o, sf = orc.gdn2_fwd(q, k, v, a, e, w, S0)
    return float(np.sum(o * do) + np.sum(sf * dsf))


def pin_bwd2_finite_differences(orc):
    """Every GDN-2 gradient against central differences of the forward
    oracle, element by element (T = 5, H = 1, d_k = 4, d_v = 3, with S_0 and
    dS_T)."""
    q, k, v, a, e, w, S0 = rand_gdn2(40, B=1, T=5, H=1, Dk=4, Dv=3)
    g = _rng(41)
    do = g.standard_normal(v.shape)
    dsf = g.standard_normal(S0.shape)
    grads = orc.gdn2_bwd(q, k, v, a, e, w, S0, do, dsf)
    args = [q, k, v, a, e, w, S0]
    h = 1e-5
    for idx, x in enumerate(args):
        num = np.zeros_like(x)
        for pos in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[pos] += h
            xm[pos] -= h
            ap, am = list(args), list(args)
            ap[idx], am[idx] = xp, xm
            num[pos] = (_gdn2_loss(orc, *ap, do, dsf) - _gdn2_loss(orc, *am, do, dsf)) / (2 * h)
        scale = max(1.0, np.abs(num).max())
        assert np.abs(grads[idx] - num).max() <= 1e-7 * scale, (idx, np.abs(grads[idx] - num).max())


def pin_bwd2_autograd_matrix_form(orc):
    """GDN-2 gradients equal autograd's through the literal matrix form
    S' = S diag(alpha), S_t = S' + (w (.) v - S'(b (.) k)) k^T, o = S_t q in
    torch fp64, on a case that crosses the oracle's 64-token segments."""
    q, k, v, a, e, w, S0 = rand_gdn2(42, B=1, T=70, H=1, Dk=5, Dv=4)
    g = _rng(43)
    do = g.standard_normal(v.shape)
    dsf = g.standard_normal(S0.shape)
    t = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v, a, e, w, S0)]
    tq, tk, tv, ta, te, tw, tS = t
    S = tS[0, 0]
    loss = 0.0
    for s in range(70):
        Sp = S @ torch.diag(ta[0, s, 0])
        S = Sp + torch.outer(tw[0, s, 0] * tv[0, s, 0] - Sp @ (te[0, s, 0] * tk[0, s, 0]), tk[0, s, 0])
        loss = loss + (S @ tq[0, s, 0] * torch.tensor(do[0, s, 0])).sum()
    loss = loss + (S * torch.tensor(dsf[0, 0])).sum()
    loss.backward()
    grads = orc.gdn2_bwd(q, k, v, a, e, w, S0, do, dsf)
    for x, gr in zip(t, grads):
        np.testing.assert_allclose(gr, x.grad.numpy(), rtol=1e-9, atol=1e-11)


# --- the block's L2 normalisation of q and k --------------------------------
def pin_l2norm_worked(orc):
    """Worked rows with eps = 0: (3, 4) -> (0.6, 0.8); (1, 1, 1, 1) ->
    (0.5, 0.5, 0.5, 0.5); (0, -2, 0) -> (0, -1, 0).  A zero row stays zero
    under eps > 0."""
    x = np.array([[3.0, 4.0, 0.0, 0.0], [1.0, 1.0, 1.0, 1.0], [0.0, -2.0, 0.0, 0.0]])
    ref = np.array([[0.6, 0.8, 0.0, 0.0], [0.5, 0.5, 0.5, 0.5], [0.0, -1.0, 0.0, 0.0]])
    np.testing.assert_allclose(orc.l2norm(x, eps=0.0), ref, rtol=0, atol=1e-15)
    np.testing.assert_array_equal(orc.l2norm(np.zeros((2, 5)), eps=1e-6), np.zeros((2, 5)))


def pin_l2norm_eps(orc):
    """eps sits inside the square root: a row of norm r becomes norm
    r / sqrt(r^2 + eps).  At r^2 = eps that is 1 / sqrt(2)."""
    for r in (1e-3, 0.37, 5.0):
        x = np.array([[r, 0.0, 0.0]])
        out = orc.l2norm(x, eps=1e-6)
        np.testing.assert_allclose(out[0, 0], r / np.sqrt(r * r + 1e-6), rtol=1e-15)
    np.testing.assert_allclose(orc.l2norm(np.array([[0.0, 1e-3]]), eps=1e-6)[0, 1],
                               1.0 / np.sqrt(2.0), rtol=1e-14)


def pin_l2norm_rows(orc):
    """Each row (last axis) on its own: with eps = 0 every row of a random
    [3, 4, 7] array of mixed scales has norm 1 and points along its input
    (out * |x| = x)."""
    g = _rng(27)
    x = g.standard_normal((3, 4, 7)) * g.uniform(0.01, 100.0, (3, 4, 1))
    out = orc.l2norm(x, eps=0.0)
    nrm = np.linalg.norm(x, axis=-1, keepdims=True)
    np.testing.assert_allclose(np.linalg.norm(out, axis=-1), 1.0, rtol=0, atol=1e-14)
    np.testing.assert_allclose(out * nrm, x, rtol=1e-13, atol=0)


def pin_l2norm_bwd_finite_differences(orc):
    """The reverse mode of the norm against central differences of
    l2norm itself, for eps = 1e-6 and 0.3 (eps enters the Jacobian)."""
    g = _rng(30)
    x = g.standard_normal((3, 5)) * g.uniform(0.1, 3.0, (3, 1))
    dy = g.standard_normal((3, 5))
    for eps in (1e-6, 0.3):
        dx = orc.l2norm_bwd(x, dy, eps=eps)
        h = 1e-6
        fd = np.zeros_like(x)
        for r in range(3):
            for c in range(5):
                xp, xm = x.copy(), x.copy()
                xp[r, c] += h
                xm[r, c] -= h
                fd[r, c] = np.sum(dy * (orc.l2norm(xp, eps=eps) - orc.l2norm(xm, eps=eps))) / (2 * h)
        np.testing.assert_allclose(dx, fd, rtol=1e-6, atol=1e-8)


def pin_l2norm_bwd_radial(orc):
    """Closed form along the row: x . dx = eps (x . dy) / n^3 with
    n = sqrt(|x|^2 + eps) (zero when eps = 0: the map ignores the length)."""
    g = _rng(31)
    x = g.standard_normal((4, 6))
    dy = g.standard_normal((4, 6))
    for eps in (0.0, 0.7):
        dx = orc.l2norm_bwd(x, dy, eps=eps)
        n = np.sqrt(np.sum(x * x, axis=-1) + eps)
        np.testing.assert_allclose(np.sum(x * dx, axis=-1), eps * np.sum(x * dy, axis=-1) / n ** 3,
                                   rtol=1e-12, atol=1e-14)


# --- the block's output gate -------------------------------------------------
def _silu(x):
    return x / (1.0 + np.exp(-x))


def pin_gate_worked(orc):
    """Worked row, eps = 0, w = 1: o = (3, 4) has mean square 12.5, so the
    normalised row is (3, 4) / sqrt(12.5); g = (0, 30) gates it by
    SiLU(0) = 0 and SiLU(30) = 30 / (1 + e^-30).  A gate of ln 3 gives
    SiLU = ln 3 * 3/4 exactly in closed form."""
    y = orc.rmsnorm_gate(np.array([[3.0, 4.0]]), np.array([[0.0, 30.0]]), eps=0.0)
    ref = np.array([[0.0, 4.0 / np.sqrt(12.5) * 30.0 / (1.0 + np.exp(-30.0))]])
    np.testing.assert_allclose(y, ref, rtol=1e-15, atol=0)
    y = orc.rmsnorm_gate(np.array([[2.0, 2.0, 2.0]]), np.full((1, 3), np.log(3.0)), eps=0.0)
    np.testing.assert_allclose(y, np.full((1, 3), np.log(3.0) * 0.75), rtol=1e-15)


def pin_gate_rms_and_eps(orc):
    """With a gate that makes SiLU = 1 and w = 1, every row comes out with
    mean square r^2 / (r^2 + eps) for an input of mean square r^2 (eps inside
    the root, mean over the row, rows independent)."""
    g0 = 1.2784645427610738                     # SiLU(g0) = 1
    assert abs(_silu(g0) - 1.0) < 1e-15
    rng = _rng(28)
    o = rng.standard_normal((5, 7)) * rng.uniform(0.001, 10.0, (5, 1))
    for eps in (0.0, 1e-6, 1e-2):
        y = orc.rmsnorm_gate(o, np.full_like(o, g0), eps=eps)
        r2 = np.mean(o * o, axis=-1)
        np.testing.assert_allclose(np.mean(y * y, axis=-1), r2 / (r2 + eps), rtol=1e-13)
        np.testing.assert_allclose(y * np.sqrt(r2 + eps)[:, None], o, rtol=1e-13)


def pin_gate_weight_axis(orc):
    """The weight scales channels (the last axis), the same for every row;
    the gate acts elementwise."""
    rng = _rng(29)
    o = rng.standard_normal((4, 6))
    g = rng.standard_normal((4, 6))
    w = rng.uniform(0.5, 2.0, 6)
    y1 = orc.rmsnorm_gate(o, g, None, eps=1e-6)
    y2 = orc.rmsnorm_gate(o, g, w, eps=1e-6)
    np.testing.assert_allclose(y2, y1 * w[None, :], rtol=1e-14)
    g2 = g.copy(); g2[1, 3] = -g2[1, 3]
    y3 = orc.rmsnorm_gate(o, g2, w, eps=1e-6)
    mask = np.ones_like(o, dtype=bool); mask[1, 3] = False
    np.testing.assert_array_equal(y3[mask], y2[mask])
    np.testing.assert_allclose(y3[1, 3] / y2[1, 3], _silu(g2[1, 3]) / _silu(g[1, 3]), rtol=1e-13)


def pin_gate_bwd_finite_differences(orc):
    """The output gate's reverse mode against central differences of the
    forward in o, g and w, with eps = 1e-6 and 0.5 (eps enters the root)."""
    rng = _rng(32)
    o = rng.standard_normal((3, 5))
    g = rng.standard_normal((3, 5)) * 2.0
    w = rng.uniform(0.5, 1.5, 5)
    dy = rng.standard_normal((3, 5))
    h = 1e-6
    for eps in (1e-6, 0.5):
        do, dg, dw = orc.rmsnorm_gate_bwd(o, g, w, dy, eps=eps)
        f = lambda oo, gg, ww: np.sum(dy * orc.rmsnorm_gate(oo, gg, ww, eps=eps))
        for x, grad, which in ((o, do, 0), (g, dg, 1)):
            fd = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = [o, g, w]
                args_m = [o, g, w]
                args_p[which], args_m[which] = xp, xm
                fd[idx] = (f(*args_p) - f(*args_m)) / (2 * h)
            np.testing.assert_allclose(grad, fd, rtol=1e-6, atol=1e-8)
        fdw = np.zeros_like(w)
        for c in range(5):
            wp, wm = w.copy(), w.copy()
            wp[c] += h
            wm[c] -= h
            fdw[c] = (f(o, g, wp) - f(o, g, wm)) / (2 * h)
        np.testing.assert_allclose(dw, fdw, rtol=1e-6, atol=1e-8)
    _, _, dw_none = orc.rmsnorm_gate_bwd(o, g, None, dy)
    assert dw_none is None


def pin_gate_bwd_scale_invariance(orc):
    """With eps = 0 the normalised row ignores the row's scale, so do is
    orthogonal to o in every row; and do scales as 1 / c when o is scaled
    by c."""
    rng = _rng(33)
    o = rng.standard_normal((4, 6))
    g = rng.standard_normal((4, 6))
    dy = rng.standard_normal((4, 6))
    do, _, _ = orc.rmsnorm_gate_bwd(o, g, None, dy, eps=0.0)
    np.testing.assert_allclose(np.sum(o * do, axis=-1), 0.0, atol=1e-13)
    do3, _, _ = orc.rmsnorm_gate_bwd(3.0 * o, g, None, dy, eps=0.0)
    np.testing.assert_allclose(do3, do / 3.0, rtol=1e-12, atol=1e-15)


ALL_PINS = [
    pin_golden_gdn, pin_golden_step, pin_golden_gdn2,
    pin_exact_matrix_form_gdn, pin_exact_matrix_form_gdn2,
    pin_a_deltanet, pin_b_pure_decay, pin_c_unit_key_write,
    pin_d_orthonormal_retrieval, pin_e_gdn2_collapse, pin_f_first_token,
    pin_g_read_only, pin_h_split, pin_h_step_chain, pin_i_sgd,
    pin_j_contraction, pin_k_kda, pin_gdn2_pure_decay, pin_gdn2_write_only,
    pin_gdn2_erase_axis, pin_gdn2_householder, pin_gdn_negative_beta,
    pin_l2norm_worked, pin_l2norm_eps, pin_l2norm_rows,
    pin_l2norm_bwd_finite_differences, pin_l2norm_bwd_radial,
    pin_gate_worked, pin_gate_rms_and_eps, pin_gate_weight_axis,
    pin_gate_bwd_finite_differences, pin_gate_bwd_scale_invariance,
    pin_bwd_finite_differences, pin_bwd_directional, pin_bwd_autograd_matrix_form,
    pin_bwd2_finite_differences, pin_bwd2_autograd_matrix_form,
]
