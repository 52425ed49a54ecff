"""fp64 CPU oracle for the gated delta rule kernels — TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never calls it, and the oracle shares no code with it.

The arithmetic lives in ``gdr_oracle.c`` (plain C, double precision, one
token at a time); this module only compiles it with gcc, loads it with
ctypes, and converts inputs to contiguous float64 arrays.  Each wrapped
function cites the passage it follows in the C source.

Functions
---------
gdn_fwd(q, k, v, alpha, beta, s0=None) -> (o, s_final)
    Gated delta rule S_t = S_{t-1} alpha_t (I - beta_t k_t k_t^T)
    + beta_t v_t k_t^T, o_t = S_t q_t.
gdn_step(q, k, v, alpha, beta, state) -> o   (state updated in place)
    One decode token for N independent sequences.
gdn2_fwd(q, k, v, alpha, erase, write, s0=None) -> (o, s_final)
    Gated Delta Rule-2: decay S by diag(alpha_t), read along erase (.) k,
    write (write (.) v - read) along k.
l2norm(x, eps=1e-6) -> x / sqrt(sum over the last axis of x^2 + eps)
    The block's L2 normalisation of q and k, applied before either rule.
gdn_bwd(q, k, v, alpha, beta, s0, dout, ds_final=None)
    -> (dq, dk, dv, dalpha, dbeta, ds0), the reverse mode of gdn_fwd.
gdn2_bwd(q, k, v, alpha, erase, write, s0, dout, ds_final=None)
    -> (dq, dk, dv, dalpha, derase, dwrite, ds0), the reverse mode of gdn2_fwd.
rmsnorm_gate(o, g, w=None, eps=1e-6) -> y
    The block's output gate: RMSNorm of o over its last axis (weight w),
    times SiLU(g).

Parity pins: every function is pinned by tests/test_oracle.py against
closed forms, invariants, exact rational worked examples
(tests/golden/) and independent formulations; none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdr_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

__all__ = ["build", "OracleLib", "default", "gdn_fwd", "gdn_step",
           "gdn2_fwd", "gdn_bwd", "gdn2_bwd", "l2norm", "rmsnorm_gate", "num_threads", "set_num_threads", "err_rms"]


def build(force: bool = True, src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle with gcc (portable x86-64, OpenMP, no fast-math)."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp"
        subprocess.check_call(["gcc", "-O3", "-fopenmp", "-fPIC", "-shared",
                               "-std=c11", "-Wall", "-o", tmp, src, "-lm"])
        os.replace(tmp, out)
    return out


def _f64(x) -> np.ndarray:
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor (CPU): exact widening to fp64
        x = x.detach().cpu().double().numpy()
    return np.ascontiguousarray(x, dtype=np.float64)


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class OracleLib:
    """ctypes view of one compiled oracle library (the default one, or a
    deliberately broken copy built by the mutation tests)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        L, P = ctypes.c_long, ctypes.c_void_p
        lib.oracle_gdn_fwd.argtypes = [L] * 5 + [P] * 8
        lib.oracle_gdn_fwd.restype = ctypes.c_int
        lib.oracle_gdn_step.argtypes = [L] * 4 + [P] * 7
        lib.oracle_gdn_step.restype = ctypes.c_int
        lib.oracle_gdn2_fwd.argtypes = [L] * 5 + [P] * 9
        lib.oracle_gdn2_fwd.restype = ctypes.c_int
        lib.oracle_gdn_bwd.argtypes = [L] * 5 + [P] * 14
        lib.oracle_gdn_bwd.restype = ctypes.c_int
        lib.oracle_gdn2_bwd.argtypes = [L] * 5 + [P] * 16
        lib.oracle_gdn2_bwd.restype = ctypes.c_int
        lib.oracle_l2norm_rows.argtypes = [L, L, P, ctypes.c_double, P]
        lib.oracle_l2norm_rows.restype = ctypes.c_int
        lib.oracle_l2norm_rows_bwd.argtypes = [L, L, P, P, ctypes.c_double, P]
        lib.oracle_l2norm_rows_bwd.restype = ctypes.c_int
        lib.oracle_rmsnorm_gate_rows_bwd.argtypes = [L, L, P, P, P, ctypes.c_double, P, P, P, P]
        lib.oracle_rmsnorm_gate_rows_bwd.restype = ctypes.c_int
        lib.oracle_rmsnorm_gate_rows.argtypes = [L, L, P, P, P, ctypes.c_double, P]
        lib.oracle_rmsnorm_gate_rows.restype = ctypes.c_int
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        self.lib = lib

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    def set_num_threads(self, n: int) -> None:
        self.lib.oracle_set_num_threads(int(n))

    def gdn_fwd(self, q, k, v, alpha, beta, s0=None, want_state=True):
        """Gated delta rule forward (``oracle_gdn_fwd`` in gdr_oracle.c).

        q, k [B,T,H,Dk]; v [B,T,H,Dv]; alpha, beta [B,T,H]; s0 [B,H,Dv,Dk]
        or None (zero state).  Returns o [B,T,H,Dv] and s_final [B,H,Dv,Dk]
        (or None), both float64.
        """
        q, k, v, a, b, s0 = map(_f64, (q, k, v, alpha, beta, s0))
        B, T, H, Dk = q.shape
        Dv = v.shape[-1]
        assert k.shape == q.shape and v.shape == (B, T, H, Dv)
        assert a.shape == (B, T, H) and b.shape == (B, T, H)
        assert s0 is None or s0.shape == (B, H, Dv, Dk)
        o = np.empty((B, T, H, Dv))
        sf = np.empty((B, H, Dv, Dk)) if want_state else None
        rc = self.lib.oracle_gdn_fwd(B, T, H, Dk, Dv, _p(q), _p(k), _p(v),
                                     _p(a), _p(b), _p(s0), _p(o), _p(sf))
        if rc:
            raise RuntimeError(f"oracle_gdn_fwd failed ({rc})")
        return o, sf

    def gdn_step(self, q, k, v, alpha, beta, state):
        """One decode token (``oracle_gdn_step``).  ``state`` is a float64
        numpy array [N,H,Dv,Dk], updated in place.  Returns o [N,H,Dv]."""
        q, k, v, a, b = map(_f64, (q, k, v, alpha, beta))
        assert isinstance(state, np.ndarray) and state.dtype == np.float64
        assert state.flags["C_CONTIGUOUS"]
        N, H, Dk = q.shape
        Dv = v.shape[-1]
        assert state.shape == (N, H, Dv, Dk) and a.shape == (N, H)
        o = np.empty((N, H, Dv))
        rc = self.lib.oracle_gdn_step(N, H, Dk, Dv, _p(q), _p(k), _p(v),
                                      _p(a), _p(b), _p(state), _p(o))
        if rc:
            raise RuntimeError(f"oracle_gdn_step failed ({rc})")
        return o

    def gdn2_fwd(self, q, k, v, alpha, erase, write, s0=None,
                 want_state=True):
        """Gated Delta Rule-2 forward (``oracle_gdn2_fwd``).

        q, k, alpha, erase [B,T,H,Dk]; v, write [B,T,H,Dv]; s0 [B,H,Dv,Dk]
        or None.  Returns o [B,T,H,Dv] and s_final, float64.
        """
        q, k, v, a, e, w, s0 = map(_f64, (q, k, v, alpha, erase, write, s0))
        B, T, H, Dk = q.shape
        Dv = v.shape[-1]
        assert k.shape == q.shape and a.shape == q.shape
        assert e.shape == q.shape
        assert v.shape == (B, T, H, Dv) and w.shape == v.shape
        assert s0 is None or s0.shape == (B, H, Dv, Dk)
        o = np.empty((B, T, H, Dv))
        sf = np.empty((B, H, Dv, Dk)) if want_state else None
        rc = self.lib.oracle_gdn2_fwd(B, T, H, Dk, Dv, _p(q), _p(k), _p(v),
                                      _p(a), _p(e), _p(w), _p(s0), _p(o),
                                      _p(sf))
        if rc:
            raise RuntimeError(f"oracle_gdn2_fwd failed ({rc})")
        return o, sf

    def gdn_bwd(self, q, k, v, alpha, beta, s0, dout, ds_final=None):
        """Reverse mode of the gated delta rule (``oracle_gdn_bwd``): the
        gradients of sum(o * dout) + sum(S_T * ds_final) with respect to q,
        k, v, alpha, beta and s0.  Returns float64 (dq, dk, dv, dalpha,
        dbeta, ds0); s0 None means a zero initial state (ds0 still
        returned)."""
        q, k, v, a, b, s0, do, dsf = map(_f64, (q, k, v, alpha, beta, s0, dout, ds_final))
        B, T, H, Dk = q.shape
        Dv = v.shape[-1]
        assert k.shape == q.shape and v.shape == (B, T, H, Dv) and do.shape == v.shape
        assert a.shape == (B, T, H) and b.shape == (B, T, H)
        assert s0 is None or s0.shape == (B, H, Dv, Dk)
        assert dsf is None or dsf.shape == (B, H, Dv, Dk)
        dq, dk = np.empty_like(q), np.empty_like(k)
        dv = np.empty_like(v)
        da, db = np.empty_like(a), np.empty_like(b)
        ds0 = np.empty((B, H, Dv, Dk))
        rc = self.lib.oracle_gdn_bwd(B, T, H, Dk, Dv, _p(q), _p(k), _p(v), _p(a), _p(b),
                                     _p(s0), _p(do), _p(dsf), _p(dq), _p(dk), _p(dv),
                                     _p(da), _p(db), _p(ds0))
        if rc:
            raise RuntimeError(f"oracle_gdn_bwd failed ({rc})")
        return dq, dk, dv, da, db, ds0

    def gdn2_bwd(self, q, k, v, alpha, erase, write, s0, dout, ds_final=None):
        """Reverse mode of Gated Delta Rule-2 (``oracle_gdn2_bwd``): gradients of
        sum(o * dout) + sum(S_T * ds_final).  Returns float64 (dq, dk, dv,
        dalpha, derase, dwrite, ds0)."""
        q, k, v, a, e, w, s0, do, dsf = map(_f64, (q, k, v, alpha, erase, write, s0, dout,
                                                   ds_final))
        B, T, H, Dk = q.shape
        Dv = v.shape[-1]
        assert k.shape == q.shape and a.shape == q.shape and e.shape == q.shape
        assert v.shape == (B, T, H, Dv) and w.shape == v.shape and do.shape == v.shape
        assert s0 is None or s0.shape == (B, H, Dv, Dk)
        assert dsf is None or dsf.shape == (B, H, Dv, Dk)
        out = [np.empty_like(q), np.empty_like(k), np.empty_like(v), np.empty_like(a),
               np.empty_like(e), np.empty_like(w), np.empty((B, H, Dv, Dk))]
        rc = self.lib.oracle_gdn2_bwd(B, T, H, Dk, Dv, _p(q), _p(k), _p(v), _p(a), _p(e), _p(w),
                                      _p(s0), _p(do), _p(dsf), *[_p(x) for x in out])
        if rc:
            raise RuntimeError(f"oracle_gdn2_bwd failed ({rc})")
        return tuple(out)

    def l2norm(self, x, eps=1e-6):
        """Rows of x (last axis) scaled to unit L2 norm,
        x / sqrt(sum x^2 + eps) (``oracle_l2norm_rows``).  float64."""
        x = _f64(x)
        d = x.shape[-1] if x.ndim else 1
        n = x.size // d if d else 0
        out = np.empty_like(x)
        rc = self.lib.oracle_l2norm_rows(n, d, _p(x), float(eps), _p(out))
        if rc:
            raise RuntimeError(f"oracle_l2norm_rows failed ({rc})")
        return out

    def l2norm_bwd(self, x, dy, eps=1e-6):
        """Gradient with respect to the raw rows x of a loss whose gradient
        with respect to l2norm(x) is dy (``oracle_l2norm_rows_bwd``).  float64."""
        x, dy = _f64(x), _f64(dy)
        assert x.shape == dy.shape
        d = x.shape[-1] if x.ndim else 1
        n = x.size // d if d else 0
        out = np.empty_like(x)
        rc = self.lib.oracle_l2norm_rows_bwd(n, d, _p(x), _p(dy), float(eps), _p(out))
        if rc:
            raise RuntimeError(f"oracle_l2norm_rows_bwd failed ({rc})")
        return out

    def rmsnorm_gate(self, o, g, w=None, eps=1e-6):
        """Output gate on rows of the last axis (``oracle_rmsnorm_gate_rows``):
        o / sqrt(mean(o^2) + eps) * w * g * sigmoid(g); w of the last axis'
        length or None (ones).  float64."""
        o, g, w = _f64(o), _f64(g), _f64(w)
        assert o.shape == g.shape and o.ndim >= 1
        d = o.shape[-1]
        assert w is None or w.shape == (d,)
        y = np.empty_like(o)
        rc = self.lib.oracle_rmsnorm_gate_rows(o.size // d, d, _p(o), _p(g), _p(w),
                                               float(eps), _p(y))
        if rc:
            raise RuntimeError(f"oracle_rmsnorm_gate_rows failed ({rc})")
        return y

    def rmsnorm_gate_bwd(self, o, g, w, dy, eps=1e-6):
        """Reverse mode of rmsnorm_gate (``oracle_rmsnorm_gate_rows_bwd``):
        returns float64 (do, dg, dw), dw summed over all rows (None when w is
        None)."""
        o, g, w, dy = _f64(o), _f64(g), _f64(w), _f64(dy)
        assert o.shape == g.shape == dy.shape and o.ndim >= 1
        d = o.shape[-1]
        assert w is None or w.shape == (d,)
        do, dg = np.empty_like(o), np.empty_like(o)
        dw = None if w is None else np.empty(d)
        rc = self.lib.oracle_rmsnorm_gate_rows_bwd(o.size // d, d, _p(o), _p(g), _p(w),
                                                   float(eps), _p(dy), _p(do), _p(dg), _p(dw))
        if rc:
            raise RuntimeError(f"oracle_rmsnorm_gate_rows_bwd failed ({rc})")
        return do, dg, dw


_default = None


def default() -> OracleLib:
    global _default
    if _default is None:
        if not os.path.exists(_LIB):
            build()
        _default = OracleLib(_LIB)
    return _default


def num_threads() -> int:
    return default().num_threads()


def set_num_threads(n: int) -> None:
    default().set_num_threads(n)


def gdn_fwd(*a, **kw):
    return default().gdn_fwd(*a, **kw)


gdn_fwd.__doc__ = OracleLib.gdn_fwd.__doc__


def gdn_step(*a, **kw):
    return default().gdn_step(*a, **kw)


gdn_step.__doc__ = OracleLib.gdn_step.__doc__


def gdn2_fwd(*a, **kw):
    return default().gdn2_fwd(*a, **kw)


gdn2_fwd.__doc__ = OracleLib.gdn2_fwd.__doc__


def gdn_bwd(*a, **kw):
    return default().gdn_bwd(*a, **kw)


gdn_bwd.__doc__ = OracleLib.gdn_bwd.__doc__


def gdn2_bwd(*a, **kw):
    return default().gdn2_bwd(*a, **kw)


gdn2_bwd.__doc__ = OracleLib.gdn2_bwd.__doc__


def l2norm(*a, **kw):
    return default().l2norm(*a, **kw)


l2norm.__doc__ = OracleLib.l2norm.__doc__


def l2norm_bwd(*a, **kw):
    return default().l2norm_bwd(*a, **kw)


l2norm_bwd.__doc__ = OracleLib.l2norm_bwd.__doc__


def rmsnorm_gate(*a, **kw):
    return default().rmsnorm_gate(*a, **kw)


rmsnorm_gate.__doc__ = OracleLib.rmsnorm_gate.__doc__


def rmsnorm_gate_bwd(*a, **kw):
    return default().rmsnorm_gate_bwd(*a, **kw)


rmsnorm_gate_bwd.__doc__ = OracleLib.rmsnorm_gate_bwd.__doc__


def err_rms(x_hat, x) -> float:
    """Parity metric: max_i |x_hat_i - x_i| / sqrt(mean_i x_i^2); the plain
    max abs error when the reference is identically zero."""
    x_hat = _f64(x_hat)
    x = _f64(x)
    assert x_hat.shape == x.shape, (x_hat.shape, x.shape)
    if x.size == 0:
        return 0.0
    if not np.all(np.isfinite(x_hat)):
        return float("inf")
    d = np.max(np.abs(x_hat - x))
    rms = np.sqrt(np.mean(x * x))
    return float(d / rms) if rms > 0 else float(d)
