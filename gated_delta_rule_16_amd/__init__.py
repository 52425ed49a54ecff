"""Python binding of libgdr, the gfx950 gated delta rule library.

Argument marshalling only: every step of every operation runs in the HIP
kernels behind the C ABI declared in ``include/gdr.h``.  PyTorch supplies
device memory and the current HIP stream.  There is no CPU or PyTorch
fallback — importing this package without the built ``libgdr.so`` fails.

Functions mirror the C calls:

    gdr_chunk_fwd(q, k, v, alpha, beta, s0=None, ...)            -> (o, s_final)
    gdr_chunk_fwd_split(q, k, v, alpha, beta, s0=None, nseg=8, ...) -> (o, s_final)
    gdr_recurrent_step(q, k, v, alpha, beta, state, ...)         -> o
    gdr2_chunk_fwd(q, k, v, alpha, erase, write, s0=None, ...)   -> (o, s_final)
    gdr_output_gate(o, g, w=None, eps=1e-6, ...)                -> y
    gdr_output_gate_bwd(o, g, w, dy, eps=1e-6, ...)             -> (do, dg, dw)
    gdr_output_gate_bwd_noalloc(o, g, w, dy, eps=1e-6, ...)     -> (do, dg, dw)
    gdr_chunk_fwd_gate(q, k, v, alpha, beta, s0, g, w, eps, ...) -> (y, s_final)
    gdr_chunk_bwd(q, k, v, alpha, beta, s0, dout, ds_final=None)
        -> (dq, dk, dv, dalpha, dbeta, ds0)
    gdr2_chunk_bwd(q, k, v, alpha, erase, write, s0, dout, ds_final=None)
        -> (dq, dk, dv, dalpha, derase, dwrite, ds0)

``l2norm_qk=True`` calls the ``_ex`` variant of the same C function with
GDR_L2NORM_QK: q and k are L2-normalised on load inside the kernels.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads the HIP runtime libgdr.so binds to

__all__ = ["gdr_chunk_fwd", "gdr_recurrent_step", "gdr2_chunk_fwd", "gdr_output_gate",
           "gdr_chunk_bwd", "gdr_chunk_bwd_workspace_size",
           "gdr2_chunk_bwd", "gdr2_chunk_bwd_workspace_size",
           "gdr_chunk_fwd_split", "gdr_chunk_fwd_split_workspace_size",
           "gdr_output_gate_bwd", "gdr_output_gate_bwd_workspace_size",
           "gdr_output_gate_bwd_noalloc", "gdr_chunk_fwd_gate",
           "gdr_chunk_fwd_gate_workspace_size",
           "gdr_chunk_bwd_split", "gdr_chunk_bwd_split_workspace_size",
           "gdr2_chunk_fwd_split", "gdr2_chunk_bwd_split", "gdr2_chunk_bwd_split_workspace_size",
           "GdrError", "status_string", "lib", "LIB_PATH", "GDR_F32",
           "GDR_BF16", "GDR_L2NORM_QK", "GDR_SPLIT_FP32_STATES"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)),
                        "libgdr.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g;"
        f" g.build()'` (hipcc, gfx950) first")

lib = ctypes.CDLL(LIB_PATH)

GDR_F32, GDR_BF16 = 0, 1
GDR_L2NORM_QK = 1
GDR_SPLIT_FP32_STATES = 2
_I64, _P, _E, _U = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_uint32

lib.gdr_chunk_fwd.argtypes = [_I64] * 5 + [_E] + [_P] * 6 + [_E, _P, _P, _P]
lib.gdr_chunk_fwd.restype = ctypes.c_int
lib.gdr2_chunk_fwd.argtypes = [_I64] * 5 + [_E] + [_P] * 7 + [_E, _P, _P, _P]
lib.gdr2_chunk_fwd.restype = ctypes.c_int
lib.gdr_recurrent_step.argtypes = [_I64] * 4 + [_E] + [_P] * 6 + [_E, _P, _P]
lib.gdr_recurrent_step.restype = ctypes.c_int
lib.gdr_chunk_fwd_ex.argtypes = [_I64] * 5 + [_E] + [_P] * 6 + [_E, _P, _P, _U, _P]
lib.gdr_chunk_fwd_ex.restype = ctypes.c_int
lib.gdr2_chunk_fwd_ex.argtypes = [_I64] * 5 + [_E] + [_P] * 7 + [_E, _P, _P, _U, _P]
lib.gdr2_chunk_fwd_ex.restype = ctypes.c_int
lib.gdr_recurrent_step_ex.argtypes = [_I64] * 4 + [_E] + [_P] * 6 + [_E, _P, _U, _P]
lib.gdr_recurrent_step_ex.restype = ctypes.c_int
lib.gdr_output_gate.argtypes = [_I64] * 3 + [_E, _P, _E, _P, _P, ctypes.c_float, _E, _P, _P]
lib.gdr_output_gate.restype = ctypes.c_int
lib.gdr_chunk_bwd_workspace_size.argtypes = [_I64] * 5
lib.gdr_chunk_bwd_workspace_size.restype = ctypes.c_size_t
lib.gdr_chunk_bwd.argtypes = ([_I64] * 5 + [_E] + [_P] * 6 + [_E, _P, _P] + [_P] * 6 +
                              [_P, ctypes.c_size_t, _P])
lib.gdr_chunk_bwd.restype = ctypes.c_int
lib.gdr_chunk_bwd_ex.argtypes = ([_I64] * 5 + [_E] + [_P] * 6 + [_E, _P, _P] + [_P] * 6 +
                                 [_P, ctypes.c_size_t, _U, _P])
lib.gdr_chunk_bwd_ex.restype = ctypes.c_int
lib.gdr2_chunk_bwd_workspace_size.argtypes = [_I64] * 5
lib.gdr2_chunk_bwd_workspace_size.restype = ctypes.c_size_t
lib.gdr2_chunk_bwd.argtypes = ([_I64] * 5 + [_E] + [_P] * 7 + [_E, _P, _P] + [_P] * 7 +
                               [_P, ctypes.c_size_t, _P])
lib.gdr2_chunk_bwd.restype = ctypes.c_int
lib.gdr2_chunk_bwd_ex.argtypes = ([_I64] * 5 + [_E] + [_P] * 7 + [_E, _P, _P] + [_P] * 7 +
                                  [_P, ctypes.c_size_t, _U, _P])
lib.gdr2_chunk_bwd_ex.restype = ctypes.c_int
lib.gdr_chunk_fwd_split_workspace_size.argtypes = [_I64] * 5 + [_E, _I64]
lib.gdr_chunk_fwd_split_workspace_size.restype = ctypes.c_size_t
lib.gdr_chunk_fwd_split.argtypes = ([_I64] * 5 + [_E] + [_P] * 6 + [_E, _P, _P, _I64, _U, _P,
                                    ctypes.c_size_t, _P])
lib.gdr_chunk_fwd_split.restype = ctypes.c_int
lib.gdr_output_gate_bwd_workspace_size.argtypes = [_I64] * 3
lib.gdr_output_gate_bwd_workspace_size.restype = ctypes.c_size_t
lib.gdr_output_gate_bwd.argtypes = ([_I64] * 3 + [_E, _P, _E, _P, _P, ctypes.c_float, _E, _P] +
                                    [_P] * 4 + [ctypes.c_size_t, _P])
lib.gdr_output_gate_bwd.restype = ctypes.c_int
lib.gdr_output_gate_bwd_noalloc.argtypes = ([_I64] * 3 + [_E, _P, _E, _P, _P, ctypes.c_float, _E,
                                            _P] + [_P] * 3 + [_P])
lib.gdr_output_gate_bwd_noalloc.restype = ctypes.c_int
lib.gdr_chunk_fwd_gate_workspace_size.argtypes = [_I64] * 5 + [_E]
lib.gdr_chunk_fwd_gate_workspace_size.restype = ctypes.c_size_t
lib.gdr_chunk_fwd_gate.argtypes = ([_I64] * 5 + [_E] + [_P] * 6 + [_E, _P, _P, ctypes.c_float, _E,
                                   _P, _P, _U, _P, ctypes.c_size_t, _P])
lib.gdr_chunk_fwd_gate.restype = ctypes.c_int
lib.gdr_chunk_bwd_split_workspace_size.argtypes = [_I64] * 5 + [_E, _I64]
lib.gdr_chunk_bwd_split_workspace_size.restype = ctypes.c_size_t
lib.gdr_chunk_bwd_split.argtypes = ([_I64] * 5 + [_E] + [_P] * 6 + [_E, _P, _P] + [_P] * 6 +
                                    [_I64, _U, _P, ctypes.c_size_t, _P])
lib.gdr_chunk_bwd_split.restype = ctypes.c_int
lib.gdr2_chunk_fwd_split.argtypes = ([_I64] * 5 + [_E] + [_P] * 7 + [_E, _P, _P, _I64, _U, _P,
                                     ctypes.c_size_t, _P])
lib.gdr2_chunk_fwd_split.restype = ctypes.c_int
lib.gdr2_chunk_bwd_split_workspace_size.argtypes = [_I64] * 5 + [_E, _I64]
lib.gdr2_chunk_bwd_split_workspace_size.restype = ctypes.c_size_t
lib.gdr2_chunk_bwd_split.argtypes = ([_I64] * 5 + [_E] + [_P] * 7 + [_E, _P, _P] + [_P] * 7 +
                                     [_I64, _U, _P, ctypes.c_size_t, _P])
lib.gdr2_chunk_bwd_split.restype = ctypes.c_int
lib.gdr_status_string.argtypes = [ctypes.c_int]
lib.gdr_status_string.restype = ctypes.c_char_p
lib.gdr_version.restype = ctypes.c_int

_DT = {torch.float32: GDR_F32, torch.bfloat16: GDR_BF16}


class GdrError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn}: {status_string(code)} (status {code})")
        self.code = code


def status_string(code: int) -> str:
    return lib.gdr_status_string(int(code)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(name, t, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _run(name, code):
    if code != 0:
        raise GdrError(name, code)


def gdr_chunk_fwd(q, k, v, alpha, beta, s0=None, *, out_dtype=None, o=None,
                  s_final=None, want_state=True, l2norm_qk=False, stream=None):
    """Chunkwise gated delta rule forward.

    q, k [B,T,H,Dk]; v [B,T,H,Dv] (fp32 or bf16, same dtype); alpha, beta
    [B,T,H] fp32; s0 [B,H,Dv,Dk] fp32 or None.  ``out_dtype`` defaults to
    the input dtype.  Returns (o [B,T,H,Dv], s_final [B,H,Dv,Dk] or None).
    ``s_final`` may be passed in (it may be ``s0`` itself).
    """
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if q.dtype not in _DT:
        raise TypeError(f"unsupported input dtype {q.dtype}")
    _check("q", q, q.dtype, (B, T, H, Dk))
    _check("k", k, q.dtype, (B, T, H, Dk))
    _check("v", v, q.dtype, (B, T, H, Dv))
    _check("alpha", alpha, torch.float32, (B, T, H))
    _check("beta", beta, torch.float32, (B, T, H))
    if s0 is not None:
        _check("s0", s0, torch.float32, (B, H, Dv, Dk))
    odt = q.dtype if out_dtype is None else out_dtype
    if odt not in _DT:
        raise TypeError(f"unsupported output dtype {odt}")
    if o is None:
        o = torch.empty((B, T, H, Dv), dtype=odt, device=q.device)
    _check("o", o, odt, (B, T, H, Dv))
    if s_final is None and want_state:
        s_final = torch.empty((B, H, Dv, Dk), dtype=torch.float32, device=q.device)
    if s_final is not None:
        _check("s_final", s_final, torch.float32, (B, H, Dv, Dk))
    args = (B, T, H, Dk, Dv, _DT[q.dtype], _ptr(q), _ptr(k), _ptr(v),
            _ptr(alpha), _ptr(beta), _ptr(s0), _DT[odt], _ptr(o), _ptr(s_final))
    if l2norm_qk:
        _run("gdr_chunk_fwd_ex", lib.gdr_chunk_fwd_ex(*args, GDR_L2NORM_QK, _stream(stream)))
    else:
        _run("gdr_chunk_fwd", lib.gdr_chunk_fwd(*args, _stream(stream)))
    return o, s_final


def gdr_chunk_fwd_gate_workspace_size(B, T, H, Dk, Dv, dtype) -> int:
    """Bytes of device workspace gdr_chunk_fwd_gate needs (0: none)."""
    return int(lib.gdr_chunk_fwd_gate_workspace_size(B, T, H, Dk, Dv, _DT[dtype]))


def gdr_chunk_fwd_gate(q, k, v, alpha, beta, s0, g, w=None, eps=1e-6, *, out_dtype=None, y=None,
                       s_final=None, want_state=True, l2norm_qk=False, workspace=None,
                       stream=None):
    """gdr_chunk_fwd followed by the output gate, y = o / sqrt(mean o^2 + eps)
    w SiLU(g), fused on the forward's stores (bf16 inputs).  g [B,T,H,Dv]
    fp32 or bf16, w [Dv] fp32 or None.  Returns (y [B,T,H,Dv], s_final or
    None); ``workspace`` (uint8 GPU tensor) is allocated here when None."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if q.dtype not in _DT or g.dtype not in _DT:
        raise TypeError("q and g must be float32 or bfloat16")
    _check("q", q, q.dtype, (B, T, H, Dk))
    _check("k", k, q.dtype, (B, T, H, Dk))
    _check("v", v, q.dtype, (B, T, H, Dv))
    _check("alpha", alpha, torch.float32, (B, T, H))
    _check("beta", beta, torch.float32, (B, T, H))
    _check("g", g, g.dtype, (B, T, H, Dv))
    if s0 is not None:
        _check("s0", s0, torch.float32, (B, H, Dv, Dk))
    if w is not None:
        _check("w", w, torch.float32, (Dv,))
    odt = q.dtype if out_dtype is None else out_dtype
    if odt not in _DT:
        raise TypeError(f"unsupported output dtype {odt}")
    if y is None:
        y = torch.empty((B, T, H, Dv), dtype=odt, device=q.device)
    _check("y", y, odt, (B, T, H, Dv))
    if s_final is None and want_state:
        s_final = torch.empty((B, H, Dv, Dk), dtype=torch.float32, device=q.device)
    if s_final is not None:
        _check("s_final", s_final, torch.float32, (B, H, Dv, Dk))
    if workspace is None:
        workspace = torch.empty(max(gdr_chunk_fwd_gate_workspace_size(B, T, H, Dk, Dv, q.dtype), 16),
                                dtype=torch.uint8, device=q.device)
    _check("workspace", workspace, torch.uint8)
    _run("gdr_chunk_fwd_gate", lib.gdr_chunk_fwd_gate(
        B, T, H, Dk, Dv, _DT[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
        _ptr(s0), _DT[g.dtype], _ptr(g), _ptr(w), float(eps), _DT[odt], _ptr(y), _ptr(s_final),
        GDR_L2NORM_QK if l2norm_qk else 0, _ptr(workspace), workspace.numel(), _stream(stream)))
    return y, s_final


def gdr_chunk_fwd_split_workspace_size(B, T, H, Dk, Dv, dtype, nseg) -> int:
    """Bytes of device workspace gdr_chunk_fwd_split needs (0: none)."""
    return int(lib.gdr_chunk_fwd_split_workspace_size(B, T, H, Dk, Dv, _DT[dtype], nseg))


def gdr_chunk_fwd_split(q, k, v, alpha, beta, s0=None, *, nseg=8, out_dtype=None, o=None,
                        s_final=None, want_state=True, l2norm_qk=False, workspace=None,
                        stream=None):
    """gdr_chunk_fwd with each sequence split into ``nseg`` segments that run
    side by side (T divisible by nseg).  Same arguments and results as
    gdr_chunk_fwd; ``workspace`` is a uint8 GPU tensor of at least
    gdr_chunk_fwd_split_workspace_size(...) bytes, allocated here when None."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if q.dtype not in _DT:
        raise TypeError(f"unsupported input dtype {q.dtype}")
    _check("q", q, q.dtype, (B, T, H, Dk))
    _check("k", k, q.dtype, (B, T, H, Dk))
    _check("v", v, q.dtype, (B, T, H, Dv))
    _check("alpha", alpha, torch.float32, (B, T, H))
    _check("beta", beta, torch.float32, (B, T, H))
    if s0 is not None:
        _check("s0", s0, torch.float32, (B, H, Dv, Dk))
    odt = q.dtype if out_dtype is None else out_dtype
    if odt not in _DT:
        raise TypeError(f"unsupported output dtype {odt}")
    if o is None:
        o = torch.empty((B, T, H, Dv), dtype=odt, device=q.device)
    _check("o", o, odt, (B, T, H, Dv))
    if s_final is None and want_state:
        s_final = torch.empty((B, H, Dv, Dk), dtype=torch.float32, device=q.device)
    if s_final is not None:
        _check("s_final", s_final, torch.float32, (B, H, Dv, Dk))
    need = gdr_chunk_fwd_split_workspace_size(B, T, H, Dk, Dv, q.dtype, nseg)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check("workspace", workspace, torch.uint8)
    _run("gdr_chunk_fwd_split", lib.gdr_chunk_fwd_split(
        B, T, H, Dk, Dv, _DT[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
        _ptr(s0), _DT[odt], _ptr(o), _ptr(s_final), nseg, GDR_L2NORM_QK if l2norm_qk else 0,
        _ptr(workspace), workspace.numel(), _stream(stream)))
    return o, s_final


def gdr2_chunk_fwd(q, k, v, alpha, erase, write, s0=None, *, out_dtype=None,
                   o=None, s_final=None, want_state=True, l2norm_qk=False,
                   stream=None):
    """Chunkwise Gated Delta Rule-2 forward.

    q, k, alpha, erase [B,T,H,Dk]; v, write [B,T,H,Dv], all one dtype (fp32
    or bf16); s0 [B,H,Dv,Dk] fp32 or None.  Returns (o, s_final).
    """
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if q.dtype not in _DT:
        raise TypeError(f"unsupported input dtype {q.dtype}")
    for name, t, d in (("q", q, Dk), ("k", k, Dk), ("alpha", alpha, Dk),
                       ("erase", erase, Dk), ("v", v, Dv), ("write", write, Dv)):
        _check(name, t, q.dtype, (B, T, H, d))
    if s0 is not None:
        _check("s0", s0, torch.float32, (B, H, Dv, Dk))
    odt = q.dtype if out_dtype is None else out_dtype
    if odt not in _DT:
        raise TypeError(f"unsupported output dtype {odt}")
    if o is None:
        o = torch.empty((B, T, H, Dv), dtype=odt, device=q.device)
    _check("o", o, odt, (B, T, H, Dv))
    if s_final is None and want_state:
        s_final = torch.empty((B, H, Dv, Dk), dtype=torch.float32, device=q.device)
    if s_final is not None:
        _check("s_final", s_final, torch.float32, (B, H, Dv, Dk))
    args = (B, T, H, Dk, Dv, _DT[q.dtype], _ptr(q), _ptr(k), _ptr(v),
            _ptr(alpha), _ptr(erase), _ptr(write), _ptr(s0), _DT[odt], _ptr(o),
            _ptr(s_final))
    if l2norm_qk:
        _run("gdr2_chunk_fwd_ex", lib.gdr2_chunk_fwd_ex(*args, GDR_L2NORM_QK, _stream(stream)))
    else:
        _run("gdr2_chunk_fwd", lib.gdr2_chunk_fwd(*args, _stream(stream)))
    return o, s_final


def gdr_recurrent_step(q, k, v, alpha, beta, state, *, out_dtype=None,
                       o=None, l2norm_qk=False, stream=None):
    """One decode token: q, k [N,H,Dk]; v [N,H,Dv]; alpha, beta [N,H] fp32;
    state [N,H,Dv,Dk] fp32, updated in place.  Returns o [N,H,Dv]."""
    N, H, Dk = q.shape
    Dv = v.shape[-1]
    if q.dtype not in _DT:
        raise TypeError(f"unsupported input dtype {q.dtype}")
    _check("q", q, q.dtype, (N, H, Dk))
    _check("k", k, q.dtype, (N, H, Dk))
    _check("v", v, q.dtype, (N, H, Dv))
    _check("alpha", alpha, torch.float32, (N, H))
    _check("beta", beta, torch.float32, (N, H))
    _check("state", state, torch.float32, (N, H, Dv, Dk))
    odt = q.dtype if out_dtype is None else out_dtype
    if o is None:
        o = torch.empty((N, H, Dv), dtype=odt, device=q.device)
    _check("o", o, odt, (N, H, Dv))
    args = (N, H, Dk, Dv, _DT[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
            _ptr(beta), _ptr(state), _DT[odt], _ptr(o))
    if l2norm_qk:
        _run("gdr_recurrent_step_ex", lib.gdr_recurrent_step_ex(
            *args, GDR_L2NORM_QK, _stream(stream)))
    else:
        _run("gdr_recurrent_step", lib.gdr_recurrent_step(*args, _stream(stream)))
    return o


def gdr_output_gate(o, g, w=None, eps=1e-6, *, out_dtype=None, y=None, stream=None):
    """The block's output gate: y = o / sqrt(mean(o^2) + eps) * w * SiLU(g)
    over the last axis (Dv = 64 or 128).  o, g [..., H, Dv] (fp32 or bf16,
    each its own dtype); w [Dv] fp32 or None.  ``y`` may be ``o`` itself
    (same dtype) for an in-place gate.  Returns y."""
    if o.dim() < 2:
        raise ValueError("o must be [..., H, Dv]")
    H, Dv = o.shape[-2], o.shape[-1]
    N = o.numel() // (H * Dv) if H * Dv else 0
    for name, t in (("o", o), ("g", g)):
        if t.dtype not in _DT:
            raise TypeError(f"unsupported {name} dtype {t.dtype}")
    _check("o", o, o.dtype, tuple(o.shape))
    _check("g", g, g.dtype, tuple(o.shape))
    if w is not None:
        _check("w", w, torch.float32, (Dv,))
    if out_dtype is None:
        odt = o.dtype if y is None else y.dtype
    else:
        odt = out_dtype
    if odt not in _DT:
        raise TypeError(f"unsupported output dtype {odt}")
    if y is None:
        y = torch.empty(o.shape, dtype=odt, device=o.device)
    _check("y", y, odt, tuple(o.shape))
    _run("gdr_output_gate", lib.gdr_output_gate(
        N, H, Dv, _DT[o.dtype], _ptr(o), _DT[g.dtype], _ptr(g), _ptr(w), float(eps),
        _DT[odt], _ptr(y), _stream(stream)))
    return y


def gdr_chunk_bwd_workspace_size(B, T, H, Dk, Dv) -> int:
    """Bytes of device workspace gdr_chunk_bwd needs for these sizes."""
    return int(lib.gdr_chunk_bwd_workspace_size(B, T, H, Dk, Dv))


def gdr_chunk_bwd(q, k, v, alpha, beta, s0, dout, ds_final=None, *, workspace=None,
                  want_ds0=True, l2norm_qk=False, stream=None):
    """Reverse mode of gdr_chunk_fwd: returns fp32 (dq, dk, dv, dalpha,
    dbeta, ds0) for dL/do = ``dout`` [B,T,H,Dv] (fp32 or bf16) and
    dL/dS_T = ``ds_final`` [B,H,Dv,Dk] fp32 or None.  Inputs as for
    gdr_chunk_fwd.  ``workspace`` is a uint8 GPU tensor of at least
    gdr_chunk_bwd_workspace_size(...) bytes, allocated here when None.
    dq and dk are summed over blocks of state rows by atomic adds, so they
    can differ from run to run in the last bits."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if q.dtype not in _DT or dout.dtype not in _DT:
        raise TypeError("q and dout must be float32 or bfloat16")
    _check("q", q, q.dtype, (B, T, H, Dk))
    _check("k", k, q.dtype, (B, T, H, Dk))
    _check("v", v, q.dtype, (B, T, H, Dv))
    _check("alpha", alpha, torch.float32, (B, T, H))
    _check("beta", beta, torch.float32, (B, T, H))
    _check("dout", dout, dout.dtype, (B, T, H, Dv))
    if s0 is not None:
        _check("s0", s0, torch.float32, (B, H, Dv, Dk))
    if ds_final is not None:
        _check("ds_final", ds_final, torch.float32, (B, H, Dv, Dk))
    need = gdr_chunk_bwd_workspace_size(B, T, H, Dk, Dv)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check("workspace", workspace, torch.uint8)
    f32 = dict(dtype=torch.float32, device=q.device)
    dq = torch.empty((B, T, H, Dk), **f32)
    dk = torch.empty((B, T, H, Dk), **f32)
    dv = torch.empty((B, T, H, Dv), **f32)
    da = torch.empty((B, T, H), **f32)
    db = torch.empty((B, T, H), **f32)
    ds0 = torch.empty((B, H, Dv, Dk), **f32) if want_ds0 else None
    args = (B, T, H, Dk, Dv, _DT[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
            _ptr(s0), _DT[dout.dtype], _ptr(dout), _ptr(ds_final), _ptr(dq), _ptr(dk), _ptr(dv),
            _ptr(da), _ptr(db), _ptr(ds0), _ptr(workspace), workspace.numel())
    if l2norm_qk:
        _run("gdr_chunk_bwd_ex", lib.gdr_chunk_bwd_ex(*args, GDR_L2NORM_QK, _stream(stream)))
    else:
        _run("gdr_chunk_bwd", lib.gdr_chunk_bwd(*args, _stream(stream)))
    return dq, dk, dv, da, db, ds0


def gdr2_chunk_bwd_workspace_size(B, T, H, Dk, Dv) -> int:
    """Bytes of device workspace gdr2_chunk_bwd needs for these sizes."""
    return int(lib.gdr2_chunk_bwd_workspace_size(B, T, H, Dk, Dv))


def gdr2_chunk_bwd(q, k, v, alpha, erase, write, s0, dout, ds_final=None, *, workspace=None,
                   want_ds0=True, l2norm_qk=False, stream=None):
    """Reverse mode of gdr2_chunk_fwd: returns fp32 (dq, dk, dv, dalpha,
    derase, dwrite, ds0) for dL/do = ``dout`` [B,T,H,Dv] (fp32 or bf16) and
    dL/dS_T = ``ds_final`` [B,H,Dv,Dk] fp32 or None.  Inputs as for
    gdr2_chunk_fwd.  ``workspace`` is a uint8 GPU tensor of at least
    gdr2_chunk_bwd_workspace_size(...) bytes, allocated here when None."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if q.dtype not in _DT or dout.dtype not in _DT:
        raise TypeError("q and dout must be float32 or bfloat16")
    for name, x, d in (("q", q, Dk), ("k", k, Dk), ("v", v, Dv), ("alpha", alpha, Dk),
                       ("erase", erase, Dk), ("write", write, Dv)):
        _check(name, x, q.dtype, (B, T, H, d))
    _check("dout", dout, dout.dtype, (B, T, H, Dv))
    if s0 is not None:
        _check("s0", s0, torch.float32, (B, H, Dv, Dk))
    if ds_final is not None:
        _check("ds_final", ds_final, torch.float32, (B, H, Dv, Dk))
    need = gdr2_chunk_bwd_workspace_size(B, T, H, Dk, Dv)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check("workspace", workspace, torch.uint8)
    f32 = dict(dtype=torch.float32, device=q.device)
    dq = torch.empty((B, T, H, Dk), **f32)
    dk = torch.empty((B, T, H, Dk), **f32)
    dv = torch.empty((B, T, H, Dv), **f32)
    da = torch.empty((B, T, H, Dk), **f32)
    de = torch.empty((B, T, H, Dk), **f32)
    dw = torch.empty((B, T, H, Dv), **f32)
    ds0 = torch.empty((B, H, Dv, Dk), **f32) if want_ds0 else None
    args = (B, T, H, Dk, Dv, _DT[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(erase),
            _ptr(write), _ptr(s0), _DT[dout.dtype], _ptr(dout), _ptr(ds_final), _ptr(dq),
            _ptr(dk), _ptr(dv), _ptr(da), _ptr(de), _ptr(dw), _ptr(ds0), _ptr(workspace),
            workspace.numel())
    if l2norm_qk:
        _run("gdr2_chunk_bwd_ex", lib.gdr2_chunk_bwd_ex(*args, GDR_L2NORM_QK, _stream(stream)))
    else:
        _run("gdr2_chunk_bwd", lib.gdr2_chunk_bwd(*args, _stream(stream)))
    return dq, dk, dv, da, de, dw, ds0


def gdr_output_gate_bwd_workspace_size(N, H, Dv) -> int:
    """Bytes of device workspace gdr_output_gate_bwd needs for dw."""
    return int(lib.gdr_output_gate_bwd_workspace_size(N, H, Dv))


def gdr_output_gate_bwd(o, g, w, dy, eps=1e-6, *, want_dw=True, workspace=None, stream=None):
    """Reverse mode of gdr_output_gate: o, g, dy [..., H, Dv] (fp32 or bf16
    each), w [Dv] fp32 or None (ones).  Returns fp32 (do, dg, dw); dw [Dv]
    is None when ``want_dw`` is False."""
    if o.dim() < 2:
        raise ValueError("o must be [..., H, Dv]")
    H, Dv = o.shape[-2], o.shape[-1]
    N = o.numel() // (H * Dv) if o.numel() else 0
    for name, t in (("o", o), ("g", g), ("dy", dy)):
        if t.dtype not in _DT:
            raise TypeError(f"{name} must be float32 or bfloat16")
        _check(name, t, t.dtype, tuple(o.shape))
    if w is not None:
        _check("w", w, torch.float32, (Dv,))
    f32 = dict(dtype=torch.float32, device=o.device)
    do = torch.empty(o.shape, **f32)
    dg = torch.empty(o.shape, **f32)
    dw = torch.empty((Dv,), **f32) if want_dw else None
    if dw is not None and workspace is None:
        workspace = torch.empty(max(gdr_output_gate_bwd_workspace_size(N, H, Dv), 16),
                                dtype=torch.uint8, device=o.device)
    if workspace is not None:
        _check("workspace", workspace, torch.uint8)
    _run("gdr_output_gate_bwd", lib.gdr_output_gate_bwd(
        N, H, Dv, _DT[o.dtype], _ptr(o), _DT[g.dtype], _ptr(g), _ptr(w), float(eps),
        _DT[dy.dtype], _ptr(dy), _ptr(do), _ptr(dg), _ptr(dw), _ptr(workspace),
        0 if workspace is None else workspace.numel(), _stream(stream)))
    return do, dg, dw


def gdr_output_gate_bwd_noalloc(o, g, w, dy, eps=1e-6, *, want_dw=True, out=None, stream=None):
    """gdr_output_gate_bwd through the C call that takes no workspace (its
    dw partials go to the library's own per-GPU array).  ``out`` may give
    preallocated fp32 (do, dg, dw) tensors; otherwise they are created here.
    Returns (do, dg, dw), dw None when ``want_dw`` is False."""
    if o.dim() < 2:
        raise ValueError("o must be [..., H, Dv]")
    H, Dv = o.shape[-2], o.shape[-1]
    N = o.numel() // (H * Dv) if o.numel() else 0
    for name, t in (("o", o), ("g", g), ("dy", dy)):
        if t.dtype not in _DT:
            raise TypeError(f"{name} must be float32 or bfloat16")
        _check(name, t, t.dtype, tuple(o.shape))
    if w is not None:
        _check("w", w, torch.float32, (Dv,))
    if out is None:
        f32 = dict(dtype=torch.float32, device=o.device)
        out = (torch.empty(o.shape, **f32), torch.empty(o.shape, **f32),
               torch.empty((Dv,), **f32) if want_dw else None)
    do, dg, dw = out
    _check("do", do, torch.float32, tuple(o.shape))
    _check("dg", dg, torch.float32, tuple(o.shape))
    if dw is not None:
        _check("dw", dw, torch.float32, (Dv,))
    _run("gdr_output_gate_bwd_noalloc", lib.gdr_output_gate_bwd_noalloc(
        N, H, Dv, _DT[o.dtype], _ptr(o), _DT[g.dtype], _ptr(g), _ptr(w), float(eps),
        _DT[dy.dtype], _ptr(dy), _ptr(do), _ptr(dg), _ptr(dw), _stream(stream)))
    return do, dg, dw


def gdr_chunk_bwd_split_workspace_size(B, T, H, Dk, Dv, dtype, nseg) -> int:
    """Bytes of device workspace gdr_chunk_bwd_split needs."""
    return int(lib.gdr_chunk_bwd_split_workspace_size(B, T, H, Dk, Dv, _DT[dtype], nseg))


def gdr_chunk_bwd_split(q, k, v, alpha, beta, s0, dout, ds_final=None, *, nseg=8, workspace=None,
                        want_ds0=True, l2norm_qk=False, stream=None):
    """gdr_chunk_bwd with each sequence split into ``nseg`` segments that run
    side by side (T divisible by nseg).  Same arguments and results as
    gdr_chunk_bwd."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if q.dtype not in _DT or dout.dtype not in _DT:
        raise TypeError("q and dout must be float32 or bfloat16")
    _check("q", q, q.dtype, (B, T, H, Dk))
    _check("k", k, q.dtype, (B, T, H, Dk))
    _check("v", v, q.dtype, (B, T, H, Dv))
    _check("alpha", alpha, torch.float32, (B, T, H))
    _check("beta", beta, torch.float32, (B, T, H))
    _check("dout", dout, dout.dtype, (B, T, H, Dv))
    if s0 is not None:
        _check("s0", s0, torch.float32, (B, H, Dv, Dk))
    if ds_final is not None:
        _check("ds_final", ds_final, torch.float32, (B, H, Dv, Dk))
    need = gdr_chunk_bwd_split_workspace_size(B, T, H, Dk, Dv, q.dtype, nseg)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check("workspace", workspace, torch.uint8)
    f32 = dict(dtype=torch.float32, device=q.device)
    dq = torch.empty((B, T, H, Dk), **f32)
    dk = torch.empty((B, T, H, Dk), **f32)
    dv = torch.empty((B, T, H, Dv), **f32)
    da = torch.empty((B, T, H), **f32)
    db = torch.empty((B, T, H), **f32)
    ds0 = torch.empty((B, H, Dv, Dk), **f32) if want_ds0 else None
    _run("gdr_chunk_bwd_split", lib.gdr_chunk_bwd_split(
        B, T, H, Dk, Dv, _DT[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
        _ptr(s0), _DT[dout.dtype], _ptr(dout), _ptr(ds_final), _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(da), _ptr(db), _ptr(ds0), nseg, GDR_L2NORM_QK if l2norm_qk else 0,
        _ptr(workspace), workspace.numel(), _stream(stream)))
    return dq, dk, dv, da, db, ds0


def gdr2_chunk_fwd_split(q, k, v, alpha, erase, write, s0=None, *, nseg=8, out_dtype=None,
                         o=None, s_final=None, want_state=True, l2norm_qk=False, workspace=None,
                         stream=None):
    """gdr2_chunk_fwd with each sequence split into ``nseg`` segments that
    run side by side (T divisible by nseg); workspace as for
    gdr_chunk_fwd_split."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if q.dtype not in _DT:
        raise TypeError(f"unsupported input dtype {q.dtype}")
    for name, x, d in (("q", q, Dk), ("k", k, Dk), ("v", v, Dv), ("alpha", alpha, Dk),
                       ("erase", erase, Dk), ("write", write, Dv)):
        _check(name, x, q.dtype, (B, T, H, d))
    if s0 is not None:
        _check("s0", s0, torch.float32, (B, H, Dv, Dk))
    odt = q.dtype if out_dtype is None else out_dtype
    if odt not in _DT:
        raise TypeError(f"unsupported output dtype {odt}")
    if o is None:
        o = torch.empty((B, T, H, Dv), dtype=odt, device=q.device)
    _check("o", o, odt, (B, T, H, Dv))
    if s_final is None and want_state:
        s_final = torch.empty((B, H, Dv, Dk), dtype=torch.float32, device=q.device)
    if s_final is not None:
        _check("s_final", s_final, torch.float32, (B, H, Dv, Dk))
    need = gdr_chunk_fwd_split_workspace_size(B, T, H, Dk, Dv, q.dtype, nseg)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check("workspace", workspace, torch.uint8)
    _run("gdr2_chunk_fwd_split", lib.gdr2_chunk_fwd_split(
        B, T, H, Dk, Dv, _DT[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(erase),
        _ptr(write), _ptr(s0), _DT[odt], _ptr(o), _ptr(s_final), nseg,
        GDR_L2NORM_QK if l2norm_qk else 0, _ptr(workspace), workspace.numel(), _stream(stream)))
    return o, s_final


def gdr2_chunk_bwd_split_workspace_size(B, T, H, Dk, Dv, dtype, nseg) -> int:
    """Bytes of device workspace gdr2_chunk_bwd_split needs."""
    return int(lib.gdr2_chunk_bwd_split_workspace_size(B, T, H, Dk, Dv, _DT[dtype], nseg))


def gdr2_chunk_bwd_split(q, k, v, alpha, erase, write, s0, dout, ds_final=None, *, nseg=8,
                         workspace=None, want_ds0=True, l2norm_qk=False, fp32_states=False,
                         stream=None):
    """gdr2_chunk_bwd with each sequence split into ``nseg`` segments that
    run side by side.  Same arguments and results as gdr2_chunk_bwd.
    ``fp32_states`` (GDR_SPLIT_FP32_STATES) runs the plain backward over
    the whole sequence instead (fp32 states throughout, no split)."""
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    if q.dtype not in _DT or dout.dtype not in _DT:
        raise TypeError("q and dout must be float32 or bfloat16")
    for name, x, d in (("q", q, Dk), ("k", k, Dk), ("v", v, Dv), ("alpha", alpha, Dk),
                       ("erase", erase, Dk), ("write", write, Dv)):
        _check(name, x, q.dtype, (B, T, H, d))
    _check("dout", dout, dout.dtype, (B, T, H, Dv))
    if s0 is not None:
        _check("s0", s0, torch.float32, (B, H, Dv, Dk))
    if ds_final is not None:
        _check("ds_final", ds_final, torch.float32, (B, H, Dv, Dk))
    need = gdr2_chunk_bwd_split_workspace_size(B, T, H, Dk, Dv, q.dtype, nseg)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check("workspace", workspace, torch.uint8)
    f32 = dict(dtype=torch.float32, device=q.device)
    out = [torch.empty((B, T, H, d), **f32) for d in (Dk, Dk, Dv, Dk, Dk, Dv)]
    ds0 = torch.empty((B, H, Dv, Dk), **f32) if want_ds0 else None
    _run("gdr2_chunk_bwd_split", lib.gdr2_chunk_bwd_split(
        B, T, H, Dk, Dv, _DT[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(erase),
        _ptr(write), _ptr(s0), _DT[dout.dtype], _ptr(dout), _ptr(ds_final),
        *[_ptr(x) for x in out], _ptr(ds0), nseg,
        (GDR_L2NORM_QK if l2norm_qk else 0) | (GDR_SPLIT_FP32_STATES if fp32_states else 0),
        _ptr(workspace), workspace.numel(), _stream(stream)))
    return tuple(out) + (ds0,)
