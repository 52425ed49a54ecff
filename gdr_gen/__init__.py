"""Seeded synthetic inputs for the gated delta rule kernels and their oracle.

This module draws random tensors and nothing else: it holds none of the
recurrence's arithmetic.  It is the one piece of code that both the fp64 CPU
oracle (``oracle/``) and the HIP path are fed from, so that both see exactly
the same bits.

Recipe (shapes follow a 1.3B Gated DeltaNet layer: 16 heads, head dim 128,
4K training length; see "Gated DeltaNet-2" on agihunt.info, the paragraph on
the 262,144-float recurrent state, and the ablation paragraph of the
meaningful96.github.io GDN review, section 4.2, for head dim 128):

* ``numpy.random.Generator(PCG64(seed))``; draws in a fixed order
  q, k, v, gate noise(s), initial state.
* q, k ~ N(0, 1) then L2-normalised per (token, head) in fp64 (the block's
  L2 step, review section 3.8); v ~ N(0, 1).  With ``raw_qk=True`` (inputs
  for the kernels' own L2 normalisation) q and k are instead left as drawn
  and each (token, head) row is scaled by exp(U(log 0.05, log 20)); those
  scales are drawn after everything else, so the other tensors keep their
  values.
* GDN scalar gates: alpha = exp(-softplus(x + shift)) with x ~ N(0, 1),
  beta = sigmoid(N(0, 1)).  GDN-2 gates: per-channel alpha of the same form,
  erase b and write w = sigmoid(N(0, 1)).
* Initial state, where present: N(0, std^2) in fp64.
* Every value is drawn in fp64, cast to fp32, then rounded to nearest-even
  bf16 where the dtype is bf16.  The oracle receives those rounded bits.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np
import torch

__all__ = [
    "GdnInputs", "Gdn2Inputs", "DecodeInputs",
    "make_gdn", "make_gdn2", "make_decode", "make_config", "CONFIGS", "make_gate",
    "make_device",
]

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _cast(x64: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x64, dtype=np.float32))
    return t.to(_DT[dtype]).contiguous()


def _unit_rows(x: np.ndarray) -> np.ndarray:
    # L2-normalise the last axis in fp64.  N(0,1) vectors of dim >= 8 are
    # never near zero, so no epsilon is added.
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True))


def _qk(g: np.random.Generator, q: np.ndarray, k: np.ndarray, raw: bool):
    # called after every other draw of a generator
    if not raw:
        return _unit_rows(q), _unit_rows(k)
    lo, hi = np.log(0.05), np.log(20.0)
    sq = np.exp(g.uniform(lo, hi, q.shape[:-1] + (1,)))
    sk = np.exp(g.uniform(lo, hi, k.shape[:-1] + (1,)))
    return q * sq, k * sk


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 0.5 * (1.0 + np.tanh(0.5 * x))


@dataclass
class GdnInputs:
    """Scalar-gated inputs: q, k [B,T,H,Dk]; v [B,T,H,Dv]; alpha, beta [B,T,H]
    fp32; s0 [B,H,Dv,Dk] fp32 or None."""
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    alpha: torch.Tensor
    beta: torch.Tensor
    s0: Optional[torch.Tensor]
    dtype: str
    name: str = ""
    meta: dict = field(default_factory=dict)


@dataclass
class Gdn2Inputs:
    """Channel-gated inputs: q, k, alpha, erase [B,T,H,Dk]; v, write
    [B,T,H,Dv], all in ``dtype``; s0 [B,H,Dv,Dk] fp32 or None."""
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    alpha: torch.Tensor
    erase: torch.Tensor
    write: torch.Tensor
    s0: Optional[torch.Tensor]
    dtype: str
    name: str = ""
    meta: dict = field(default_factory=dict)


@dataclass
class DecodeInputs:
    """Decode steps: state0 [N,H,Dv,Dk] fp32; q, k [steps,N,H,Dk];
    v [steps,N,H,Dv] in ``dtype``; alpha, beta [steps,N,H] fp32."""
    state0: torch.Tensor
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    alpha: torch.Tensor
    beta: torch.Tensor
    dtype: str
    name: str = ""
    meta: dict = field(default_factory=dict)


def make_gdn(B: int, T: int, H: int, Dk: int, Dv: int, dtype: str = "bf16",
             seed: int = 0, alpha_shift: float = 2.0,
             s0_std: Optional[float] = None, name: str = "",
             raw_qk: bool = False) -> GdnInputs:
    """Scalar-gated inputs; alpha = exp(-softplus(N(0,1) + alpha_shift))."""
    g = _rng(seed)
    q = g.standard_normal((B, T, H, Dk))
    k = g.standard_normal((B, T, H, Dk))
    v = g.standard_normal((B, T, H, Dv))
    a = np.exp(-_softplus(g.standard_normal((B, T, H)) + alpha_shift))
    b = _sigmoid(g.standard_normal((B, T, H)))
    s0 = None
    if s0_std is not None:
        s0 = _cast(s0_std * g.standard_normal((B, H, Dv, Dk)), "f32")
    q, k = _qk(g, q, k, raw_qk)
    return GdnInputs(_cast(q, dtype), _cast(k, dtype), _cast(v, dtype),
                     _cast(a, "f32"), _cast(b, "f32"), s0, dtype, name,
                     dict(B=B, T=T, H=H, Dk=Dk, Dv=Dv, seed=seed,
                          alpha_shift=alpha_shift, s0_std=s0_std,
                          raw_qk=raw_qk))


def make_gdn2(B: int, T: int, H: int, Dk: int, Dv: int, dtype: str = "bf16",
              seed: int = 0, alpha_shift: float = 2.0,
              s0_std: Optional[float] = None, name: str = "",
              raw_qk: bool = False) -> Gdn2Inputs:
    """Channel-gated inputs; per-channel alpha = exp(-softplus(N + shift)),
    erase and write = sigmoid(N(0,1))."""
    g = _rng(seed)
    q = g.standard_normal((B, T, H, Dk))
    k = g.standard_normal((B, T, H, Dk))
    v = g.standard_normal((B, T, H, Dv))
    a = np.exp(-_softplus(g.standard_normal((B, T, H, Dk)) + alpha_shift))
    e = _sigmoid(g.standard_normal((B, T, H, Dk)))
    w = _sigmoid(g.standard_normal((B, T, H, Dv)))
    s0 = None
    if s0_std is not None:
        s0 = _cast(s0_std * g.standard_normal((B, H, Dv, Dk)), "f32")
    q, k = _qk(g, q, k, raw_qk)
    return Gdn2Inputs(_cast(q, dtype), _cast(k, dtype), _cast(v, dtype),
                      _cast(a, dtype), _cast(e, dtype), _cast(w, dtype), s0,
                      dtype, name,
                      dict(B=B, T=T, H=H, Dk=Dk, Dv=Dv, seed=seed,
                           alpha_shift=alpha_shift, s0_std=s0_std,
                           raw_qk=raw_qk))


def make_decode(N: int, H: int, Dk: int, Dv: int, steps: int,
                dtype: str = "bf16", seed: int = 0, alpha_shift: float = 2.0,
                state_std: float = 0.02, name: str = "",
                raw_qk: bool = False) -> DecodeInputs:
    """Decode inputs: a random fp32 state and ``steps`` fresh tokens."""
    g = _rng(seed)
    q = g.standard_normal((steps, N, H, Dk))
    k = g.standard_normal((steps, N, H, Dk))
    v = g.standard_normal((steps, N, H, Dv))
    a = np.exp(-_softplus(g.standard_normal((steps, N, H)) + alpha_shift))
    b = _sigmoid(g.standard_normal((steps, N, H)))
    s = _cast(state_std * g.standard_normal((N, H, Dv, Dk)), "f32")
    q, k = _qk(g, q, k, raw_qk)
    return DecodeInputs(s, _cast(q, dtype), _cast(k, dtype), _cast(v, dtype),
                        _cast(a, "f32"), _cast(b, "f32"), dtype, name,
                        dict(N=N, H=H, Dk=Dk, Dv=Dv, steps=steps, seed=seed,
                             alpha_shift=alpha_shift, state_std=state_std,
                             raw_qk=raw_qk))


@dataclass
class GateInputs:
    o: torch.Tensor
    g: torch.Tensor
    w: Optional[torch.Tensor]
    meta: dict = field(default_factory=dict)


def make_gate(N: int, H: int, Dv: int, o_dtype: str = "f32", g_dtype: str = "bf16",
              seed: int = 0, weight: bool = True) -> GateInputs:
    """Inputs of the output gate: o ~ N(0, 1) with each (token, head) row
    scaled by exp(U(log 0.01, log 10)) (outputs of the rule span decades),
    the gate pre-activation g ~ N(0, 2^2), the norm weight w ~ U(0.5, 1.5)."""
    g_ = _rng(seed)
    o = g_.standard_normal((N, H, Dv)) * np.exp(g_.uniform(np.log(0.01), np.log(10.0), (N, H, 1)))
    gt = 2.0 * g_.standard_normal((N, H, Dv))
    w = g_.uniform(0.5, 1.5, Dv) if weight else None
    return GateInputs(_cast(o, o_dtype), _cast(gt, g_dtype),
                      None if w is None else _cast(w, "f32"),
                      dict(N=N, H=H, Dv=Dv, o_dtype=o_dtype, g_dtype=g_dtype, seed=seed,
                           weight=weight))


# The five workloads.  Seed = 1000 + index.  The long-context workload draws
# alpha near one as exp(-softplus(N(0,1) - 4)) (median ~0.98); the literal
# "+4" form is kept as workload "2lit" (median ~0.018).
CONFIGS = {
    0: dict(kind="gdn", B=1, T=256, H=2, Dk=64, Dv=64, dtype="f32",
            alpha_shift=2.0, s0_std=None),
    1: dict(kind="gdn", B=8, T=4096, H=16, Dk=128, Dv=128, dtype="bf16",
            alpha_shift=2.0, s0_std=None),
    2: dict(kind="gdn", B=1, T=32768, H=16, Dk=128, Dv=128, dtype="bf16",
            alpha_shift=-4.0, s0_std=0.02),
    "2lit": dict(kind="gdn", B=1, T=32768, H=16, Dk=128, Dv=128,
                 dtype="bf16", alpha_shift=4.0, s0_std=0.02),
    3: dict(kind="decode", N=256, H=16, Dk=128, Dv=128, steps=64,
            dtype="bf16", alpha_shift=2.0, state_std=0.02),
    4: dict(kind="gdn2", B=4, T=4096, H=16, Dk=128, Dv=128, dtype="bf16",
            alpha_shift=2.0, s0_std=None),
}

CONFIG_NAMES = {
    0: "tiny fp32 GDN fwd B1 H2 T256 d64",
    1: "GDN fwd B8 H16 T4096 d128 bf16",
    2: "long-context GDN fwd B1 H16 T32768 d128 bf16 (alpha near 1)",
    "2lit": "long-context GDN fwd B1 H16 T32768 d128 bf16 (alpha as N+4)",
    3: "decode N256 H16 d128 bf16, 64 steps",
    4: "GDN-2 fwd B4 H16 T4096 d128 bf16",
}


def make_config(idx, seed: Optional[int] = None, **overrides):
    """Build workload ``idx`` (0-4 or "2lit"); ``overrides`` replace shape
    fields (e.g. ``T=512``) for reduced-size parity cases."""
    c = dict(CONFIGS[idx])
    c.update(overrides)
    kind = c.pop("kind")
    if seed is None:
        seed = 1000 + (2 if idx == "2lit" else int(idx))
    name = CONFIG_NAMES[idx]
    if kind == "gdn":
        return make_gdn(seed=seed, name=name, **c)
    if kind == "gdn2":
        return make_gdn2(seed=seed, name=name, **c)
    return make_decode(seed=seed, name=name, **c)


def make_device(shapes: dict, seed: int, device="cuda", slab: int = 1 << 27) -> dict:
    """Large inputs drawn directly in device memory, for sizes a host draw
    would take minutes to produce (flat offsets past 2^31 elements).

    ``shapes`` maps a name to (shape, kind, dtype): kind "unit" is N(0, 1)
    rows L2-normalised over the last axis (in fp32), "normal" is N(0, 1),
    "decay" is exp(-softplus(N(0, 1) + 2)), "gate" is sigmoid(N(0, 1)).
    Tensors are drawn in the dict's order from one seeded
    ``torch.Generator`` on ``device``, ``slab`` elements (whole rows) at a
    time, in fp32, then cast to ``dtype``.  Same seed, same device type:
    same values.  Callers copy the parts they check to the host and give
    those bits to the oracle."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    out = {}
    for name, (shape, kind, dtype) in shapes.items():
        t = torch.empty(shape, dtype=dtype, device=device)
        flat = t.view(-1, shape[-1])
        rows = max(1, slab // shape[-1])
        for r0 in range(0, flat.shape[0], rows):
            n = min(rows, flat.shape[0] - r0)
            x = torch.randn((n, shape[-1]), generator=gen, device=device)
            if kind == "unit":
                x = x / x.norm(dim=-1, keepdim=True)
            elif kind == "decay":
                x = torch.exp(-torch.nn.functional.softplus(x + 2.0))
            elif kind == "gate":
                x = torch.sigmoid(x)
            elif kind != "normal":
                raise ValueError(kind)
            flat[r0:r0 + n] = x.to(dtype)
            del x
        out[name] = t
    return out
