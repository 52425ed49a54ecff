"""A seeded sweep of small, odd shapes over every call, each against the
fp64 oracle at the call's tolerance (bf16 inputs 2e-2, fp32 inputs 1e-3 for
the forwards, plus a bf16 output's own rounding as in test_parity.py; 1e-3
for the fp32 backward).  The cases are drawn once from a
fixed seed: batch, heads, length (ragged against every chunk size), head
dims, input and output dtypes, with or without an initial state, and with
or without the fused q, k normalisation."""
import numpy as np
import pytest
import torch

import oracle
from gdr_gen import make_gdn, make_gdn2

pytestmark = pytest.mark.gpu

DIMS = [(64, 64), (64, 128), (128, 64), (128, 128)]


def _cases(n, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    out = []
    for i in range(n):
        out.append(dict(
            B=int(g.integers(1, 4)), H=int(g.integers(1, 4)), T=int(g.integers(1, 200)),
            dims=DIMS[int(g.integers(0, 4))], dt=["bf16", "f32"][int(g.integers(0, 2))],
            odt=["f32", "bf16"][int(g.integers(0, 2))], s0=bool(g.integers(0, 2)),
            norm=bool(g.integers(0, 2)), shift=float(g.uniform(-4.0, 3.0)), seed=2000 + i))
    return out


def _tol_s(c):
    """The input dtype's tolerance (the state is always fp32)."""
    return 2e-2 if c["dt"] == "bf16" else 1e-3


def _tol_o(c, o_ref):
    """The input dtype's tolerance; a bf16 output also gets its own
    rounding, measured on the oracle's output (half a bf16 ulp per element
    on this metric), as in test_parity.py."""
    t = _tol_s(c)
    if c["odt"] == "bf16":
        ob = torch.from_numpy(np.asarray(o_ref, dtype=np.float32)).to(torch.bfloat16)
        t += oracle.err_rms(ob.double().numpy(), o_ref)
    return t


def _g(x):
    return None if x is None else x.cuda()


def _norm(x, on):
    return torch.from_numpy(oracle.l2norm(x)) if on else x


TDT = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.mark.parametrize("c", _cases(16, 11), ids=lambda c: f"s{c['seed']}")
def test_sweep_gdn(gdr_lib, c):
    Dk, Dv = c["dims"]
    inp = make_gdn(B=c["B"], T=c["T"], H=c["H"], Dk=Dk, Dv=Dv, dtype=c["dt"], seed=c["seed"],
                   alpha_shift=c["shift"], s0_std=0.1 if c["s0"] else None, raw_qk=c["norm"])
    print(f"gdn {c}", flush=True)
    o_ref, s_ref = oracle.gdn_fwd(_norm(inp.q, c["norm"]), _norm(inp.k, c["norm"]), inp.v,
                                  inp.alpha, inp.beta, inp.s0)
    o, s = gdr_lib.gdr_chunk_fwd(_g(inp.q), _g(inp.k), _g(inp.v), _g(inp.alpha), _g(inp.beta),
                                 _g(inp.s0), out_dtype=TDT[c["odt"]], l2norm_qk=c["norm"])
    torch.cuda.synchronize()
    eo, es = oracle.err_rms(o.cpu(), o_ref), oracle.err_rms(s.cpu(), s_ref)
    print(f"  err(o)={eo:.2e} err(S)={es:.2e}")
    assert eo <= _tol_o(c, o_ref) and es <= _tol_s(c), (eo, es)


@pytest.mark.parametrize("c", _cases(16, 12), ids=lambda c: f"s{c['seed']}")
def test_sweep_gdn2(gdr_lib, c):
    Dk, Dv = c["dims"]
    inp = make_gdn2(B=c["B"], T=c["T"], H=c["H"], Dk=Dk, Dv=Dv, dtype=c["dt"], seed=c["seed"],
                    alpha_shift=c["shift"], s0_std=0.1 if c["s0"] else None, raw_qk=c["norm"])
    print(f"gdn2 {c}", flush=True)
    o_ref, s_ref = oracle.gdn2_fwd(_norm(inp.q, c["norm"]), _norm(inp.k, c["norm"]), inp.v,
                                   inp.alpha, inp.erase, inp.write, inp.s0)
    o, s = gdr_lib.gdr2_chunk_fwd(_g(inp.q), _g(inp.k), _g(inp.v), _g(inp.alpha), _g(inp.erase),
                                  _g(inp.write), _g(inp.s0), out_dtype=TDT[c["odt"]],
                                  l2norm_qk=c["norm"])
    torch.cuda.synchronize()
    eo, es = oracle.err_rms(o.cpu(), o_ref), oracle.err_rms(s.cpu(), s_ref)
    print(f"  err(o)={eo:.2e} err(S)={es:.2e}")
    assert eo <= _tol_o(c, o_ref) and es <= _tol_s(c), (eo, es)


@pytest.mark.parametrize("c", _cases(8, 13), ids=lambda c: f"s{c['seed']}")
def test_sweep_bwd(gdr_lib, c):
    """Both backward calls on the same draw (fp32 inputs and gradients)."""
    Dk, Dv = c["dims"]
    g = np.random.Generator(np.random.PCG64(c["seed"]))
    B, T, H = c["B"], c["T"], c["H"]
    do = torch.from_numpy(g.standard_normal((B, T, H, Dv)).astype(np.float32))
    dsf = torch.from_numpy((0.1 * g.standard_normal((B, H, Dv, Dk))).astype(np.float32))
    s0 = 0.1 if c["s0"] else None
    inp = make_gdn(B=B, T=T, H=H, Dk=Dk, Dv=Dv, dtype="f32", seed=c["seed"],
                   alpha_shift=c["shift"], s0_std=s0, raw_qk=c["norm"])
    print(f"bwd {c}", flush=True)
    ref = list(oracle.gdn_bwd(_norm(inp.q, c["norm"]), _norm(inp.k, c["norm"]), inp.v,
                              inp.alpha, inp.beta, inp.s0, do, dsf))
    if c["norm"]:
        ref[0], ref[1] = oracle.l2norm_bwd(inp.q, ref[0]), oracle.l2norm_bwd(inp.k, ref[1])
    got = gdr_lib.gdr_chunk_bwd(_g(inp.q), _g(inp.k), _g(inp.v), _g(inp.alpha), _g(inp.beta),
                                _g(inp.s0), _g(do), _g(dsf), l2norm_qk=c["norm"])
    torch.cuda.synchronize()
    errs = [oracle.err_rms(x.cpu(), y) for x, y in zip(got, ref)]
    print("  " + " ".join(f"{e:.2e}" for e in errs))
    assert max(errs) <= 1e-3, errs
    inp2 = make_gdn2(B=B, T=T, H=H, Dk=Dk, Dv=Dv, dtype="f32", seed=c["seed"],
                     alpha_shift=c["shift"], s0_std=s0, raw_qk=c["norm"])
    ref2 = list(oracle.gdn2_bwd(_norm(inp2.q, c["norm"]), _norm(inp2.k, c["norm"]), inp2.v,
                                inp2.alpha, inp2.erase, inp2.write, inp2.s0, do, dsf))
    if c["norm"]:
        ref2[0], ref2[1] = oracle.l2norm_bwd(inp2.q, ref2[0]), oracle.l2norm_bwd(inp2.k, ref2[1])
    got2 = gdr_lib.gdr2_chunk_bwd(_g(inp2.q), _g(inp2.k), _g(inp2.v), _g(inp2.alpha),
                                  _g(inp2.erase), _g(inp2.write), _g(inp2.s0), _g(do), _g(dsf),
                                  l2norm_qk=c["norm"])
    torch.cuda.synchronize()
    errs2 = [oracle.err_rms(x.cpu(), y) for x, y in zip(got2, ref2)]
    print("  " + " ".join(f"{e:.2e}" for e in errs2))
    assert max(errs2) <= 1e-3, errs2
