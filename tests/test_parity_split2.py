"""GPU parity of the Gated Delta Rule-2 sequence-split calls
(gdr2_chunk_fwd_split, gdr2_chunk_bwd_split) against the oracle: the plain
calls' tolerances (forward: 2e-2 for bf16 inputs, 1e-3 for fp32; backward
1e-3)."""
import numpy as np
import pytest
import torch

import oracle
from gdr_gen import make_gdn2

pytestmark = pytest.mark.gpu


def _g(x):
    return None if x is None else x.cuda()


def _args(inp):
    return (inp.q, inp.k, inp.v, inp.alpha, inp.erase, inp.write, inp.s0)


@pytest.mark.parametrize("nseg,dt,dims", [(2, "bf16", (128, 128)), (4, "bf16", (128, 128)),
                                          (5, "f32", (128, 128)), (4, "bf16", (64, 128)),
                                          (5, "f32", (128, 64)), (2, "f32", (64, 128))])
def test_gdr2_fwd_split(gdr_lib, nseg, dt, dims):
    """Dk != Dv sends the P pass's output to the workspace's bf16 buffer."""
    inp = make_gdn2(B=1, T=160, H=2, Dk=dims[0], Dv=dims[1], dtype=dt,
                    seed=820 + nseg + (0 if dims == (128, 128) else 40 + dims[0] // 16 + dims[1]),
                    alpha_shift=-3.0,
                    s0_std=0.1)
    print(f"gdr2 split fwd nseg={nseg} {inp.meta}", flush=True)
    o_ref, s_ref = oracle.gdn2_fwd(*_args(inp))
    o, s = gdr_lib.gdr2_chunk_fwd_split(*[_g(x) for x in _args(inp)], nseg=nseg,
                                        out_dtype=torch.float32)
    torch.cuda.synchronize()
    tol = 2e-2 if dt == "bf16" else 1e-3
    eo, es = oracle.err_rms(o.cpu(), o_ref), oracle.err_rms(s.cpu(), s_ref)
    print(f"  err(o)={eo:.2e} err(S)={es:.2e}")
    assert eo <= tol and es <= tol, (eo, es)


@pytest.mark.parametrize("nseg,dims", [(2, (128, 128)), (4, (64, 128)), (3, (128, 64))])
def test_gdr2_bwd_split(gdr_lib, nseg, dims):
    Dk, Dv = dims
    inp = make_gdn2(B=1, T=96, H=2, Dk=Dk, Dv=Dv, dtype="f32", seed=830 + nseg,
                    alpha_shift=-3.0, s0_std=0.1)
    print(f"gdr2 split bwd nseg={nseg} {inp.meta}", flush=True)
    g = np.random.Generator(np.random.PCG64(nseg))
    do = torch.from_numpy(g.standard_normal((1, 96, 2, Dv)).astype(np.float32))
    dsf = torch.from_numpy((0.1 * g.standard_normal((1, 2, Dv, Dk))).astype(np.float32))
    ref = oracle.gdn2_bwd(*_args(inp), do, dsf)
    got = gdr_lib.gdr2_chunk_bwd_split(*[_g(x) for x in _args(inp)], _g(do), _g(dsf), nseg=nseg)
    torch.cuda.synchronize()
    names = ("dq", "dk", "dv", "dalpha", "derase", "dwrite", "ds0")
    errs = {n: oracle.err_rms(x.cpu(), y) for n, x, y in zip(names, got, ref)}
    print("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    bad = {n: e for n, e in errs.items() if not e <= 1e-3}
    assert not bad, bad
