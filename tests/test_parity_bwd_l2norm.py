"""GPU parity of the backward with q, k normalised on load (GDR_L2NORM_QK,
the _ex backward calls): gradients with respect to the raw q and k against
the oracle's backward on the normalised inputs taken through the oracle's
reverse mode of the normalisation; every other gradient is the oracle's
backward on the normalised inputs.  1e-3 of rms, as for the plain backward."""
import numpy as np
import pytest
import torch

import oracle
from gdr_gen import make_gdn, make_gdn2

pytestmark = pytest.mark.gpu

TOL = 1e-3


def _grads_in(shape_v, shape_s, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    do = torch.from_numpy(g.standard_normal(shape_v).astype(np.float32))
    dsf = torch.from_numpy((0.1 * g.standard_normal(shape_s)).astype(np.float32))
    return do, dsf


def _compare(names, got, ref):
    errs = {n: oracle.err_rms(x.cpu(), y) for n, x, y in zip(names, got, ref)}
    print("  " + " ".join(f"{n}={e:.2e}" for n, e in errs.items()))
    bad = {n: e for n, e in errs.items() if not e <= TOL}
    assert not bad, bad


@pytest.mark.parametrize("dims", [(128, 128), (64, 128), (128, 64)])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_bwd_l2norm(gdr_lib, dims, dt):
    Dk, Dv = dims
    inp = make_gdn(B=1, T=90, H=2, Dk=Dk, Dv=Dv, dtype=dt, seed=800 + Dk + Dv, s0_std=0.2,
                   raw_qk=True)
    print(f"bwd l2norm {inp.meta}", flush=True)
    do, dsf = _grads_in(inp.v.shape, (1, 2, Dv, Dk), 1)
    qn, kn = oracle.l2norm(inp.q), oracle.l2norm(inp.k)
    ref = list(oracle.gdn_bwd(qn, kn, inp.v, inp.alpha, inp.beta, inp.s0, do, dsf))
    ref[0] = oracle.l2norm_bwd(inp.q, ref[0])
    ref[1] = oracle.l2norm_bwd(inp.k, ref[1])
    c = lambda x: None if x is None else x.cuda()
    got = gdr_lib.gdr_chunk_bwd(c(inp.q), c(inp.k), c(inp.v), c(inp.alpha), c(inp.beta),
                                c(inp.s0), c(do), c(dsf), l2norm_qk=True)
    torch.cuda.synchronize()
    _compare(("dq", "dk", "dv", "dalpha", "dbeta", "ds0"), got, ref)


@pytest.mark.parametrize("dims", [(128, 128), (64, 64)])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_bwd2_l2norm(gdr_lib, dims, dt):
    Dk, Dv = dims
    inp = make_gdn2(B=1, T=70, H=2, Dk=Dk, Dv=Dv, dtype=dt, seed=810 + Dk + Dv, s0_std=0.2,
                    raw_qk=True)
    print(f"bwd2 l2norm {inp.meta}", flush=True)
    do, dsf = _grads_in(inp.v.shape, (1, 2, Dv, Dk), 2)
    qn, kn = oracle.l2norm(inp.q), oracle.l2norm(inp.k)
    ref = list(oracle.gdn2_bwd(qn, kn, inp.v, inp.alpha, inp.erase, inp.write, inp.s0, do, dsf))
    ref[0] = oracle.l2norm_bwd(inp.q, ref[0])
    ref[1] = oracle.l2norm_bwd(inp.k, ref[1])
    c = lambda x: None if x is None else x.cuda()
    got = gdr_lib.gdr2_chunk_bwd(c(inp.q), c(inp.k), c(inp.v), c(inp.alpha), c(inp.erase),
                                 c(inp.write), c(inp.s0), c(do), c(dsf), l2norm_qk=True)
    torch.cuda.synchronize()
    _compare(("dq", "dk", "dv", "dalpha", "derase", "dwrite", "ds0"), got, ref)
